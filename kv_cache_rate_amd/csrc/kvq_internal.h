// Internal declarations shared by the libkvq translation units: block
// geometry, device helpers and the host-side launch functions of each
// kernel file.  Not part of the public ABI (include/kvq.h).
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>
#include <stddef.h>
#include <stdint.h>

#include "kvq.h"

namespace kvq {

constexpr int kMaxBlock = KVQ_MAX_BLOCK;          // entries per block
constexpr int kMaxS = KVQ_MAX_S;                  // codebook size limit
constexpr int kMaxCand = 1 + 2 * (kMaxS - 2);     // 29 grid candidates
constexpr int kMaxStats = 80;                     // >= 73 distinct quantile ranks
constexpr int kAlpha = KVQ_MAX_ALPHABET;             // 32
constexpr int kMaxPairs = kAlpha * (kAlpha - 1) / 2; // 496
constexpr int kMaxBeam = KVQ_MAX_BEAM;                // 8
constexpr int kMaxLam = 64;                       // multipliers per solve pass
constexpr int kAlphaLam = 8;                       // multipliers per alphabet-search pass
constexpr int64_t kManyBlocks = 65536;             // grid searches at least this large probe
                                                   // fewer multipliers per pass
// Same-address atomics from every workgroup serialise (about 11 ns each
// here: 2048 of them cost a 12-point alphabet-search pass 22 us of its 44),
// so the solve's rate sums are spread over this many addresses each.
constexpr int kRateStripes = 16;

// Device status bits (workspace header).
constexpr uint32_t kStatusNonFinite = 1u;
constexpr uint32_t kStatusAnsOverflow = 2u;  // an entropy-coded block outgrew its region
constexpr uint32_t kStatusAnsCorrupt = 4u;   // a decoded block's states did not return to 2^16
constexpr uint32_t kStatusFusedStall = 8u;   // one-launch admission: a predecessor's offset never came

// Fixed header at the start of the caller's workspace.  All solve state lives
// here so the whole bracket search runs on the device without host syncs.
struct WsHeader {
    uint32_t status;     // kStatus* bits set by kernels
    int32_t phase;       // solve phase (see kvq_solve.hip)
    int32_t done;        // 1 once lam_final is known
    int32_t err;         // KVQ_EINFEASIBLE when the doubling overflows
    int32_t nlam;        // multipliers probed by the next rates pass
    int32_t bits_left;   // halvings still to emulate
    int32_t bits_now;    // halvings covered by the current pass
    int32_t bits_max;    // halvings per multisection pass (2^b - 1 multipliers)
    int32_t dbl_n;       // powers of two probed per doubling pass
    int32_t dbl_base;    // exponent of the current doubling pass's first probe
    double lo, hi;       // bracket
    double lam_final;    // multiplier the blocks are chosen at
    uint64_t rate_final; // fixed-point rate of the final choice
    uint64_t Btot_fx;    // budget in the same fixed point
    double lam[kMaxLam + 8];
    unsigned long long sums[kMaxLam + 8];
    uint32_t pool_n;          // greedy post-pass: upgrades collected
    uint32_t pool_overflow;   // 1 if they exceeded the pool
    uint32_t swaps;           // upgrades applied
    uint32_t pad1;
    uint64_t part_rate[16];   // few-block final pass: fixed-point rate per workgroup
    // (the host reads the header up to here)
    // a rates pass adds its blocks' rates into kRateStripes accumulators
    // per multiplier, chosen by workgroup, and the pass's select folds them
    // into sums; the final pass likewise into rate_part, folded into
    // rate_final by fold_rate_kernel
    unsigned long long rsum[kMaxLam][kRateStripes];
    unsigned long long rate_part[kRateStripes];
};
// bytes of the header the host reads back after a solve
constexpr size_t kWsHeaderReadBytes = offsetof(WsHeader, rsum);
static_assert(kWsHeaderReadBytes <= 8192, "solve read-back fits the staging buffer");
constexpr size_t kWsHeaderBytes = 16384;
constexpr uint32_t kGreedyPool = 16384;  // (block, candidate) pairs in the workspace pool
// workspace = header, scan tile sums, greedy pool (8 bytes per pair)
__host__ __device__ inline size_t ws_pool_offset(int64_t R) {
    const int64_t tiles = (R + 1023) / 1024 + 1;
    return (kWsHeaderBytes + (size_t)tiles * sizeof(uint64_t) + 255) & ~(size_t)255;
}
static_assert(sizeof(WsHeader) <= kWsHeaderBytes, "workspace header");
// Static device scratch of kvq_admit_noalloc: header plus scan tile sums
// (no greedy pool), enough for ws_pool_offset(R) with R up to 3,668,992,
// then the one-launch admission's published words (kFusedWordsBytes).
constexpr size_t kNoAllocSolveBytes = 45056;
constexpr size_t kFusedWordsBytes = 2 * 1024 * sizeof(uint64_t);  // 2 x kFusedMaxBlocks words
constexpr size_t kNoAllocScratchBytes = kNoAllocSolveBytes + kFusedWordsBytes;

// Block geometry as the kernels see it (passed by value).
struct Geom {
    const void* data[KVQ_MAX_TENSORS];
    int64_t nb0;                          // blocks of tensor 0
    int64_t stride[KVQ_MAX_TENSORS][4];   // element strides
    int32_t heads, chunks, groups;        // same for every tensor
    int32_t Tb, Db, n;                    // block shape, n = Tb * Db
    int32_t dtype;                        // KVQ_F16 | KVQ_F32
    int32_t contig;                       // 1: every block is n contiguous entries
};

// Tensor index and element offset of entry 0 of block r (block order:
// tensor, outer, head, token chunk, feature group).
__device__ __forceinline__ int64_t block_base(const Geom& g, int64_t r, int& ti) {
    ti = r >= g.nb0 ? 1 : 0;
    int64_t rl = ti ? r - g.nb0 : r;
    const int64_t gr = rl % g.groups;
    rl /= g.groups;
    const int64_t c = rl % g.chunks;
    rl /= g.chunks;
    const int64_t h = rl % g.heads;
    const int64_t o = rl / g.heads;
    return o * g.stride[ti][0] + h * g.stride[ti][1] + c * (int64_t)g.Tb * g.stride[ti][2] +
           gr * (int64_t)g.Db * g.stride[ti][3];
}

// Offset of entry t (row-major token, feature) from the block base.
__device__ __forceinline__ int64_t entry_off(const Geom& g, int ti, int t) {
    if (g.contig) return t;
    const int tok = t / g.Db;
    const int col = t - tok * g.Db;
    return tok * g.stride[ti][2] + col * g.stride[ti][3];
}

__device__ __forceinline__ float load_entry(const Geom& g, int ti, int64_t off) {
    if (g.dtype == KVQ_F16) return __half2float(reinterpret_cast<const __half*>(g.data[ti])[off]);
    return reinterpret_cast<const float*>(g.data[ti])[off];
}

// Order-preserving map of fp32 bit patterns to unsigned keys.
__device__ __forceinline__ uint32_t f32_key(float v) {
    const uint32_t u = __float_as_uint(v);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float key_f32(uint32_t k) {
    const uint32_t u = (k & 0x80000000u) ? (k & 0x7fffffffu) : ~k;
    return __uint_as_float(u);
}

// Rank of point j of the k-point empirical-quantile grid over n sorted
// entries: j (n-1)/(k-1) rounded half up.
__host__ __device__ __forceinline__ int quantile_rank(int j, int k, int n) {
    return (2 * j * (n - 1) + (k - 1)) / (2 * (k - 1));
}

// Point j of the k-point uniform grid on [mn, mx]: fp64 round-to-nearest
// mn + ((mx - mn) * j) / (k - 1) with no contraction, then fp32.
__device__ __forceinline__ float uniform_point(float mn, float mx, int j, int k) {
#pragma clang fp contract(off)
    const double dmn = (double)mn;
    const double span = (double)mx - dmn;
    const double v = dmn + (span * (double)j) / (double)(k - 1);
    return (float)v;
}

// Philox4x32-10 (Salmon, Moraes, Dror, Shaw, SC'11): ten rounds of two
// 32x32->64 multiplies with the published multipliers, Weyl key schedule.
__device__ __forceinline__ void philox4x32_10(uint32_t& c0, uint32_t& c1, uint32_t& c2,
                                              uint32_t& c3, uint32_t k0, uint32_t k1) {
#pragma unroll
    for (int rnd = 0; rnd < 10; ++rnd) {
        const uint64_t p0 = (uint64_t)0xD2511F53u * c0;
        const uint64_t p1 = (uint64_t)0xCD9E8D57u * c2;
        // three-input XOR (truth table 0x96) in one gfx950 v_bitop3_b32
        const uint32_t n0 = __builtin_amdgcn_bitop3_b32((uint32_t)(p1 >> 32), c1, k0, 0x96);
        const uint32_t n2 = __builtin_amdgcn_bitop3_b32((uint32_t)(p0 >> 32), c3, k1, 0x96);
        c0 = n0;
        c1 = (uint32_t)p1;
        c2 = n2;
        c3 = (uint32_t)p0;
        k0 += 0x9E3779B9u;
        k1 += 0xBB67AE85u;
    }
}

__host__ __device__ __forceinline__ int code_width(int m) {
    int w = 0;
    while ((1 << w) < m) ++w;
    return w;
}

// ---- wave64 cross-lane operations through DPP (gfx9 family) ----
// row_shr:k moves lane l - k to lane l inside each 16-lane row (lanes whose
// source falls outside the row keep `old`); row_bcast:15 / row_bcast:31 copy
// lane 15 of a row (lane 31) into the following row(s) selected by row_mask.
constexpr int kDppRowShr1 = 0x111, kDppRowShr2 = 0x112, kDppRowShr4 = 0x114,
              kDppRowShr8 = 0x118, kDppBcast15 = 0x142, kDppBcast31 = 0x143,
              kDppRowMirror = 0x140, kDppRowHalfMirror = 0x141;

template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t old, uint32_t v) {
    return (uint32_t)__builtin_amdgcn_update_dpp((int)old, (int)v, CTRL, ROW_MASK, 0xF, false);
}
template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ double dpp_f64(double old, double v) {
    const uint64_t o = (uint64_t)__double_as_longlong(old), x = (uint64_t)__double_as_longlong(v);
    const uint32_t lo = dpp_u32<CTRL, ROW_MASK>((uint32_t)o, (uint32_t)x);
    const uint32_t hi = dpp_u32<CTRL, ROW_MASK>((uint32_t)(o >> 32), (uint32_t)(x >> 32));
    return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}
template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ uint64_t dpp_u64(uint64_t old, uint64_t v) {
    const uint32_t lo = dpp_u32<CTRL, ROW_MASK>((uint32_t)old, (uint32_t)v);
    const uint32_t hi = dpp_u32<CTRL, ROW_MASK>((uint32_t)(old >> 32), (uint32_t)(v >> 32));
    return ((uint64_t)hi << 32) | lo;
}

// row_shr with bound_ctrl: lanes whose source falls outside the row read 0
// (no `old` operand, so no register has to be cleared first).
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_zero_u32(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, CTRL, 0xF, 0xF, true);
}
template <int CTRL>
__device__ __forceinline__ double dpp_zero_f64(double v) {
    const uint64_t x = (uint64_t)__double_as_longlong(v);
    const uint32_t lo = dpp_zero_u32<CTRL>((uint32_t)x);
    const uint32_t hi = dpp_zero_u32<CTRL>((uint32_t)(x >> 32));
    return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}
template <int CTRL>
__device__ __forceinline__ uint64_t dpp_zero_u64(uint64_t x) {
    const uint32_t lo = dpp_zero_u32<CTRL>((uint32_t)x);
    const uint32_t hi = dpp_zero_u32<CTRL>((uint32_t)(x >> 32));
    return ((uint64_t)hi << 32) | lo;
}

// Inclusive prefix sum over the 64 lanes of a wave.
__device__ __forceinline__ uint32_t wave_scan_add_u32(uint32_t v) {
    v += dpp_u32<kDppRowShr1>(0u, v);
    v += dpp_u32<kDppRowShr2>(0u, v);
    v += dpp_u32<kDppRowShr4>(0u, v);
    v += dpp_u32<kDppRowShr8>(0u, v);
    v += dpp_u32<kDppBcast15, 0xA>(0u, v);
    v += dpp_u32<kDppBcast31, 0xC>(0u, v);
    return v;
}
__device__ __forceinline__ double wave_scan_add_f64(double v) {
    v += dpp_zero_f64<kDppRowShr1>(v);
    v += dpp_zero_f64<kDppRowShr2>(v);
    v += dpp_zero_f64<kDppRowShr4>(v);
    v += dpp_zero_f64<kDppRowShr8>(v);
    v += dpp_f64<kDppBcast15, 0xA>(0.0, v);
    v += dpp_f64<kDppBcast31, 0xC>(0.0, v);
    return v;
}
__device__ __forceinline__ uint64_t wave_scan_add_u64(uint64_t v) {
    v += dpp_zero_u64<kDppRowShr1>(v);
    v += dpp_zero_u64<kDppRowShr2>(v);
    v += dpp_zero_u64<kDppRowShr4>(v);
    v += dpp_zero_u64<kDppRowShr8>(v);
    v += dpp_u64<kDppBcast15, 0xA>(0ull, v);
    v += dpp_u64<kDppBcast31, 0xC>(0ull, v);
    return v;
}
// Value of lane 63 (the wave total after an inclusive scan), wave-uniform.
__device__ __forceinline__ uint32_t wave_last_u32(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}
__device__ __forceinline__ double wave_last_f64(double v) {
    const uint64_t x = (uint64_t)__double_as_longlong(v);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)x, 63);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(x >> 32), 63);
    return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}
// Wave-wide min / max (every lane gets the result).
__device__ __forceinline__ uint32_t wave_min_u32_dpp(uint32_t v) {
    v = min(v, dpp_u32<kDppRowShr1>(0xffffffffu, v));
    v = min(v, dpp_u32<kDppRowShr2>(0xffffffffu, v));
    v = min(v, dpp_u32<kDppRowShr4>(0xffffffffu, v));
    v = min(v, dpp_u32<kDppRowShr8>(0xffffffffu, v));
    v = min(v, dpp_u32<kDppBcast15, 0xA>(0xffffffffu, v));
    v = min(v, dpp_u32<kDppBcast31, 0xC>(0xffffffffu, v));
    return wave_last_u32(v);
}
__device__ __forceinline__ uint32_t wave_max_u32_dpp(uint32_t v) {
    v = max(v, dpp_u32<kDppRowShr1>(0u, v));
    v = max(v, dpp_u32<kDppRowShr2>(0u, v));
    v = max(v, dpp_u32<kDppRowShr4>(0u, v));
    v = max(v, dpp_u32<kDppRowShr8>(0u, v));
    v = max(v, dpp_u32<kDppBcast15, 0xA>(0u, v));
    v = max(v, dpp_u32<kDppBcast31, 0xC>(0u, v));
    return wave_last_u32(v);
}
// Sum over each 16-lane row; the row total lands in the row's lane 15.
__device__ __forceinline__ double row_sum_f64(double v) {
    v += dpp_zero_f64<kDppRowShr1>(v);
    v += dpp_zero_f64<kDppRowShr2>(v);
    v += dpp_zero_f64<kDppRowShr4>(v);
    v += dpp_zero_f64<kDppRowShr8>(v);
    return v;
}
// Wave-wide sum, wave-uniform result: row sums, then the four row totals
// added in row order.
__device__ __forceinline__ double wave_sum_f64(double v) {
    v = row_sum_f64(v);
    const uint64_t x = (uint64_t)__double_as_longlong(v);
    double t[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)x, 16 * k + 15);
        const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(x >> 32), 16 * k + 15);
        t[k] = __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
    }
    return (t[0] + t[1]) + (t[2] + t[3]);
}

// Workgroups are dispatched round-robin over the 8 XCDs (each with its own
// L2).  Mapping workgroup b to block r so that XCD x owns the contiguous
// range of blocks [start_x, start_x + count_x) lets neighbouring blocks'
// writes into block-interleaved tables combine in one L2.  Bijective on
// [0, R).
constexpr int kXcds = 8;
__device__ __forceinline__ int64_t xcd_block(int64_t b, int64_t R) {
    const int64_t x = b % kXcds, idx = b / kXcds;
    const int64_t q = R / kXcds, rem = R % kXcds;
    return x * q + (x < rem ? x : rem) + idx;
}

// Pairs (i < j) of an M-point alphabet, and the index of one in row-major
// upper-triangle order.
__host__ __device__ __forceinline__ int n_pairs(int M) { return M * (M - 1) / 2; }
__host__ __device__ __forceinline__ int pair_index(int i, int j, int M) {
    return i * (2 * M - i - 1) / 2 + (j - i - 1);
}

// Quantile-rank lookup: stats column of rank quantile_rank(j, k, n).
struct RankTable {
    uint8_t col[kMaxS + 1][kMaxS];
    int32_t rank[kMaxStats];
    int32_t n_stats;
};

// ---- host-side launchers (defined in the kernel files) ----
hipError_t launch_eval_grids(const Geom& g, int64_t R, int s, const RankTable& rt, double* D,
                             double* H, float* stats, void* ws, hipStream_t st);
hipError_t launch_eval16(const void* x0, const void* x1, int64_t nb0, int64_t R, const RankTable& rt,
                         double* D, double* H, float* stats, void* ws, hipStream_t st);
hipError_t launch_eval_alphabet(const Geom& g, int64_t R, int alpha_m, double* D, double* H,
                                float* stats, void* ws, hipStream_t st);
hipError_t launch_ws_reset(void* ws, hipStream_t st);
// One launch of the admission step at a known multiplier for up to
// kFusedMaxBlocks fp16 blocks of 4096 contiguous entries with s = 16 (grid
// search): scoring, the choice at lam_in, the codebook, the offsets, the
// stochastic rounding and packing, the rate sum; the last block writes the
// workspace header whole.  `out` (pinned host memory, may be null) receives
// the solve's result fields.  `words` (kFusedWordsBytes of device memory that
// only these launches write) holds the blocks' published word counts and
// rates, tagged with `epoch` (1 .. kFusedEpochMax): every launch on one words
// buffer takes a new epoch, and the buffer is cleared
// (launch_fused_words_clear) before its first launch and whenever the epochs
// start over, so a word is never read as a later launch's.
constexpr int64_t kFusedMaxBlocks = 1024;
static_assert(kFusedWordsBytes == 2 * kFusedMaxBlocks * sizeof(uint64_t), "fused words");
constexpr uint32_t kFusedEpochMax = (1u << 28) - 1u;
hipError_t launch_admit_fused(const void* x0, const void* x1, int64_t nb0, int64_t R, const RankTable& rt,
                              double lam_in, int shift, uint64_t seed, double* D, double* H, float* stats,
                              int32_t* choice, float* codebook, uint8_t* m, uint64_t* off, uint32_t* codes,
                              void* ws, uint64_t* words, uint32_t epoch, struct SolveOut* out, hipStream_t st);
hipError_t launch_fused_words_clear(uint64_t* words, hipStream_t st);
// Read `bytes` (<= kStagingBytes) of device memory into host memory `dst`
// on stream st and wait for it, through the calling thread's pinned staging
// buffer (hipHostMalloc'd on first use and kept until the process ends; a
// plain pageable copy if the allocation fails).  With staging = false the
// copy goes straight to `dst` and nothing is allocated.
constexpr size_t kStagingBytes = 8192;
hipError_t read_back(void* dst, const void* src, size_t bytes, hipStream_t st, bool staging = true);
// The calling thread's pinned staging buffer (kStagingBytes, allocated on
// first use), or null if it cannot be allocated; *dev (if dev is not null)
// receives its device-side address, or null.
void* staging_buffer(void** dev);
// The header fields the host reads after a solve.  The one-workgroup final
// pass writes them straight into pinned host memory, which saves the copy.
struct SolveOut {
    uint32_t status;
    int32_t err;
    uint32_t pool_overflow;
    uint32_t pad;
    double lam_final;
    uint64_t rate_final;
};
// `out` (pinned host memory, may be null): if the solve's last kernel wrote
// the result there, *direct is set and the caller only has to synchronise.
// staging: whether the mid-solve read-back may use the pinned staging buffer
// (false: a plain copy, no allocation).
hipError_t launch_solve(const kvq_plan& p, const RankTable& rt, const double* D,
                        const double* H, const double* wgt, const float* stats, double B,
                        int mode, int iters,
                        double lam_in, int32_t* choice, float* codebook, uint8_t* m,
                        uint64_t* off, void* ws, SolveOut* out, bool* direct, hipStream_t st,
                        bool staging = true);
hipError_t launch_quantize(const Geom& g, int64_t R, int s, const float* codebook,
                           const uint8_t* m, const uint64_t* off, uint64_t seed,
                           uint32_t* codes, hipStream_t st);
hipError_t launch_dequantize(int64_t R, int n, int s, const uint32_t* codes,
                             const float* codebook, const uint8_t* m, const uint64_t* off,
                             float* xhat, hipStream_t st);
// off[0] = 0 and off[1..R] = sizes -> exclusive prefix sums (tile sums in ws)
hipError_t launch_offsets_scan(uint64_t* off, int64_t R, void* ws, hipStream_t st);
// entropy coding (kvq_ans.hip): per-block scratch margin, encode, decode
__host__ __device__ uint64_t ans_margin_bytes(int n);
hipError_t launch_ans_encode(const uint32_t* codes, const uint8_t* m, const uint64_t* word_off,
                             int64_t R, int n, int s, uint16_t* scratch, uint8_t* stream,
                             uint64_t* block_off, void* ws, hipStream_t st);
// decode attention over the quantized cache (kvq_attn.hip)
uint64_t attn_workspace_bytes(int64_t outer, int heads, int chunks, int group);
hipError_t launch_decode_attention(const uint32_t* codes, const float* codebook, const uint8_t* m,
                                   const uint64_t* word_off, int64_t nbK, int64_t outer, int heads,
                                   int chunks, int s, int group, const float* q, float scale,
                                   float* out, void* work, hipStream_t st);
hipError_t launch_ans_decode(const uint8_t* stream, const uint64_t* block_off, const float* codebook,
                             const uint8_t* m, int64_t R, int n, int s, float* xhat, void* ws,
                             hipStream_t st);

}  // namespace kvq
