// Candidate scoring for fp16 blocks of 4096 contiguous entries (the
// head x 32-token x 128 blocks of KV caches), without sorting.
//
// Page "Rate-adaptive KV-cache quantizer": Implementation notes (candidate
// alphabet from the block's minimum, maximum and quantiles; D_r from interval
// statistics; H_r from expected frequencies) and Key formulas (3).
//
// Every candidate interval [a, b) only needs the count C and sum S1 of the
// entries inside it: the mass sent to b is (S1 - a C)/(b - a), the mass sent
// to a is C minus that, and the block distortion follows from the identity
//     D = sum_t (q_{i+1} - x_t)(x_t - q_i) = sum_j q_j^2 M_j - sum_t x_t^2,
// (M_j the total mass at q_j), because the conditional second moment of the
// interpolated value is x^2 + (q_{i+1} - x)(x - q_i).  So the kernel needs,
// at every codepoint q, the number of entries below q and their sum.
//
// fp16 entries are mapped to order-preserving 16-bit keys.  A key's top 10
// bits pick a coarse bin (1024 bins); inside a bin the 64 values are
// v = B + f U (f = low 6 key bits, U = the bin's ulp), so a bin is summarised
// exactly by (count, sum of f) packed in one 32-bit LDS word, count in the
// top 13 bits.  Sweep 1 fills these; a prefix over bins gives counts and
// exact fp64 sums at bin edges (fp16 sums of 4096 entries are exact in fp64).
// The bins that hold a wanted order statistic or a uniform-grid threshold
// claim a slot; sweep 2 gives each slot per-key 16-bit counts and packed
// (count, sum f) totals of its eight 8-key groups.  One lane per threshold
// then finishes its prefix inside the bin with two branch-free 8-step scans
// (groups, then keys).  Order statistics are therefore exact data values and
// every prefix is exact; only the per-interval algebra rounds (fp64).
//
// Candidate phase: one lane per candidate interval (239 intervals over the 29
// candidates, packed two candidates to a 16-lane row so that a row shift
// brings in the neighbouring interval), then one lane per candidate sums its
// intervals' terms in a fixed order.
//
// Workgroup = one block, 256 threads x 16 entries kept in registers.
#include <math.h>
#include <string.h>

#include "kvq_grid_choice.h"
#include "kvq_internal.h"
#include "kvq_quant_block.h"

namespace kvq {

namespace {

constexpr int kT = 256;            // threads per block
constexpr int kW = kT / 64;        // waves per block
constexpr int kPer = 16;           // entries per thread
constexpr int kCL = 256;           // candidate-interval lanes
constexpr int kNC = 1024;          // coarse bins
constexpr int kSlotsLarge = 112;   // claimed bins held at once in large launches (see the rounds below)
constexpr int kFW = 32;            // per-key count words of a slot (64 x 16 bit)
constexpr int kSW = 40;            // words per slot: 32 per-key + 8 group totals
constexpr int kNU = 71;            // distinct interior uniform fractions, s = 16
constexpr int kNQ = 73;            // order statistics, s = 16, n = 4096
constexpr int kPU = 2;             // point table: 0 = min, 1 = max,
constexpr int kPQ = kPU + kNU;     //   then uniform thresholds, then order statistics
constexpr int kNP = kPQ + kNQ;     // 146 points
constexpr int kSlotsAll = kNQ + kNU;   // 144: every claimable bin (small launches)
constexpr int64_t kEvalSmallLaunch = 16384;  // blocks below which kSlotsAll is used
constexpr int kRows = 15;          // 16-lane rows of candidate intervals
constexpr uint32_t kNoSlot = 0xffffffffu, kClaim = 0xfffffffeu;
constexpr uint32_t kSlotOff = 0x3fffffffu;    // slot map: byte offset ...
constexpr uint32_t kRound2 = 0x40000000u;     // ... | this bit for the second round
constexpr uint32_t kCnt1 = 1u << 19;       // one entry in a packed (count, sum f) word
constexpr uint32_t kLowF = kCnt1 - 1u;     // sum-of-f field
constexpr uint32_t kNoLane = 0xffffu;      // lane without an interval
constexpr int kDppRowShl1 = 0x101;         // row_shl:1, lane l reads lane l + 1

struct Point {                     // a codepoint and the entries below it
    float v;
    uint32_t cnt;
    double s1;
};

struct PhaseA {                    // sweep 1 .. threshold search
    uint32_t cnt[kNC + 4];         // payload, then exclusive prefix counts
    double ps1[kNC + 1];           // exclusive prefix sums
};
template <int kSlots>
struct PhaseB {                    // sweep 2 .. prefix finish
    uint32_t w[kSlots * kSW];
};
struct PhaseC {                    // candidate intervals, written only by a wave
    double mr[kCL];                //   that holds a zero-width interval:
    double ma[kCL];                // mass at the interval's right point, mass it
    float bv[kCL];                 // sends to its left point, right point
    double cd[kMaxCand];           // one-launch admission: the block's D and H
    double chh[kMaxCand];
};

template <int kSlots>
struct Shared {
    union alignas(16) {
        PhaseA a;
        PhaseB<kSlots> b;
        PhaseC c;
        QuantLds q;                // one-launch admission: the block's quantization
    } u;
    alignas(16) float book[kMaxS]; // one-launch admission: the chosen codebook
    int32_t fz_m;
    uint64_t fz_ob;                // this block's word count
    uint64_t fz_rate;              // this block's fixed-point rate
    uint32_t fz_nf;                // this block holds NaN or Inf
    uint64_t fz_part[kW];          // per wave: words of the preceding blocks
    uint64_t fz_rpart[kW];         // per wave: their rates (last block only)
    uint32_t fz_flags[kW];         // per wave: their status bits (last block only)
    alignas(16) uint32_t slot[kNC];  // bin -> byte offset of its slot, or kNoSlot
    alignas(16) Point P[kNP];
    uint16_t tbin[kNQ];
    uint16_t tloc[kNQ];
    uint16_t ukey[kNU];
    double lg_c[64];
    double lg_inv[64];
    uint32_t rcol[(kMaxS + 1) * kMaxS / 4];  // one-launch admission: the rank table's columns
    uint32_t wmin[kW], wmax[kW], wtot[kW];
    double wsq[kW], wts1[kW];
    uint32_t nslots;
};

typedef unsigned short ushort2_t __attribute__((ext_vector_type(2)));
typedef short short2_t __attribute__((ext_vector_type(2)));
typedef _Float16 half2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t half_key(uint32_t h) {
    return (h & 0x8000u) ? (~h & 0xffffu) : (h | 0x8000u);
}
__device__ __forceinline__ float key_value(uint32_t key) {
    const uint32_t h = (key & 0x8000u) ? (key & 0x7fffu) : (~key & 0xffffu);
    return __half2float(__ushort_as_half((unsigned short)h));
}
// Smallest fp16 key whose value is >= t (t finite, within the fp16 range).
__device__ __forceinline__ uint32_t key_ceil(float t) {
    const __half h = __float2half_rn(t);
    uint32_t bits = __half_as_ushort(h);
    if (bits == 0x8000u) bits = 0;
    uint32_t key = half_key(bits);
    if (key_value(key) < t) key += 1;
    return key;
}

// Order-preserving 16-bit keys of the two fp16 values of a 32-bit word;
// x + (+0) maps -0 to +0 and leaves every other value (NaN stays NaN).
__device__ __forceinline__ uint32_t pair_keys(uint32_t hw, half2_t& hv) {
    hv = __builtin_bit_cast(half2_t, hw) + (half2_t){(_Float16)0.0f, (_Float16)0.0f};
    const uint32_t w = __builtin_bit_cast(uint32_t, hv);
    const short2_t sg = __builtin_bit_cast(short2_t, w) >> (short2_t){15, 15};
    const uint32_t msk = (__builtin_bit_cast(uint32_t, sg) & 0x7fff7fffu) | 0x80008000u;
    return w ^ msk;
}
__device__ __forceinline__ uint32_t pair_keys(uint32_t hw) {
    half2_t hv;
    return pair_keys(hw, hv);
}

// A round's slot tag as a compile-time value.
template <uint32_t V>
struct RoundTag {
    static constexpr uint32_t value = V;
};

// Fixed instruction forms for sweep 2's per-entry address arithmetic (the
// compiler rewrites the builtins into longer shift/mask sequences).
// (x >> off) & ((1 << w) - 1), off and w immediate:
template <uint32_t kOff, uint32_t kWid>
__device__ __forceinline__ uint32_t bfe_u32(uint32_t x) {
    uint32_t r;
    asm("v_bfe_u32 %0, %1, %2, %3" : "=v"(r) : "v"(x), "i"(kOff), "i"(kWid));
    return r;
}
// a * b + c on the low 24 bits of a and b:
__device__ __forceinline__ uint32_t mad_u24(uint32_t a, uint32_t b, uint32_t c) {
    uint32_t r;
    asm("v_mad_u32_u24 %0, %1, %2, %3" : "=v"(r) : "v"(a), "s"(b), "i"(c));
    return r;
}

// a.lo * b.lo + a.hi * b.hi + c on the 16-bit halves of a and b (exact:
// the sums here stay below 2^32).
__device__ __forceinline__ uint32_t udot2(uint32_t a, uint32_t b, uint32_t c) {
    return __builtin_amdgcn_udot2(__builtin_bit_cast(ushort2_t, a), __builtin_bit_cast(ushort2_t, b), c, false);
}

// 1/x to ~1 ulp: hardware reciprocal estimate and two Newton steps.
__device__ __forceinline__ double recip(double x) {
    double r = __builtin_amdgcn_rcp(x);
    double e = fma(-x, r, 1.0);
    r = fma(r, e, r);
    e = fma(-x, r, 1.0);
    return fma(r, e, r);
}

// a * b + c in fp64 with c a compile-time constant kept in a scalar register
// (v_fma_f64 takes one scalar operand; otherwise the constant would be
// copied into vector registers for every use).
__device__ __forceinline__ double fma_sc(double a, double b, double c) {
    double r;
    asm("v_fma_f64 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "s"(c));
    return r;
}

// log2 of x in (0, 1], relative error ~1e-16: x = m 2^e with m in [1, 2);
// c = 1 + (2i + 1)/128 is the centre of the 1/64-wide cell i of m, so
// log2 m = log2 c + log1p(t)/ln 2 with t = (m - c)/c, |t| < 2^-7, and the
// log1p series to t^7 (truncation below 2^-56/8).
__device__ __forceinline__ double log2_unit(double x, const double* lg_c, const double* lg_inv) {
    const double m = 2.0 * __builtin_amdgcn_frexp_mant(x);  // [1, 2)
    const int e = __builtin_amdgcn_frexp_exp(x) - 1;
    const uint32_t mhi = (uint32_t)((uint64_t)__double_as_longlong(m) >> 32);
    const int i = (int)((mhi >> 14) & 63u);
    // c: m's exponent and top 6 mantissa bits, then the half-cell bit
    const double c = __longlong_as_double((long long)((uint64_t)((mhi & 0xffffc000u) | 0x2000u) << 32));
    const double t = (m - c) * lg_inv[i];
    double p = 1.0 / 7.0;
    p = fma_sc(p, t, -1.0 / 6.0);
    p = fma_sc(p, t, 1.0 / 5.0);
    p = fma_sc(p, t, -1.0 / 4.0);
    p = fma_sc(p, t, 1.0 / 3.0);
    p = fma(p, t, -0.5);
    p = fma(p, t, 1.0);
    const double l1p = p * t;
    return ((double)e + lg_c[i]) + l1p * 1.4426950408889634;  // 1/ln 2
}

// -pi log2 pi of a point holding mass m of the 4096 entries.
__device__ __forceinline__ double point_entropy(double m, const double* lg_c, const double* lg_inv) {
    const double pi = __builtin_amdgcn_ldexp(m, -12);
    return pi > 0.0 ? -pi * log2_unit(pi, lg_c, lg_inv) : 0.0;
}

// One step of segmented inclusive scans within 16-lane rows: add the values
// of the lane K back when it belongs to the same run (off >= K).
template <int CTRL, int K>
__device__ __forceinline__ void seg_scan_step(uint32_t off, double& a, double& b) {
    const double ta = dpp_zero_f64<CTRL>(a);  // lanes without a source read 0
    const double tb = dpp_zero_f64<CTRL>(b);
    if (off >= (uint32_t)K) {
        a += ta;
        b += tb;
    }
}
template <int CTRL, int K>
__device__ __forceinline__ void seg_scan_step(uint32_t off, uint32_t& z) {
    const uint32_t tz = dpp_zero_u32<CTRL>(z);
    if (off >= (uint32_t)K) z += tz;
}

// Claim a slot for coarse bin `bin` (first caller wins; the slot's entry is
// visible after the next barrier).  Claims past kSlots are served by a
// second round that reuses the slot memory: entry = byte offset | kRound2.
template <int kSlots>
__device__ __forceinline__ void claim_slot(Shared<kSlots>& sh, uint32_t bin) {
    if (atomicCAS(&sh.slot[bin], kNoSlot, kClaim) == kNoSlot) {
        const uint32_t k = atomicAdd(&sh.nslots, 1u);
        sh.slot[bin] = k < (uint32_t)kSlots ? k * (uint32_t)(4 * kSW)
                                            : (k - kSlots) * (uint32_t)(4 * kSW) | kRound2;
    }
}

// 16-byte quad q of the slot at byte offset sb (q 0..7: per-key counts of
// group q; 8, 9: the group totals).
template <int kSlots>
__device__ __forceinline__ uint4 slot_quad(const Shared<kSlots>& sh, uint32_t sb, uint32_t q) {
    const char* p = reinterpret_cast<const char*>(sh.u.b.w) + sb + 16u * q;
    return *reinterpret_cast<const uint4*>(__builtin_assume_aligned(p, 16));
}

// 16-bit count of key i (0..7) of a group held in four words.
__device__ __forceinline__ uint32_t key_count(const uint4& w, int i) {
    const uint32_t x = (i >> 1) == 0 ? w.x : (i >> 1) == 1 ? w.y : (i >> 1) == 2 ? w.z : w.w;
    return (i & 1) ? (x >> 16) : (x & 0xffffu);
}
__device__ __forceinline__ uint32_t word_of(const uint4& a, const uint4& b, int i) {
    switch (i) {
        case 0: return a.x;
        case 1: return a.y;
        case 2: return a.z;
        case 3: return a.w;
        case 4: return b.x;
        case 5: return b.y;
        case 6: return b.z;
        default: return b.w;
    }
}

}  // namespace

// Tables from the host.
struct Eval16Tables {
    RankTable rt;
    uint8_t unum[kNU];              // numerator of distinct fraction u
    uint8_t uden[kNU];              // denominator
    uint16_t red[kMaxCand];         // candidate c: first lane | interval count << 8
    uint16_t desc[kCL];             // lane: left point | right point << 8, or kNoLane
    uint16_t lseg[kCL];             // lane: candidate | offset in its run << 5 | last << 9,
                                    //   or kNoLane
                                    //   (a candidate's last interval ends at point 1)
    double lg_c[64];                // log2(1 + (2i+1)/128)
    double lg_inv[64];              // 1 / (1 + (2i+1)/128)
};

// Words a block publishes for the blocks after it (relaxed device-scope
// atomics: each word carries its own flag and the launch's epoch, so no fence
// orders one against another and nothing clears them between launches).
//   count word: kPub | kPubNF | epoch << 34 | rate bits 35..56 << 12 | words
//   rate word:  kPub | epoch << 35 | rate bits 0..34
// A block's fixed-point rate is below 2^55 (4096 entries x 4 bits x 2^40).
constexpr uint64_t kPub = 1ull << 63;      // the word is published
constexpr uint64_t kPubNF = 1ull << 62;    // count word: the block holds NaN or Inf
constexpr uint32_t kEpochMask = kFusedEpochMax;
constexpr uint64_t kRateLoMask = (1ull << 35) - 1ull;
__device__ __forceinline__ uint32_t count_epoch(uint64_t v) { return (uint32_t)(v >> 34) & kEpochMask; }
__device__ __forceinline__ uint32_t rate_epoch(uint64_t v) { return (uint32_t)(v >> 35) & kEpochMask; }
constexpr uint32_t kDescSpins = 1u << 22;  // polls before a missing predecessor is reported

// The rest of the admission step at a known multiplier, run by the same
// workgroup after scoring its block (one-launch admission).
struct FusedArgs {
    double lam;                    // multiplier the blocks are chosen at
    int shift;                     // fixed-point scale of the rate sums
    uint32_t k0, k1;               // Philox key (seed lo, seed hi)
    int32_t* choice;
    float* codebook;               // [R][16]
    uint8_t* m;
    uint64_t* off;                 // [R + 1]
    uint32_t epoch;                // this launch's tag (1 .. kEpochMask), new for every launch
    uint64_t* desc;                // [R] published count words (see kPub)
    uint64_t* rates;               // [R] published rate words
    uint32_t* codes;
    SolveOut* out;                 // pinned host memory, or null
};

// After scoring: choose the block's candidate at fa.lam (lowest index among
// equal objectives, as the solve does), write its codebook, level count and
// choice, add its fixed-point rate, publish its word count and sum those of
// the preceding blocks for its word offset, then quantize and pack it (page
// "Rate-adaptive KV-cache quantizer", Key formulas (2)-(4); Implementation
// notes).  The last block's workgroup also writes the rate and the status
// for the host.
template <int kSlots>
__device__ __forceinline__ void fused_tail(Shared<kSlots>& sh, const Eval16Tables& tb, const FusedArgs& fa,
                                           WsHeader* ws, int64_t r, int64_t R, const uint32_t (&hw)[kPer / 2]) {
    const int tid = threadIdx.x;
    __syncthreads();  // every candidate's D and H are in LDS
    if (tid < 64) {
        // the choice: lane c scores candidate c, and the lowest index among
        // equal minimal objectives wins (as in the solve's final pass).  The
        // objectives are >= 0 (+ 0.0 turns a -0 into +0), so their bit
        // patterns order as their values.
        const PhaseC& pc = sh.u.c;
        const double lamd = fa.lam * 4096.0;
        const double o = tid < kMaxCand ? objective(pc.cd[tid], pc.chh[tid], lamd) + 0.0 : __builtin_huge_val();
        const uint64_t key = (uint64_t)__double_as_longlong(o);
        const uint32_t khi = (uint32_t)(key >> 32), klo = (uint32_t)key;
        const uint32_t mhi = wave_min_u32_dpp(khi);
        const uint32_t mlo = wave_min_u32_dpp(khi == mhi ? klo : 0xffffffffu);
        const int bc = __builtin_amdgcn_readfirstlane(__builtin_ctzll(__ballot(khi == mhi && klo == mlo)));
        // its codebook, the points of write_grid_codebook one per lane:
        // lane j computes point j, keeps it unless it equals point j - 1,
        // and stores it at the count of kept points before it
        const float mn = sh.P[kPQ].v, mx = sh.P[kPQ + kNQ - 1].v;
        const int k = bc == 0 ? 2 : 3 + (bc - 1) / 2;
        const bool uni = bc != 0 && ((bc - 1) & 1) == 0;
        const int j = tid;
        float v = 0.0f;
        if (j < k) {
            if (bc == 0)
                v = j == 0 ? mn : mx;
            else if (uni)
                v = uniform_point(mn, mx, j, k);
            else
                v = sh.P[kPQ + reinterpret_cast<const uint8_t*>(sh.rcol)[k * kMaxS + j]].v;
        }
        const float prev = __shfl_up(v, 1, 64);
        const bool keep = mn == mx ? j == 0 : (j < k && (j == 0 || v != prev));
        const uint64_t kb = __ballot(keep);
        const int m = __popcll(kb);
        if (j < kMaxS) sh.book[j] = 0.0f;
        if (keep) sh.book[__popcll(kb & ((1ull << j) - 1ull))] = mn == mx ? mn : v;
        if (tid == 0) {
            const double bestH = pc.chh[bc];
            fa.choice[r] = bc;
            fa.m[r] = (uint8_t)m;
            const uint64_t words = (4096u * (uint32_t)code_width(m) + 31u) / 32u;
            const uint64_t rate = rate_fx(4096.0, bestH, fa.shift);
            const uint64_t ep = fa.epoch;
            __hip_atomic_store(&fa.desc[r],
                               kPub | (sh.fz_nf ? kPubNF : 0ull) | (ep << 34) | ((rate >> 35) << 12) | words,
                               __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(&fa.rates[r], kPub | (ep << 35) | (rate & kRateLoMask), __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
            if (r == 0) fa.off[0] = 0;
            sh.fz_m = m;
            sh.fz_ob = words;
            sh.fz_rate = rate;
        }
    }
    __syncthreads();
    if (tid < kMaxS) fa.codebook[r * kMaxS + tid] = sh.book[tid];
    const int m = sh.fz_m;
    const float cbv = tid < m ? sh.book[tid] : __builtin_huge_valf();
    __syncthreads();  // the quantizer's tables reuse the phase memory
    // the block's codes (kept in registers until the block's word offset is
    // known), from the data the thread loaded for scoring: its entries are
    // the quantizer's 256-thread chunks tid and 256 + tid
    uint4 all[2][2] = {};
    all[0][0] = make_uint4(hw[0], hw[1], hw[2], hw[3]);
    all[1][0] = make_uint4(hw[4], hw[5], hw[6], hw[7]);
    uint32_t bits[2] = {0u, 0u};
    const int w = quantize_block4096<kT, KVQ_F16, true>(sh.u.q, r, kMaxS, cbv, m, 0, all, nullptr, 0, fa.k0,
                                                        fa.k1, nullptr, bits);
    // word offset: every thread sums the published counts of its share of
    // the blocks before this one (published soon after each is scored;
    // blocks with lower indices were dispatched first); the last block also
    // sums their rates and status bits for the host
    const bool last = r == R - 1;
    uint64_t part = 0, rpart = 0;
    uint32_t flags = 0;
    for (int64_t j = tid; j < r; j += kT) {
        uint32_t spins = 0;
        uint64_t v, q = 0;
        for (;;) {
            v = __hip_atomic_load(&fa.desc[j], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            if (last) q = __hip_atomic_load(&fa.rates[j], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            const bool vok = (v & kPub) && count_epoch(v) == fa.epoch;
            const bool qok = !last || ((q & kPub) && rate_epoch(q) == fa.epoch);
            if (vok && qok) break;
            if (++spins > kDescSpins) {  // never expected: report, do not hang
                flags |= kStatusFusedStall;
                v = 0;
                q = 0;
                break;
            }
            __builtin_amdgcn_s_sleep(1);
        }
        part += v & 0xfffull;
        rpart += (((v >> 12) & 0x3fffffull) << 35) | (q & kRateLoMask);
        if (v & kPubNF) flags |= kStatusNonFinite;
    }
    part = wave_scan_add_u64(part);  // lane 63: the wave's total
    if (last) {
        rpart = wave_scan_add_u64(rpart);
        flags = (__any((flags & kStatusNonFinite) != 0u) ? kStatusNonFinite : 0u) |
                (__any((flags & kStatusFusedStall) != 0u) ? kStatusFusedStall : 0u);
    }
    if ((tid & 63) == 63) {
        sh.fz_part[tid >> 6] = part;
        sh.fz_rpart[tid >> 6] = rpart;
        sh.fz_flags[tid >> 6] = flags;
    }
    __syncthreads();
    const uint64_t ob = (sh.fz_part[0] + sh.fz_part[1]) + (sh.fz_part[2] + sh.fz_part[3]);
    if (w) {
        uint8_t* out = reinterpret_cast<uint8_t*>(fa.codes + ob);
        store_bytes(out + w * tid, bits[0], w);
        store_bytes(out + w * (tid + kT), bits[1], w);
    }
    if (tid == 0) {
        fa.off[r + 1] = ob + sh.fz_ob;
        if (last) {
            const unsigned long long t = (sh.fz_rpart[0] + sh.fz_rpart[1]) + (sh.fz_rpart[2] + sh.fz_rpart[3]) +
                                         sh.fz_rate;
            const uint32_t status = (sh.fz_flags[0] | sh.fz_flags[1] | sh.fz_flags[2] | sh.fz_flags[3]) |
                                    (sh.fz_nf ? kStatusNonFinite : 0u);
            // the header is written whole: nothing clears it before a launch
            ws->status = status;
            ws->phase = 0;
            ws->nlam = 0;
            ws->err = 0;
            ws->done = 1;
            ws->pool_overflow = 0;
            ws->lam_final = fa.lam;
            ws->rate_final = t;
            if (fa.out) {
                SolveOut o;
                o.status = status;
                o.err = 0;
                o.pool_overflow = 0u;
                o.pad = 0u;
                o.lam_final = fa.lam;
                o.rate_final = t;
                *fa.out = o;
                __threadfence_system();
            }
        }
    }
}

// kSlots = kSlotsAll (one round, 5 workgroups per CU) for small launches,
// where a block's latency matters; kSlotsLarge (6 workgroups per CU) for
// large ones, where throughput does.  kFused: the one-launch admission (the
// block is blockIdx.x, so that every block whose word count a workgroup
// waits for was dispatched before it).
template <int kSlots, bool kFused = false>
__global__ void __launch_bounds__(kT, kFused ? 2 : (kSlots == kSlotsAll ? 5 : 6))
eval16_kernel(const __half* __restrict__ x0, const __half* __restrict__ x1, int64_t nb0,
              Eval16Tables tb, double* __restrict__ Dout, double* __restrict__ Hout,
              float* __restrict__ stats, WsHeader* ws, FusedArgs fa) {
    __shared__ Shared<kSlots> sh;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int64_t R = gridDim.x;
    const int64_t r = kFused ? (int64_t)blockIdx.x : xcd_block(blockIdx.x, R);
    const __half* src = r < nb0 ? x0 + r * 4096 : x1 + (r - nb0) * 4096;

    // ---- load: thread owns entries [8 tid, 8 tid + 8) and [2048 + 8 tid, ...)
    uint32_t hw[kPer / 2];
    {
        const uint4 a = reinterpret_cast<const uint4*>(src)[tid];
        const uint4 b = reinterpret_cast<const uint4*>(src)[256 + tid];
        hw[0] = a.x; hw[1] = a.y; hw[2] = a.z; hw[3] = a.w;
        hw[4] = b.x; hw[5] = b.y; hw[6] = b.z; hw[7] = b.w;
    }
    reinterpret_cast<uint4*>(sh.u.a.cnt)[tid] = make_uint4(0u, 0u, 0u, 0u);
    if (tid < 64) {
        sh.lg_c[tid] = tb.lg_c[tid];
        sh.lg_inv[tid] = tb.lg_inv[tid];
    }
    if (kFused && tid < (kMaxS + 1) * kMaxS / 4)
        sh.rcol[tid] = reinterpret_cast<const uint32_t*>(&tb.rt.col[0][0])[tid];
    if (tid == 0) {
        sh.nslots = 0u;
        if (kFused) sh.fz_nf = 0u;
    }
    const uint32_t d = tid < kCL ? tb.desc[tid] : kNoLane;  // this lane's candidate interval
    // and its run (read here, with the other table words, so the candidate
    // phase does not wait on a memory load)
    const uint32_t sg = tb.lseg[tid];
    // this lane's threshold parameters: an order statistic's rank, or a
    // uniform threshold's numerator | denominator << 8
    uint32_t tpar = 0u;
    if (tid < kNQ)
        tpar = (uint32_t)tb.rt.rank[tid];
    else if (tid >= 128 && tid < 128 + kNU)
        tpar = (uint32_t)tb.unum[tid - 128] | ((uint32_t)tb.uden[tid - 128] << 8);
    __syncthreads();

    // ---- sweep 1 (two entries per 32-bit word): canonical -0, keys,
    //      coarse histogram, min/max keys, sum of squares.  NaN and Inf land
    //      in bins 0..15 and 1008..1023, which hold nothing else.
    ushort2_t kmin2 = {0xffff, 0xffff}, kmax2 = {0, 0};
    double sq = 0.0;
    uint32_t keys2[kPer / 2];
#pragma unroll
    for (int p = 0; p < kPer / 2; ++p) {
        half2_t hv;
        const uint32_t k2 = pair_keys(hw[p], hv);  // order-preserving keys of both halves
        keys2[p] = k2;
        const ushort2_t kv = __builtin_bit_cast(ushort2_t, k2);
        kmin2 = __builtin_elementwise_min(kmin2, kv);
        kmax2 = __builtin_elementwise_max(kmax2, kv);
        const double v0 = (double)(float)hv.x, v1 = (double)(float)hv.y;
        sq = fma(v0, v0, sq);
        sq = fma(v1, v1, sq);
        const uint32_t klo = k2 & 0xffffu, khi = k2 >> 16;
        atomicAdd(&sh.u.a.cnt[klo >> 6], (klo & 63u) | kCnt1);
        atomicAdd(&sh.u.a.cnt[khi >> 6], (khi & 63u) | kCnt1);
    }
    {
        const uint32_t kmin = wave_min_u32_dpp(min((uint32_t)kmin2.x, (uint32_t)kmin2.y));
        const uint32_t kmax = wave_max_u32_dpp(max((uint32_t)kmax2.x, (uint32_t)kmax2.y));
        const double sqw = wave_sum_f64(sq);
        if (lane == 0) {
            sh.wmin[wave] = kmin;
            sh.wmax[wave] = kmax;
            sh.wsq[wave] = sqw;
        }
    }
    __syncthreads();
    uint32_t kmin = sh.wmin[0], kmax = sh.wmax[0];
#pragma unroll
    for (int w = 1; w < kW; ++w) {
        kmin = min(kmin, sh.wmin[w]);
        kmax = max(kmax, sh.wmax[w]);
    }
    const double sumsq = (sh.wsq[0] + sh.wsq[1]) + (sh.wsq[2] + sh.wsq[3]);
    const float mn = key_value(kmin);
    const float mx = key_value(kmax);

    // ---- coarse prefix: thread owns bins [4 tid, 4 tid + 4) = keys
    //      [256 tid, 256 tid + 256), one binade: value = B0 + (key offset) U
    {
        // the Inf/NaN code bins (threads 0..3, 252..255) get base and ulp 0:
        // they hold no finite entry, so every prefix term they add is 0
        const bool finite_bins = tid >= 4 && tid < kT - 4;
        const float B0 = finite_bins ? key_value((uint32_t)tid << 8) : 0.0f;
        const double U = finite_bins ? (double)(key_value(((uint32_t)tid << 8) | 1u) - B0) : 0.0;
        const uint4 pw = reinterpret_cast<const uint4*>(sh.u.a.cnt)[tid];
        const uint32_t c[4] = {pw.x >> 19, pw.y >> 19, pw.z >> 19, pw.w >> 19};
        const uint32_t acc[4] = {pw.x & kLowF, 64u * c[1] + (pw.y & kLowF),
                                 128u * c[2] + (pw.z & kLowF), 192u * c[3] + (pw.w & kLowF)};
        const uint32_t ct = (c[0] + c[1]) + (c[2] + c[3]);
        const uint32_t at = (acc[0] + acc[1]) + (acc[2] + acc[3]);
        if ((tid < 4 || tid >= kT - 4) && ct != 0u) {
            if (kFused)
                sh.fz_nf = 1u;  // reported through the count word and the last block
            else
                atomicOr(&ws->status, kStatusNonFinite);
        }
        const double st = (double)ct * (double)B0 + U * (double)at;
        const uint32_t ic = wave_scan_add_u32(ct);
        const double is = wave_scan_add_f64(st);
        if (lane == 63) {
            sh.wtot[wave] = ic;
            sh.wts1[wave] = is;
        }
        __syncthreads();
        const int wv = __builtin_amdgcn_readfirstlane(wave);
        uint32_t oc = 0;
        double os = 0.0;
        for (int w = 0; w < wv; ++w) {  // uniform trip count
            oc += sh.wtot[w];
            os += sh.wts1[w];
        }
        const uint32_t base_c = oc + ic - ct;
        const double base_s = os + (is - st);
        uint32_t runc = 0, runa = 0;
        uint32_t pc[4];
        double ps[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            pc[k] = base_c + runc;
            ps[k] = base_s + (double)runc * (double)B0 + U * (double)runa;
            runc += c[k];
            runa += acc[k];
        }
        reinterpret_cast<uint4*>(sh.u.a.cnt)[tid] = make_uint4(pc[0], pc[1], pc[2], pc[3]);
        reinterpret_cast<double2*>(sh.u.a.ps1)[2 * tid] = make_double2(ps[0], ps[1]);
        reinterpret_cast<double2*>(sh.u.a.ps1)[2 * tid + 1] = make_double2(ps[2], ps[3]);
        reinterpret_cast<uint4*>(sh.slot)[tid] = make_uint4(kNoSlot, kNoSlot, kNoSlot, kNoSlot);
        if (tid == kT - 1) {
            sh.u.a.cnt[kNC] = base_c + ct;
            sh.u.a.ps1[kNC] = base_s + st;
        }
    }
    __syncthreads();

    // ---- order statistics on threads 0..72, uniform thresholds on threads
    //      128..198: find the bin, read its prefix, claim a slot
    if (tid < kNQ) {
        const uint32_t rank = tpar;
        // last bin with prefix count <= rank: 4-way search, the three
        // probes of a step are independent reads
        uint32_t lo = 0;
#pragma unroll
        for (uint32_t step = kNC / 4; step; step >>= 2) {
            const uint32_t c1 = sh.u.a.cnt[lo + step], c2 = sh.u.a.cnt[lo + 2 * step],
                           c3 = sh.u.a.cnt[lo + 3 * step];
            lo += step * ((c1 <= rank ? 1u : 0u) + (c2 <= rank ? 1u : 0u) + (c3 <= rank ? 1u : 0u));
        }
        const uint32_t pc = sh.u.a.cnt[lo];
        sh.tbin[tid] = (uint16_t)lo;
        sh.tloc[tid] = (uint16_t)(rank - pc);
        sh.P[kPQ + tid].cnt = pc;
        sh.P[kPQ + tid].s1 = sh.u.a.ps1[lo];
        claim_slot(sh, lo);
    } else if (tid >= 128 && tid < 128 + kNU) {
        const int u = tid - 128;
        float t;
        {
#pragma clang fp contract(off)
            const double dmn = (double)mn;
            const double span = (double)mx - dmn;
            t = (float)(dmn + (span * (double)(tpar & 0xffu)) / (double)(tpar >> 8));
        }
        const uint32_t key = key_ceil(t);
        const uint32_t bin = key >> 6;
        const uint32_t pc = sh.u.a.cnt[bin];
        sh.ukey[u] = (uint16_t)key;
        sh.P[kPU + u].v = t;
        sh.P[kPU + u].cnt = pc;
        sh.P[kPU + u].s1 = sh.u.a.ps1[bin];
        if (sh.u.a.cnt[bin + 1] != pc) claim_slot(sh, bin);  // an empty bin's edge is exact
    } else if (tid == kT - 1) {
        sh.P[0].v = mn;
        sh.P[0].cnt = 0u;
        sh.P[0].s1 = 0.0;
        sh.P[1].v = mx;
        sh.P[1].cnt = 4096u;
        sh.P[1].s1 = sh.u.a.ps1[kNC];
    }
    __syncthreads();
    const uint32_t nslots = sh.nslots;

    // ---- sweep 2 and the in-bin finish, per round for the slots tagged
    //      `tag` (the keys pass through an empty asm so that sweep 1's
    //      payloads are recomputed here rather than held in registers across
    //      the phases).
    //      At most kNQ + kNU <= 2 kSlots bins are claimed.  Up to kSlots of
    //      them fit the slot memory; a block with more (common for
    //      unit-scale normal or Laplace data, not for data whose outliers
    //      stretch the uniform grid) runs sweep 2 and the finish a second
    //      time for the rest, with its keys recomputed from a second read
    //      of the block.  kSlotsLarge keeps the LDS at 6 workgroups per CU.
    const int rounds = nslots > (uint32_t)kSlots ? 2 : 1;
    uint32_t k2s[kPer / 2];
#pragma unroll
    for (int p = 0; p < kPer / 2; ++p) k2s[p] = keys2[p];
    for (int rnd = 0;; ++rnd) {
    const uint32_t tag = rnd ? kRound2 : 0u;  // slot entries served this round
    const uint32_t ns = rnd ? nslots - (uint32_t)kSlots : min(nslots, (uint32_t)kSlots);
    // each entry's slot entry (the slot table lies outside the memory
    // cleared next, so these reads overlap the clearing and its barrier)
    uint32_t sl[kPer];
#pragma unroll
    for (int p = 0; p < kPer / 2; ++p) {
        asm volatile("" : "+v"(k2s[p]));
        sl[2 * p] = sh.slot[(k2s[p] & 0xffffu) >> 6];
        sl[2 * p + 1] = sh.slot[k2s[p] >> 22];
    }
    for (uint32_t i = tid; i < ns * (kSW / 4); i += kT)
        reinterpret_cast<uint4*>(sh.u.b.w)[i] = make_uint4(0u, 0u, 0u, 0u);
    __syncthreads();
    // the per-entry loop is compiled once per round tag, so the first
    // round (tag 0, the only one for most blocks) needs no XOR
    auto sweep2 = [&](auto tagc) {
    constexpr uint32_t kTag = decltype(tagc)::value;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
        // served this round iff the entry's two high bits equal the tag; then
        // so is the slot's byte offset (kNoSlot ^ tag has a high bit set)
        const uint32_t so = sl[i] ^ kTag;
        if (so < kRound2) {
            // key f = bits [kb, kb + 6) of the word holding both keys; it
            // counts 1 in the 16-bit half f & 1 of word f >> 1 of the slot
            const uint32_t k2 = k2s[i >> 1];
            uint32_t cword, one;
            if (i & 1) {
                cword = bfe_u32<17, 5>(k2);
                one = mad_u24(bfe_u32<16, 1>(k2), 0xffffu, 1u);
            } else {
                cword = bfe_u32<1, 5>(k2);
                one = mad_u24(k2 & 1u, 0xffffu, 1u);
            }
            uint32_t* slotw = reinterpret_cast<uint32_t*>(reinterpret_cast<char*>(sh.u.b.w) + so);
            atomicAdd(slotw + cword, one);
        }
    }
    };
    if (rnd == 0)
        sweep2(RoundTag<0u>{});
    else
        sweep2(RoundTag<kRound2>{});
    __syncthreads();
    // ---- group totals of this round's slots, (count << 19) + sum of f over
    //      each 8-key group, from the per-key counters: one (slot, group) per
    //      thread and step.  Group g is the slot's quad g (keys 8g .. 8g+7,
    //      word m holding keys 8g + 2m and 8g + 2m + 1).  Adding these in
    //      sweep 2 instead, one LDS atomic per entry into 8 words per slot,
    //      serialises on equal addresses: those atomics alone cost ~9% of
    //      the kernel; this pass and its barrier give back most of that
    //      (net 2%, and 1% better than each finishing lane summing its own
    //      slot's groups).
    for (uint32_t t = tid; t < ns * 8u; t += kT) {
        const uint32_t sb = (t >> 3) * (uint32_t)(4 * kSW), g = t & 7u;
        const uint4 q = slot_quad(sh, sb, g);
        const uint32_t c = udot2(q.w, 0x00010001u, udot2(q.z, 0x00010001u,
                                 udot2(q.y, 0x00010001u, udot2(q.x, 0x00010001u, 0u))));
        const uint32_t fl = udot2(q.w, 0x00070006u, udot2(q.z, 0x00050004u,
                                  udot2(q.y, 0x00030002u, udot2(q.x, 0x00010000u, 0u))));
        reinterpret_cast<uint32_t*>(reinterpret_cast<char*>(sh.u.b.w) + sb)[kFW + g] =
            (c << 19) + 8u * g * c + fl;
    }
    __syncthreads();
    // ---- finish the prefixes inside the bins
    const uint32_t sv = tid < kNQ ? sh.slot[sh.tbin[tid]]
                      : (tid >= 128 && tid < 128 + kNU ? sh.slot[sh.ukey[tid - 128] >> 6] : kNoSlot);
    const uint32_t s = sv & kSlotOff;
    if (tid < kNQ && (sv & ~kSlotOff) == tag) {
        const uint32_t bin = sh.tbin[tid];
        const uint32_t loc = sh.tloc[tid];
        const uint4 ga = slot_quad(sh, s, 8), gb = slot_quad(sh, s, 9);
        // group holding local rank loc: groups whose running count <= loc
        const uint32_t lim = (loc + 1u) << 19;
        uint32_t S = 0, Pg = 0, gi = 0;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            S += word_of(ga, gb, i);
            const bool take = S < lim;
            gi += take ? 1u : 0u;
            Pg = take ? S : Pg;
        }
        gi = min(gi, 7u);
        const uint4 fw = slot_quad(sh, s, gi);
        const uint32_t rlim = (loc - (Pg >> 19) + 1u) << 19;
        uint32_t T = 0, Ts = 0, kk = 0;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            T += key_count(fw, i) * (kCnt1 + (uint32_t)i);
            const bool take = T < rlim;
            kk += take ? 1u : 0u;
            Ts = take ? T : Ts;
        }
        const uint32_t f = min(8u * gi + kk, 63u);
        const uint32_t nl = Ts >> 19;
        const uint32_t N = (Pg >> 19) + nl;
        const uint32_t F = (Pg & kLowF) + 8u * gi * nl + (Ts & kLowF);
        const float B = key_value(bin << 6);
        const float U = key_value((bin << 6) | 1u) - B;
        const float v = key_value((bin << 6) | f);
        sh.P[kPQ + tid].v = v;
        sh.P[kPQ + tid].cnt += N;
        if (N) sh.P[kPQ + tid].s1 += (double)B * (double)N + (double)U * (double)F;
        stats[tid * R + r] = v;
    } else if (tid >= 128 && tid < 128 + kNU && (sv & ~kSlotOff) == tag) {
        const int u = tid - 128;
        const uint32_t key = sh.ukey[u];
        const uint32_t bin = key >> 6;
        {
            const uint32_t f = key & 63u;
            const uint32_t gs = f >> 3, fs = f & 7u;
            const uint4 ga = slot_quad(sh, s, 8), gb = slot_quad(sh, s, 9);
            uint32_t S = 0;
#pragma unroll
            for (int i = 0; i < 8; ++i) S += (uint32_t)i < gs ? word_of(ga, gb, i) : 0u;
            const uint4 fw = slot_quad(sh, s, gs);
            uint32_t T = 0;
#pragma unroll
            for (int i = 0; i < 8; ++i)
                T += (uint32_t)i < fs ? key_count(fw, i) * (kCnt1 + (uint32_t)i) : 0u;
            const uint32_t nl = T >> 19;
            const uint32_t N = (S >> 19) + nl;
            const uint32_t F = (S & kLowF) + 8u * gs * nl + (T & kLowF);
            const float B = key_value(bin << 6);
            const float U = key_value((bin << 6) | 1u) - B;
            sh.P[kPU + u].cnt += N;
            if (N) sh.P[kPU + u].s1 += (double)B * (double)N + (double)U * (double)F;
        }
    }
    __syncthreads();  // phase-B storage is reused by the next round or below
    if (rnd + 1 >= rounds) break;
    {
        const uint4 a = reinterpret_cast<const uint4*>(src)[tid];
        const uint4 b = reinterpret_cast<const uint4*>(src)[256 + tid];
        const uint32_t hw2[kPer / 2] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
        for (int p = 0; p < kPer / 2; ++p) k2s[p] = pair_keys(hw2[p]);
    }
    }

    // ---- candidate intervals, one per lane: masses to both ends, the
    //      distortion term a^2 M_a + b^2 M_b and the entropy term of the
    //      right point (its mass: this interval's share plus the next one's)
    const bool last = ((d >> 8) & 0xffu) == 1u;  // right point is the maximum
    double ma = 0.0, mb = 0.0, dterm = 0.0;
    float bq = 0.0f;
    bool zero_width = false;
    if (d != kNoLane) {
        const Point pa = sh.P[d & 0xffu];
        const Point pb = sh.P[(d >> 8) & 0xffu];
        const double A = pa.v, Bq = pb.v;
        const double C = (double)(pb.cnt - pa.cnt);
        const double wd = Bq - A;
        mb = C;  // an interval between equal points carries the entries equal
                 // to them (possible only at the closed maximum)
        if (wd > 0.0) {
            mb = (pb.s1 - pa.s1 - A * C) * recip(wd);
            mb = fmin(fmax(mb, 0.0), C);
        } else {
            zero_width = true;
        }
        ma = C - mb;
        dterm = A * A * ma + Bq * Bq * mb;
        bq = pb.v;
    }
    const double ma_next = dpp_zero_f64<kDppRowShl1>(ma);  // 0 in a row's last lane
    const double mr = last ? mb : mb + ma_next;

    // ---- per candidate: D = sum of its intervals' terms - sum x^2 and
    //      H = sum of its points' entropy terms.  A candidate's intervals
    //      are consecutive lanes of one 16-lane row, so both sums are
    //      segmented inclusive scans within the row (shifts of 1, 2, 4, 8
    //      lanes, added when the source lane is of the same candidate); the
    //      candidate's last lane writes them.  The first interval also
    //      carries the entropy term of its left point.
    const bool live = sg != kNoLane;
    const uint32_t off = (sg >> 5) & 15u;
    double dsum = live ? dterm : 0.0;
    double hsum = 0.0;
    if (live) {
        hsum = point_entropy(mr, sh.lg_c, sh.lg_inv);
        if (off == 0u) hsum += point_entropy(ma, sh.lg_c, sh.lg_inv);
    }
    seg_scan_step<kDppRowShr1, 1>(off, dsum, hsum);
    seg_scan_step<kDppRowShr2, 2>(off, dsum, hsum);
    seg_scan_step<kDppRowShr4, 4>(off, dsum, hsum);
    seg_scan_step<kDppRowShr8, 8>(off, dsum, hsum);
    // equal consecutive points (tied data only): a candidate with a
    // zero-width interval merges their masses first, from its intervals'
    // values that its wave leaves in LDS
    PhaseC& pc = sh.u.c;
    uint32_t zw = 0u;  // zero-width intervals up to this lane in its candidate
    if (__any(zero_width)) {
        zw = zero_width ? 1u : 0u;
        seg_scan_step<kDppRowShr1, 1>(off, zw);
        seg_scan_step<kDppRowShr2, 2>(off, zw);
        seg_scan_step<kDppRowShr4, 4>(off, zw);
        seg_scan_step<kDppRowShr8, 8>(off, zw);
        pc.mr[tid] = mr;
        pc.ma[tid] = ma;
        pc.bv[tid] = bq;
        __builtin_amdgcn_wave_barrier();
    }
    if (live && (sg >> 9) != 0u) {
        const uint32_t c = sg & 31u;
        const double dout = mx > mn ? fmax(dsum - sumsq, 0.0) : 0.0;
        Dout[c * R + r] = dout;
        if (kFused) pc.cd[c] = dout;
        double h = hsum;
        if (zw != 0u) {
            const uint32_t first = (uint32_t)tid - off;
            h = 0.0;
            double acc = pc.ma[first];
            float val = mn;
            for (uint32_t i = first; i <= (uint32_t)tid; ++i) {
                const float b = pc.bv[i];
                const double m = pc.mr[i];
                if (b == val) {
                    acc += m;
                } else {
                    h += point_entropy(acc, sh.lg_c, sh.lg_inv);
                    acc = m;
                    val = b;
                }
            }
            h += point_entropy(acc, sh.lg_c, sh.lg_inv);
        }
        const double hout = mx > mn ? fmax(h, 0.0) : 0.0;
        Hout[c * R + r] = hout;
        if (kFused) pc.chh[c] = hout;
    }
    if constexpr (kFused) fused_tail(sh, tb, fa, ws, r, R, hw);
}

// The kernel's tables: distinct uniform fractions, lane layout of the
// candidate intervals, log2 cells.
static hipError_t build_tables(const RankTable& rt, Eval16Tables& tb) {
    memset(&tb, 0, sizeof tb);
    tb.rt = rt;
    // distinct interior fractions j/(k-1), k = 3..16, in order of first appearance
    uint8_t ucol[kMaxS + 1][kMaxS];
    memset(ucol, 0, sizeof ucol);
    int nu = 0;
    for (int k = 3; k <= kMaxS; ++k)
        for (int j = 1; j <= k - 2; ++j) {
            int a = j, b = k - 1;
            int g0 = a, g1 = b;  // gcd
            while (g1) {
                const int t = g0 % g1;
                g0 = g1;
                g1 = t;
            }
            a /= g0;
            b /= g0;
            int found = -1;
            for (int u = 0; u < nu; ++u)
                if (tb.unum[u] == a && tb.uden[u] == b) found = u;
            if (found < 0) {
                tb.unum[nu] = (uint8_t)a;
                tb.uden[nu] = (uint8_t)b;
                found = nu++;
            }
            ucol[k][j] = (uint8_t)found;
        }
    if (nu != kNU || rt.n_stats != kNQ) return hipErrorInvalidValue;
    // Candidates: 0 = {min, max}; 1 + 2(k-3) = U_k, 2 + 2(k-3) = E_k.
    // Point j of a k-point candidate in the point table.
    auto point = [&](int c, int j) -> int {
        const int k = c == 0 ? 2 : 3 + (c - 1) / 2;
        if (j == 0) return 0;
        if (j == k - 1) return 1;
        const bool uni = ((c - 1) & 1) == 0;
        return uni ? kPU + ucol[k][j] : kPQ + rt.col[k][j];
    };
    auto cand = [](int k, bool uni) { return k == 2 ? 0 : (uni ? 1 : 2) + 2 * (k - 3); };
    // Rows of 16 lanes, each holding the intervals (k - 1 per candidate) of
    // whole candidates: {U16, {min,max}}, {E16}, {U/E k, U/E 18 - k} for
    // k = 15..10, {U9, E9}.
    int rows[kRows][2];
    int nr = 0;
    rows[nr][0] = cand(16, true);  rows[nr][1] = cand(2, true); ++nr;
    rows[nr][0] = cand(16, false); rows[nr][1] = -1; ++nr;
    for (int k = 15; k >= 10; --k) {
        rows[nr][0] = cand(k, true);  rows[nr][1] = cand(18 - k, true); ++nr;
        rows[nr][0] = cand(k, false); rows[nr][1] = cand(18 - k, false); ++nr;
    }
    rows[nr][0] = cand(9, true); rows[nr][1] = cand(9, false); ++nr;
    if (nr != kRows) return hipErrorInvalidValue;
    for (int l = 0; l < kCL; ++l) tb.desc[l] = tb.lseg[l] = (uint16_t)kNoLane;
    int placed = 0;
    for (int row = 0; row < kRows; ++row) {
        int lane = 16 * row;
        for (int h = 0; h < 2; ++h) {
            const int c = rows[row][h];
            if (c < 0) continue;
            const int k = c == 0 ? 2 : 3 + (c - 1) / 2;
            if (lane + (k - 1) > 16 * (row + 1)) return hipErrorInvalidValue;
            tb.red[c] = (uint16_t)(lane | ((k - 1) << 8));
            for (int j = 0; j < k - 1; ++j, ++lane) {
                tb.desc[lane] = (uint16_t)(point(c, j) | (point(c, j + 1) << 8));
                tb.lseg[lane] = (uint16_t)(c | (j << 5) | ((j == k - 2 ? 1 : 0) << 9));
            }
            ++placed;
        }
    }
    if (placed != kMaxCand) return hipErrorInvalidValue;
    for (int i = 0; i < 64; ++i) {
        const double c = 1.0 + (double)(2 * i + 1) / 128.0;
        tb.lg_c[i] = log2(c);
        tb.lg_inv[i] = 1.0 / c;
    }
    return hipSuccess;
}

// The tables for rt, built once per thread and rank table (they are the
// same for every call of a given block size and s).
static hipError_t make_tables(const RankTable& rt, Eval16Tables& tb) {
    thread_local RankTable last_rt;
    thread_local Eval16Tables last_tb;
    thread_local bool have = false;
    if (!have || memcmp(&last_rt, &rt, sizeof rt) != 0) {
        const hipError_t e = build_tables(rt, last_tb);
        if (e != hipSuccess) return e;
        last_rt = rt;
        have = true;
    }
    tb = last_tb;
    return hipSuccess;
}

hipError_t launch_eval16(const void* x0, const void* x1, int64_t nb0, int64_t R, const RankTable& rt,
                         double* D, double* H, float* stats, void* ws, hipStream_t st) {
    if (R == 0) return hipSuccess;
    Eval16Tables tb;
    const hipError_t te = make_tables(rt, tb);
    if (te != hipSuccess) return te;
    if (R < kEvalSmallLaunch)
        hipLaunchKernelGGL(eval16_kernel<kSlotsAll>, dim3((unsigned)R), dim3(kT), 0, st, (const __half*)x0,
                       (const __half*)x1, nb0, tb, D, H, stats, (WsHeader*)ws, FusedArgs{});
    else
        hipLaunchKernelGGL(eval16_kernel<kSlotsLarge>, dim3((unsigned)R), dim3(kT), 0, st, (const __half*)x0,
                       (const __half*)x1, nb0, tb, D, H, stats, (WsHeader*)ws, FusedArgs{});
    return hipGetLastError();
}

// Clears a one-launch admission's words buffer (both arrays).
__global__ void __launch_bounds__(1024) fused_words_clear_kernel(uint64_t* words) {
    const int tid = threadIdx.x;
    words[tid] = 0u;
    words[kFusedMaxBlocks + tid] = 0u;
}
static_assert(kFusedMaxBlocks == 1024, "one thread per block index");

hipError_t launch_fused_words_clear(uint64_t* words, hipStream_t st) {
    hipLaunchKernelGGL(fused_words_clear_kernel, dim3(1), dim3(1024), 0, st, words);
    return hipGetLastError();
}

hipError_t launch_admit_fused(const void* x0, const void* x1, int64_t nb0, int64_t R, const RankTable& rt,
                              double lam_in, int shift, uint64_t seed, double* D, double* H, float* stats,
                              int32_t* choice, float* codebook, uint8_t* m, uint64_t* off, uint32_t* codes,
                              void* ws, uint64_t* words, uint32_t epoch, SolveOut* out, hipStream_t st) {
    if (R < 1 || R > kFusedMaxBlocks || epoch < 1u || epoch > kFusedEpochMax) return hipErrorInvalidValue;
    Eval16Tables tb;
    const hipError_t te = make_tables(rt, tb);
    if (te != hipSuccess) return te;
    WsHeader* h = (WsHeader*)ws;
    uint64_t* desc = words;
    uint64_t* rates = words + kFusedMaxBlocks;
    FusedArgs fa;
    fa.epoch = epoch;
    fa.lam = lam_in;
    fa.shift = shift;
    fa.k0 = (uint32_t)seed;
    fa.k1 = (uint32_t)(seed >> 32);
    fa.choice = choice;
    fa.codebook = codebook;
    fa.m = m;
    fa.off = off;
    fa.desc = desc;
    fa.rates = rates;
    fa.codes = codes;
    fa.out = out;
    hipLaunchKernelGGL((eval16_kernel<kSlotsAll, true>), dim3((unsigned)R), dim3(kT), 0, st, (const __half*)x0,
                       (const __half*)x1, nb0, tb, D, H, stats, h, fa);
    return hipGetLastError();
}

}  // namespace kvq
