// Entropy coding of each block's symbol stream with interleaved rANS.
//
// Page "Rate-adaptive KV-cache quantizer", Implementation notes: the stored
// form is the codebook, the symbol stream and the block lengths, and the
// stream is arithmetic-coded.  rANS (J. Duda, "Asymmetric numeral systems",
// arXiv:1311.2540) codes each block with its own symbol counts as the model:
//   * n entries, k = ceil(log2 n), M = 2^k; f_j = count of symbol j, the most
//     frequent symbol (lowest index among equals) also takes M - n;
//     C_j = f_0 + ... + f_{j-1};
//   * 32-bit states in [2^16, 2^32), 16-bit words; encoding s from x: if
//     x >> (32 - k) >= f_s emit x & 0xffff and x >>= 16, then
//     x = floor(x / f_s) 2^k + (x mod f_s) + C_s; decoding inverts it and
//     refills a word whenever x < 2^16;
//   * 8 states per block, state i codes entries i, i + 8, i + 16, ...; the
//     words emitted at step j, in state order, form group j;
//   * block layout (16-bit little-endian words): f_0 .. f_{m-1}, the final
//     states as (hi, lo) pairs in state order, groups j = 0, 1, ..., then a
//     zero word if needed to fill a 32-bit word.
//
// Eight lanes code one block in lock step; a wave holds 8 blocks and a
// workgroup 32.  The encoder runs backwards from the block's last step and
// places each group below the previous one in a per-block scratch region
// (sized from the fixed-width stream plus a margin); a scan of the block
// sizes and a copy kernel then give the dense stream.  The decoder runs
// forwards, one refill word per state at most per step, and writes the
// decoded codepoints (fp32) directly.
#include "kvq_internal.h"

namespace kvq {

namespace {

constexpr int kAL = 8;                    // states per block
constexpr int kAT = 256;                  // threads per workgroup
constexpr int kAB = kAT / kAL;            // blocks per workgroup
constexpr uint32_t kStateLow = 1u << 16;

struct AnsSym {                           // one symbol of a block's model
    uint32_t f, c;                        // frequency, cumulative frequency
    double rcp;                           // 1 / f (round to nearest)
};

// This block's 8 bits of a wave ballot, for the lane's group of 8.
__device__ __forceinline__ uint32_t group_bits(uint64_t ballot, int lane) {
    return (uint32_t)(ballot >> (lane & ~7)) & 0xffu;
}

}  // namespace

__host__ __device__ uint64_t ans_margin_bytes(int n) { return 128u + 4u * (uint64_t)((n + 63) / 64); }

__global__ void __launch_bounds__(kAT)
ans_encode_kernel(const uint32_t* __restrict__ codes, const uint8_t* __restrict__ m_in,
                  const uint64_t* __restrict__ word_off, int64_t R, int n, int s, int k,
                  uint16_t* __restrict__ scratch, uint64_t* __restrict__ block_bytes, WsHeader* ws) {
    __shared__ uint32_t cnt[kAB][kMaxS];
    __shared__ AnsSym tab[kAB][kMaxS];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int bl = tid >> 3;          // block slot in the workgroup
    const int i = tid & 7;            // state
    const int64_t r = (int64_t)blockIdx.x * kAB + bl;
    const bool valid = r < R;
    for (int j = i; j < kMaxS; j += kAL) cnt[bl][j] = 0u;
    const int m = valid ? min(max((int)m_in[r], 1), s) : 1;
    const int w = code_width(m);
    const uint32_t mask = (1u << w) - 1u;
    const uint64_t w0 = valid ? word_off[r] : 0, w1 = valid ? word_off[r + 1] : 0;
    const uint32_t* cw = codes + w0;
    const uint32_t nwords = (uint32_t)(w1 - w0);
    const int steps = (n + kAL - 1) / kAL;
    // The two stream words holding step j's 8 w bits, loaded raw into a
    // ring slot kPf steps before the step uses them: the loads are
    // unconditional (past the block's words, or for j < 0, they read
    // word_off[0]) and the out-of-range words are zeroed only at the use,
    // and each slot is a fixed register (the loops are unrolled by kPf).  A
    // load under a branch was waited on in its own step; with the ring the
    // waits come at most once per round (the compiler still drains the
    // counter around the coding loop's conditional stores): encode of the
    // long-context stream 4.47 -> 4.35 ms.
    const uint32_t* dummy = reinterpret_cast<const uint32_t*>(word_off);
    auto word_at = [&](int j) { return j >= 0 ? (uint32_t)(8 * w * j) >> 5 : nwords; };
    auto fetch = [&](int j, uint32_t& lo, uint32_t& hi) {
        const uint32_t q = word_at(j);
        lo = *(q < nwords ? cw + q : dummy);
        hi = *(q + 1 < nwords ? cw + q + 1 : dummy);
    };
    // step j's bits from its raw words (only the low 8 w are meaningful)
    auto bits_of = [&](uint32_t lo, uint32_t hi, int j) {
        const uint32_t q = word_at(j);
        const uint64_t win = ((uint64_t)(q + 1 < nwords ? hi : 0u) << 32) | (q < nwords ? lo : 0u);
        return (uint32_t)(win >> ((8u * (uint32_t)w * (uint32_t)j) & 31u));
    };
    constexpr int kPf = 4;
    __syncthreads();
    // ---- symbol counts: lane i takes steps i, i + 8, ... (all 8 codes of a
    //      step from one read of the stream)
    if (valid) {
        uint32_t clo[kPf], chi[kPf];
#pragma unroll
        for (int d = 0; d < kPf; ++d) fetch(i + kAL * d < steps ? i + kAL * d : -1, clo[d], chi[d]);
        for (int j0 = i; j0 < steps; j0 += kAL * kPf) {
#pragma unroll
            for (int u = 0; u < kPf; ++u) {
                const int j = j0 + kAL * u;
                if (j < steps) {
                    const uint32_t b8 = w ? bits_of(clo[u], chi[u], j) : 0u;
                    const int jn = j + kAL * kPf;
                    fetch(jn < steps ? jn : -1, clo[u], chi[u]);
#pragma unroll
                    for (int e = 0; e < kAL; ++e)
                        if (kAL * j + e < n) atomicAdd(&cnt[bl][(b8 >> (w * e)) & mask], 1u);
                }
            }
        }
    }
    __syncthreads();
    // ---- model: lanes 0 and 1 of each block fill 8 symbols each
    if (valid && i < 2) {
        uint32_t best = 0, bestc = cnt[bl][0];
        for (int j = 1; j < m; ++j)
            if (cnt[bl][j] > bestc) { best = j; bestc = cnt[bl][j]; }
        const uint32_t extra = (1u << k) - (uint32_t)n;
        uint32_t c = 0;
        for (int j = 0; j < m; ++j) {
            const uint32_t f = cnt[bl][j] + ((uint32_t)j == best ? extra : 0u);
            if (j >= 8 * i && j < 8 * i + 8) {
                tab[bl][j].f = f;
                tab[bl][j].c = c;
                tab[bl][j].rcp = f ? 1.0 / (double)f : 0.0;
            }
            c += f;
        }
    }
    __syncthreads();
    if (!valid) return;
    // ---- code the steps backwards; groups are placed downwards from the end
    //      of the block's region, which starts with a 4-byte start marker
    const uint64_t base = (4u * w0 + (uint64_t)r * ans_margin_bytes(n)) / 2;  // in words
    const uint64_t capw = (4u * (w1 - w0) + ans_margin_bytes(n)) / 2;
    const int64_t lowest = (int64_t)(base + 2 + (uint64_t)m + 2 * kAL);  // marker, table, states
    int64_t ptr = (int64_t)(base + capw);
    uint32_t x = kStateLow;
    bool overflow = false;
    // steps j .. j - kPf + 1 have their words in flight while step j is
    // coded (ring slot u holds step j0 - u of the round j0)
    uint32_t plo[kPf], phi[kPf];
#pragma unroll
    for (int d = 0; d < kPf; ++d) fetch(steps - 1 - d, plo[d], phi[d]);
    for (int j0 = steps - 1; j0 >= 0; j0 -= kPf) {
#pragma unroll
    for (int u = 0; u < kPf; ++u) {
        const int j = j0 - u;
        if (j < 0) continue;  // the same for every lane
        const int t = kAL * j + i;
        const bool act = t < n;
        const uint32_t b_cur = bits_of(plo[u], phi[u], j);
        fetch(j - kPf, plo[u], phi[u]);
        const uint32_t sym = (act && w) ? (b_cur >> (w * i)) & mask : 0u;
        const AnsSym e = tab[bl][sym];
        const bool emit = act && (x >> (32 - k)) >= e.f;
        const uint32_t bits = group_bits(__ballot(emit), lane);
        ptr -= __popc(bits);
        if (emit) {
            const int64_t at = ptr + __popc(bits & ((1u << i) - 1u));
            if (at >= lowest) scratch[at] = (uint16_t)(x & 0xffffu);
            else overflow = true;
            x >>= 16;
        }
        if (act) {
            // floor(x / f): x / f + 2^-19 is within 2^-18 of x / f and more
            // than 2^-13 below the next integer, so truncation is exact
            const uint32_t q = (uint32_t)fma((double)x, e.rcp, 0x1p-19);
            x = (q << k) + (x - q * e.f) + e.c;
        }
    }
    }
    // final states (hi, lo) in state order, then the table below them; a
    // region too small (not expected: see ans_margin_bytes) is reported and
    // left with a size that stays inside it
    int64_t st0 = ptr - 2 * kAL;
    if (st0 - m >= (int64_t)base + 2) {
        scratch[st0 + 2 * i] = (uint16_t)(x >> 16);
        scratch[st0 + 2 * i + 1] = (uint16_t)(x & 0xffffu);
        for (int j = i; j < m; j += kAL) scratch[st0 - m + j] = (uint16_t)tab[bl][j].f;
    } else {
        overflow = true;
        st0 = (int64_t)base + 2 + m;
    }
    if (i == 0) {
        const uint64_t start = (uint64_t)(st0 - m);
        const uint64_t words = base + capw - start;
        reinterpret_cast<uint32_t*>(scratch + base)[0] = (uint32_t)(start - base);
        block_bytes[r + 1] = (2 * words + 3) & ~(uint64_t)3;
        if (r == 0) block_bytes[0] = 0;
    }
    if (overflow) atomicOr(&ws->status, kStatusAnsOverflow);
}

// Copy each block's coded words from its scratch region to the dense stream
// at the scanned byte offset, with the zero fill word.
__global__ void __launch_bounds__(kAT)
ans_compact_kernel(const uint16_t* __restrict__ scratch, const uint64_t* __restrict__ word_off,
                   int64_t R, int n, const uint64_t* __restrict__ block_off, uint8_t* __restrict__ stream) {
    const int64_t r = blockIdx.x;
    const uint64_t w0 = word_off[r], w1 = word_off[r + 1];
    const uint64_t base = (4u * w0 + (uint64_t)r * ans_margin_bytes(n)) / 2;
    const uint64_t capw = (4u * (w1 - w0) + ans_margin_bytes(n)) / 2;
    const uint64_t start = base + reinterpret_cast<const uint32_t*>(scratch + base)[0];
    const uint64_t words = base + capw - start;
    // 4-byte units: the destination is 4-byte aligned, the source start may
    // sit on a 2-byte boundary (then each unit straddles two aligned words)
    uint32_t* out = reinterpret_cast<uint32_t*>(stream + block_off[r]);
    const uint64_t units = (block_off[r + 1] - block_off[r]) / 4;
    const uint32_t* src = reinterpret_cast<const uint32_t*>(scratch);
    const uint64_t a0 = start >> 1;
    const bool odd = start & 1u;
    for (uint64_t q = threadIdx.x; q < units; q += kAT) {
        uint32_t v;
        if (2 * q + 1 < words) {
            // both halves are data; with an odd start u16 start + 2q is the
            // high half of word a0 + q (regions have even ends, so word
            // a0 + q + 1 still lies inside this block's region)
            v = odd ? __builtin_amdgcn_alignbit(src[a0 + q + 1], src[a0 + q], 16) : src[a0 + q];
        } else {
            v = scratch[start + 2 * q];   // the last data word, then the zero fill word
        }
        out[q] = v;
    }
}

// Decode every block and write its codepoints (fp32, entries row-major).
// A workgroup is one wave of 8 blocks.  The 8 blocks' coded bytes are
// consecutive in the stream; when they fit kDecodeStage bytes the wave
// first copies them into LDS with coalesced 4-byte loads, so the refills
// that sit on every state update come from LDS; larger workgroups (over 2
// coded bits per entry on average) refill from global memory.
constexpr int kDB = 8;                    // blocks per decode workgroup
constexpr int kDT = kDB * kAL;            // 64 threads
constexpr uint32_t kDecodeStage = 8448;   // staged bytes per workgroup

// The decode loop of one block's state i over a word stream wd (LDS or
// global memory); false if the stream runs out or the state does not end
// at its start value.
template <typename WordPtr>
__device__ __forceinline__ bool decode_steps(WordPtr wd, uint32_t nwd, const uint32_t* cum,
                                             const uint32_t* frq, const float* q, int m, int n, int k,
                                             int i, int lane, float* __restrict__ out) {
    const uint32_t M = 1u << k;
    uint32_t x = ((uint32_t)wd[m + 2 * i] << 16) | wd[m + 2 * i + 1];
    uint32_t ptr = (uint32_t)m + 2 * kAL;
    bool bad = false;
    const int steps = (n + kAL - 1) / kAL;
    for (int j = 0; j < steps; ++j) {
        const int t = kAL * j + i;
        const bool act = t < n;
        const uint32_t slot = x & (M - 1u);
        // last symbol with C_sym <= slot (C is padded with M past m)
        uint32_t sym = 0;
#pragma unroll
        for (uint32_t h = kMaxS / 2; h; h >>= 1)
            if (cum[sym + h] <= slot) sym += h;
        if (act) x = frq[sym] * (x >> k) + slot - cum[sym];
        const bool need = act && x < kStateLow;
        const uint32_t bits = group_bits(__ballot(need), lane);
        if (need) {
            const uint32_t at = ptr + __popc(bits & ((1u << i) - 1u));
            const uint32_t word = at < nwd ? wd[at] : 0u;
            bad |= at >= nwd;
            x = (x << 16) | word;
        }
        ptr += __popc(bits);
        if (act) out[t] = q[sym];
    }
    return x == kStateLow && !bad;
}

__global__ void __launch_bounds__(kDT)
ans_decode_kernel(const uint8_t* __restrict__ stream, const uint64_t* __restrict__ block_off,
                  const float* __restrict__ codebook, const uint8_t* __restrict__ m_in, int64_t R,
                  int n, int s, int k, float* __restrict__ xhat, WsHeader* ws) {
    __shared__ __align__(16) uint32_t lds_words[kDecodeStage / 4];
    __shared__ uint32_t cum[kDB][kMaxS + 1];   // C_j, padded with 2^k
    __shared__ uint32_t frq[kDB][kMaxS];
    __shared__ float q[kDB][kMaxS];
    const int tid = threadIdx.x;
    const int bl = tid >> 3;
    const int i = tid & 7;
    const int64_t r0 = (int64_t)blockIdx.x * kDB;
    const int64_t r = r0 + bl;
    const bool valid = r < R;
    const int64_t rl = min(r0 + kDB, R);          // one past the workgroup's last block
    const uint64_t b0 = block_off[r0], b1 = block_off[rl];
    // stage the workgroup's bytes (whole 4-byte words: block sizes are
    // multiples of 4 and the stream is 4-byte aligned)
    const bool staged = b1 - b0 <= kDecodeStage;
    if (staged) {
        const uint32_t nw = (uint32_t)((b1 - b0) / 4);
        const uint32_t* src = reinterpret_cast<const uint32_t*>(stream + b0);
        for (uint32_t t = tid; t < nw; t += kDT) lds_words[t] = src[t];
    }
    const int m = valid ? min(max((int)m_in[r], 1), s) : 1;
    const uint32_t M = 1u << k;
    __syncthreads();
    const uint64_t wbeg = valid ? (block_off[r] - b0) / 2 : 0;   // block start, in words
    const uint64_t wend = valid ? (block_off[r + 1] - b0) / 2 : 0;
    // kept apart so that each path's refills use its own memory's loads
    const uint16_t* ld = reinterpret_cast<const uint16_t*>(lds_words) + wbeg;
    const uint16_t* gd = reinterpret_cast<const uint16_t*>(stream + b0) + wbeg;
    const uint32_t nwd = (uint32_t)min(wend - wbeg, (uint64_t)0xffffffffu);
    if (valid && i == 0) {
        // the 16 table words first (independent loads), then the prefix
        uint32_t fw[kMaxS];
        if (staged) {
#pragma unroll
            for (int j = 0; j < kMaxS; ++j) fw[j] = j < m && (uint32_t)j < nwd ? ld[j] : 0u;
        } else {
#pragma unroll
            for (int j = 0; j < kMaxS; ++j) fw[j] = j < m && (uint32_t)j < nwd ? gd[j] : 0u;
        }
        uint32_t c = 0;
#pragma unroll
        for (int j = 0; j < kMaxS; ++j) {
            cum[bl][j] = j < m ? c : M;
            frq[bl][j] = fw[j];
            q[bl][j] = j < m ? codebook[r * s + j] : 0.0f;
            c += fw[j];
        }
        cum[bl][kMaxS] = M;
    }
    __syncthreads();
    if (!valid) return;
    const uint32_t hdr = (uint32_t)m + 2 * kAL;
    if (nwd < hdr) {
        atomicOr(&ws->status, kStatusAnsCorrupt);
        return;
    }
    const bool ok = staged ? decode_steps(ld, nwd, cum[bl], frq[bl], q[bl], m, n, k, i, tid & 63,
                                          xhat + r * (int64_t)n)
                           : decode_steps(gd, nwd, cum[bl], frq[bl], q[bl], m, n, k, i, tid & 63,
                                          xhat + r * (int64_t)n);
    if (!ok) atomicOr(&ws->status, kStatusAnsCorrupt);
}

hipError_t launch_ans_encode(const uint32_t* codes, const uint8_t* m, const uint64_t* word_off,
                             int64_t R, int n, int s, uint16_t* scratch, uint8_t* stream,
                             uint64_t* block_off, void* ws, hipStream_t st) {
    if (R == 0) return hipSuccess;
    const int k = n <= 1 ? 1 : 32 - __builtin_clz((unsigned)(n - 1));
    const unsigned grid = (unsigned)((R + kAB - 1) / kAB);
    hipLaunchKernelGGL(ans_encode_kernel, dim3(grid), dim3(kAT), 0, st, codes, m, word_off, R, n, s, k,
                       scratch, block_off, (WsHeader*)ws);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    e = launch_offsets_scan(block_off, R, ws, st);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(ans_compact_kernel, dim3((unsigned)R), dim3(kAT), 0, st, scratch, word_off, R, n,
                       block_off, stream);
    return hipGetLastError();
}

hipError_t launch_ans_decode(const uint8_t* stream, const uint64_t* block_off, const float* codebook,
                             const uint8_t* m, int64_t R, int n, int s, float* xhat, void* ws,
                             hipStream_t st) {
    if (R == 0) return hipSuccess;
    const int k = n <= 1 ? 1 : 32 - __builtin_clz((unsigned)(n - 1));
    const unsigned grid = (unsigned)((R + kDB - 1) / kDB);
    hipLaunchKernelGGL(ans_decode_kernel, dim3(grid), dim3(kDT), 0, st, stream, block_off, codebook, m, R,
                       n, s, k, xhat, (WsHeader*)ws);
    return hipGetLastError();
}

}  // namespace kvq
