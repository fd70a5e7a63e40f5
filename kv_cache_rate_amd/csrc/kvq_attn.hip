// Decode attention over the quantized cache, decoding K and V in registers.
//
// Page "Rate-adaptive KV-cache quantizer", Implementation notes: the cache is
// decoded before attention; here the decode happens inside the attention
// kernel, so HBM carries only the fixed-width codes and the codebooks.  For
// one new query per query head (grouped heads: G query heads per KV head):
//     o = sum_t softmax_t(scale q . k_t) v_t,
// k_t, v_t the codepoints stored for token t (Key formulas (3)).
//
// Cache: the plan's two tensors are K (tensor 0) and V (tensor 1), blocks of
// 32 tokens x 128 features (one head); the block of (outer o, head h, chunk
// c) is ((o H + h) C + c) in tensor 0 and the same index plus the K block
// count in tensor 1.
//
// Kernel 1: a workgroup takes (o, h, split of 16 chunks).  Thread (slot j,
// feature group f) owns tokens j and j + 16 of every chunk and features
// 8f..8f+7; it decodes its 8 K and 8 V entries per token, finishes the G dot
// products with its 15 partners by DPP row sums, and keeps a running
// maximum, sum of weights and weighted V sum (online softmax) per query
// head.  The 16 token slots are merged by log-sum-exp (shuffles inside a
// wave, LDS across the 4 waves) into one partial per query head and split.
// Kernel 2 merges the splits and divides.
#include <math.h>

#include "kvq_internal.h"

namespace kvq {

namespace {

constexpr int kAT2 = 256;                 // threads per workgroup
constexpr int kChunkSplit = 16;           // chunks (32-token blocks) per workgroup
constexpr int kHD = 128;                  // head dim
constexpr int kTB = 32;                   // tokens per block

// The 8 codes of width w >= 1 of entries 8u .. 8u + 7 of a block's code
// stream of nwords >= 1 words sit in words q = (w u) / 4 and q + 1, shifted
// by sh = 8 ((w u) mod 4) bits (8 w <= 32 bits, so one funnel shift gathers
// them).  The second word is needed only when the group straddles a word
// boundary, which never happens in the block's last word, so its index is
// clamped into the stream and both loads are issued unconditionally.  The
// words are kept apart from the shift so that a load is waited on only where
// its codes are used.
struct CodeWords {
    uint32_t a, b;
};

// (w u < 2^24: a 24-bit multiply suffices)
__device__ __forceinline__ CodeWords load_codes8(const uint32_t* cw, uint32_t nwords, int w, int u) {
    const uint32_t q = __umul24((uint32_t)w, (uint32_t)u) >> 2;
    return {cw[q], cw[min(q + 1, nwords - 1)]};
}

__device__ __forceinline__ uint32_t codes8(CodeWords x, int w, int u) {
    const uint32_t sh = 8u * (__umul24((uint32_t)w, (uint32_t)u) & 3u);
    return (uint32_t)((((uint64_t)x.b << 32) | x.a) >> sh);
}

// Field [off, off + w) of x.
__device__ __forceinline__ uint32_t field(uint32_t x, uint32_t off, uint32_t w) {
    return __builtin_amdgcn_ubfe(x, off, w);
}

// Sum over a 16-lane row, the same bits in every lane: partner swaps inside
// quads (lane ^ 1, lane ^ 2), then the half-row mirror (quad q <-> 1 - q)
// and the row mirror (half h <-> 1 - h); each step adds a value to its
// mirror image, so both partners round identically.  DPP moves, no LDS.
constexpr int kDppQuadXor1 = 0xB1;       // quad_perm [1, 0, 3, 2]
constexpr int kDppQuadXor2 = 0x4E;       // quad_perm [2, 3, 0, 1]
constexpr int kDppRowHalfMirror = 0x141;
constexpr int kDppRowMirror = 0x140;

// Every source lane of these patterns lies in the row, so bound_ctrl never
// takes effect; it lets the move fold into the add (v_add_f32_dpp).
template <int kCtrl>
__device__ __forceinline__ float dpp_f32(float v) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), kCtrl, 0xF, 0xF, true));
}

__device__ __forceinline__ float xor_sum16(float v) {
    v = dpp_f32<kDppQuadXor1>(v) + v;
    v = dpp_f32<kDppQuadXor2>(v) + v;
    v = dpp_f32<kDppRowHalfMirror>(v) + v;
    v = dpp_f32<kDppRowMirror>(v) + v;
    return v;
}

// 2^x on the transcendental unit (scores live in base-2 units: q is
// pre-scaled by log2 e, so 2^(s - m) is the softmax weight e^(s' - m')).
__device__ __forceinline__ float pow2(float x) { return __builtin_amdgcn_exp2f(x); }

constexpr float kLog2e = 1.4426950408889634f;

}  // namespace

template <int G>
__global__ void __launch_bounds__(kAT2)
attn_split_kernel(const uint32_t* __restrict__ codes, const float* __restrict__ codebook,
                  const uint8_t* __restrict__ m_in, const uint64_t* __restrict__ word_off,
                  int64_t nbK, int heads, int chunks, int s, const float* __restrict__ q,
                  float scale, float* __restrict__ part, int splits, int gtot, int goff) {
    __shared__ float cb[2][kChunkSplit][kMaxS];
    __shared__ int wdt[2][kChunkSplit];
    __shared__ uint64_t wof[2][kChunkSplit];
    __shared__ uint32_t nwd[2][kChunkSplit];
    __shared__ float xm[4][G], xl[4][G];
    __shared__ float xa[4][G][kHD];
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int j = tid >> 4, f = tid & 15;
    const int sp = blockIdx.x, h = blockIdx.y, o = blockIdx.z;
    const int c0 = sp * kChunkSplit, c1 = min(c0 + kChunkSplit, chunks);
    const int64_t rbase = ((int64_t)o * heads + h) * chunks;
    // codebooks, widths and offsets of the split's K and V blocks
    for (int e = tid; e < 2 * kChunkSplit * kMaxS; e += kAT2) {
        const int t = e / (kChunkSplit * kMaxS), rem = e % (kChunkSplit * kMaxS);
        const int c = rem / kMaxS, k = rem % kMaxS;
        if (c0 + c < c1) {
            const int64_t r = rbase + c0 + c + (t ? nbK : 0);
            const int mm = min(max((int)m_in[r], 1), s);
            cb[t][c][k] = k < mm ? codebook[r * s + k] : 0.0f;
            if (k == 0) {
                wdt[t][c] = code_width(mm);
                wof[t][c] = word_off[r];
                nwd[t][c] = (uint32_t)(word_off[r + 1] - word_off[r]);
            }
        }
    }
    float qv[G][8];
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
        for (int i = 0; i < 8; ++i)
            qv[g][i] = (scale * kLog2e) * q[((int64_t)o * heads * gtot + h * gtot + goff + g) * kHD + 8 * f + i];
    __syncthreads();
    float mx[G], sl[G], acc[G][8];
#pragma unroll
    for (int g = 0; g < G; ++g) {
        mx[g] = -__builtin_huge_valf();
        sl[g] = 0.0f;
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[g][i] = 0.0f;
    }
    // Per chunk: the K codes of tokens j and j + 16 give two partial scores
    // per query head, summed over the row's 16 feature groups; one maximum
    // update covers both tokens; then the V codes are weighted in.  The next
    // chunk's codes are loaded before this chunk's work, hiding their latency.
    const int nc = c1 - c0;
    const int ug[2] = {16 * j + f, 16 * (j + 16) + f};  // 8-entry groups of tokens j, j + 16
    CodeWords kn[2] = {}, vn[2] = {};
    auto load = [&](int c, CodeWords (&kw)[2], CodeWords (&vw)[2]) {
        const int wk = __builtin_amdgcn_readfirstlane(wdt[0][c]);
        const int wv = __builtin_amdgcn_readfirstlane(wdt[1][c]);
        if (wk) {
            const uint32_t* cw = codes + wof[0][c];
#pragma unroll
            for (int t = 0; t < 2; ++t) kw[t] = load_codes8(cw, nwd[0][c], wk, ug[t]);
        }
        if (wv) {
            const uint32_t* cw = codes + wof[1][c];
#pragma unroll
            for (int t = 0; t < 2; ++t) vw[t] = load_codes8(cw, nwd[1][c], wv, ug[t]);
        }
    };
    if (nc > 0) load(0, kn, vn);
    for (int c = 0; c < nc; ++c) {
        const uint32_t wk = (uint32_t)__builtin_amdgcn_readfirstlane(wdt[0][c]);
        const uint32_t wv = (uint32_t)__builtin_amdgcn_readfirstlane(wdt[1][c]);
        // this chunk's codes from the words loaded one iteration ago (width 0,
        // a one-point codebook, leaves them unread; field() of width 0 is 0
        // whatever they hold), then the next chunk's loads into the same
        // registers
        const uint32_t kc[2] = {codes8(kn[0], wk, ug[0]), codes8(kn[1], wk, ug[1])};
        const uint32_t vc[2] = {codes8(vn[0], wv, ug[0]), codes8(vn[1], wv, ug[1])};
        if (c + 1 < nc) load(c + 1, kn, vn);
        float sc[2][G];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
#pragma unroll
            for (int g = 0; g < G; ++g) sc[t][g] = 0.0f;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const float kv = cb[0][c][field(kc[t], wk * i, wk)];
#pragma unroll
                for (int g = 0; g < G; ++g) sc[t][g] = fmaf(qv[g][i], kv, sc[t][g]);
            }
#pragma unroll
            for (int g = 0; g < G; ++g) sc[t][g] = xor_sum16(sc[t][g]);
        }
#pragma unroll
        for (int g = 0; g < G; ++g) {
            const float mn = fmaxf(mx[g], fmaxf(sc[0][g], sc[1][g]));
            if (mn > mx[g]) {  // new maximum: rescale the running sums
                const float corr = pow2(mx[g] - mn);
                mx[g] = mn;
                sl[g] *= corr;
#pragma unroll
                for (int i = 0; i < 8; ++i) acc[g][i] *= corr;
            }
            sc[0][g] = pow2(sc[0][g] - mx[g]);
            sc[1][g] = pow2(sc[1][g] - mx[g]);
            sl[g] += sc[0][g] + sc[1][g];
        }
#pragma unroll
        for (int t = 0; t < 2; ++t) {
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const float vv = cb[1][c][field(vc[t], wv * i, wv)];
#pragma unroll
                for (int g = 0; g < G; ++g) acc[g][i] = fmaf(sc[t][g], vv, acc[g][i]);
            }
        }
    }
    // merge the 4 token slots of the wave (lanes 16j' + f share f)
#pragma unroll
    for (int g = 0; g < G; ++g) {
        float M = mx[g];
        M = fmaxf(M, __shfl_xor(M, 16, 64));
        M = fmaxf(M, __shfl_xor(M, 32, 64));
        const float e = mx[g] == -__builtin_huge_valf() ? 0.0f : pow2(mx[g] - M);
        float L = sl[g] * e;
        L += __shfl_xor(L, 16, 64);
        L += __shfl_xor(L, 32, 64);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            float a = acc[g][i] * e;
            a += __shfl_xor(a, 16, 64);
            a += __shfl_xor(a, 32, 64);
            acc[g][i] = a;
        }
        if (lane == 0) {
            xm[wave][g] = M;
            xl[wave][g] = L;
        }
        if (lane < 16) {
#pragma unroll
            for (int i = 0; i < 8; ++i) xa[wave][g][8 * f + i] = acc[g][i];
        }
    }
    __syncthreads();
    // merge the 4 waves: thread -> (query head g, feature d)
    for (int e = tid; e < G * kHD; e += kAT2) {
        const int g = e / kHD, d = e % kHD;
        float M = xm[0][g];
#pragma unroll
        for (int w = 1; w < 4; ++w) M = fmaxf(M, xm[w][g]);
        float L = 0.0f, A = 0.0f;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            const float e2 = xm[w][g] == -__builtin_huge_valf() ? 0.0f : pow2(xm[w][g] - M);
            L = fmaf(xl[w][g], e2, L);
            A = fmaf(xa[w][g][d], e2, A);
        }
        // partial layout: [o][query head h * gtot + goff + g][split][kHD + 2]
        // = (A..., M, L), M in base-2 units
        float* pp = part + (((int64_t)o * heads * gtot + h * gtot + goff + g) * splits + sp) * (kHD + 2);
        pp[d] = A;
        if (d == 0) {
            pp[kHD] = M;
            pp[kHD + 1] = L;
        }
    }
}

__global__ void __launch_bounds__(kHD)
attn_merge_kernel(const float* __restrict__ part, int splits, float* __restrict__ out) {
    const int64_t row = blockIdx.x;  // (o, query head)
    const int d = threadIdx.x;
    const float* pp = part + row * splits * (kHD + 2);
    // unrolled so that several splits' loads are in flight at once
    float M = -__builtin_huge_valf();
#pragma unroll 8
    for (int sp = 0; sp < splits; ++sp) M = fmaxf(M, pp[sp * (kHD + 2) + kHD]);
    float L = 0.0f, A = 0.0f;
#pragma unroll 8
    for (int sp = 0; sp < splits; ++sp) {
        const float m = pp[sp * (kHD + 2) + kHD];
        const float e = m == -__builtin_huge_valf() ? 0.0f : pow2(m - M);
        L = fmaf(pp[sp * (kHD + 2) + kHD + 1], e, L);
        A = fmaf(pp[sp * (kHD + 2) + d], e, A);
    }
    out[row * kHD + d] = A / L;
}

uint64_t attn_workspace_bytes(int64_t outer, int heads, int chunks, int group) {
    const int64_t splits = (chunks + kChunkSplit - 1) / kChunkSplit;
    return (uint64_t)outer * heads * group * splits * (kHD + 2) * sizeof(float);
}

hipError_t launch_decode_attention(const uint32_t* codes, const float* codebook, const uint8_t* m,
                                   const uint64_t* word_off, int64_t nbK, int64_t outer, int heads,
                                   int chunks, int s, int group, const float* q, float scale,
                                   float* out, void* work, hipStream_t st) {
    if (outer == 0 || heads == 0 || chunks == 0) return hipSuccess;
    const int splits = (chunks + kChunkSplit - 1) / kChunkSplit;
    const dim3 grid((unsigned)splits, (unsigned)heads, (unsigned)outer);
    float* part = (float*)work;
    // a group of any size runs as launches over 4, 2 and 1 of its query
    // heads (each reads the codes once); 4 is the most that the registers
    // hold at full occupancy
    if (group < 1) return hipErrorInvalidValue;
    for (int goff = 0; goff < group;) {
        const int left = group - goff;
        if (left >= 4) {
            hipLaunchKernelGGL(attn_split_kernel<4>, grid, dim3(kAT2), 0, st, codes, codebook, m, word_off,
                               nbK, heads, chunks, s, q, scale, part, splits, group, goff);
            goff += 4;
        } else if (left >= 2) {
            hipLaunchKernelGGL(attn_split_kernel<2>, grid, dim3(kAT2), 0, st, codes, codebook, m, word_off,
                               nbK, heads, chunks, s, q, scale, part, splits, group, goff);
            goff += 2;
        } else {
            hipLaunchKernelGGL(attn_split_kernel<1>, grid, dim3(kAT2), 0, st, codes, codebook, m, word_off,
                               nbK, heads, chunks, s, q, scale, part, splits, group, goff);
            goff += 1;
        }
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(attn_merge_kernel, dim3((unsigned)(outer * heads * group)), dim3(kHD), 0, st,
                       part, splits, out);
    return hipGetLastError();
}

}  // namespace kvq
