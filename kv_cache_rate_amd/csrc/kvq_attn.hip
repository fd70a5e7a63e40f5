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

// The 8 codes of width w of entries 8u .. 8u + 7 of a block's code stream
// (8 w <= 32 bits, so one funnel shift gathers them).
__device__ __forceinline__ uint32_t codes8(const uint32_t* cw, uint32_t nwords, int w, int u) {
    if (w == 0) return 0u;
    const uint32_t byte = (uint32_t)w * (uint32_t)u;  // w bytes per 8 codes
    const uint32_t q = byte >> 2, sh = 8u * (byte & 3u);
    const uint32_t a = cw[q];
    const uint32_t b = (sh + 8u * (uint32_t)w > 32u && q + 1 < nwords) ? cw[q + 1] : 0u;
    return (uint32_t)((((uint64_t)b << 32) | a) >> sh);
}

// Sum over a 16-lane row, the same bits in every lane: partner swaps inside
// quads (lane ^ 1, lane ^ 2), then the half-row mirror (quad q <-> 1 - q)
// and the row mirror (half h <-> 1 - h); each step adds a value to its
// mirror image, so both partners round identically.  DPP moves, no LDS.
constexpr int kDppQuadXor1 = 0xB1;       // quad_perm [1, 0, 3, 2]
constexpr int kDppQuadXor2 = 0x4E;       // quad_perm [2, 3, 0, 1]
constexpr int kDppRowHalfMirror = 0x141;
constexpr int kDppRowMirror = 0x140;

template <int kCtrl>
__device__ __forceinline__ float dpp_f32(float v) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), kCtrl, 0xF, 0xF, false));
}

__device__ __forceinline__ float xor_sum16(float v) {
    v += dpp_f32<kDppQuadXor1>(v);
    v += dpp_f32<kDppQuadXor2>(v);
    v += dpp_f32<kDppRowHalfMirror>(v);
    v += dpp_f32<kDppRowMirror>(v);
    return v;
}

}  // namespace

template <int G>
__global__ void __launch_bounds__(kAT2)
attn_split_kernel(const uint32_t* __restrict__ codes, const float* __restrict__ codebook,
                  const uint8_t* __restrict__ m_in, const uint64_t* __restrict__ word_off,
                  int64_t nbK, int heads, int chunks, int s, const float* __restrict__ q,
                  float scale, float* __restrict__ part, int splits) {
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
            qv[g][i] = scale * q[((int64_t)o * heads * G + h * G + g) * kHD + 8 * f + i];
    __syncthreads();
    float mx[G], sl[G], acc[G][8];
#pragma unroll
    for (int g = 0; g < G; ++g) {
        mx[g] = -__builtin_huge_valf();
        sl[g] = 0.0f;
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[g][i] = 0.0f;
    }
    for (int c = 0; c < c1 - c0; ++c) {
        const int wk = wdt[0][c], wv = wdt[1][c];
        const uint32_t mk = (1u << wk) - 1u, mv = (1u << wv) - 1u;
#pragma unroll
        for (int half = 0; half < 2; ++half) {
            const int u = 16 * (j + 16 * half) + f;  // 8-entry group of token j + 16 half
            const uint32_t kc = codes8(codes + wof[0][c], nwd[0][c], wk, u);
            float sc[G];
#pragma unroll
            for (int g = 0; g < G; ++g) sc[g] = 0.0f;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const float kv = cb[0][c][(kc >> (wk * i)) & mk];
#pragma unroll
                for (int g = 0; g < G; ++g) sc[g] = fmaf(qv[g][i], kv, sc[g]);
            }
#pragma unroll
            for (int g = 0; g < G; ++g) {
                const float sg = xor_sum16(sc[g]);
                if (sg > mx[g]) {  // new maximum: rescale the running sums
                    const float corr = __expf(mx[g] - sg);
                    mx[g] = sg;
                    sl[g] *= corr;
#pragma unroll
                    for (int i = 0; i < 8; ++i) acc[g][i] *= corr;
                }
                sc[g] = __expf(sg - mx[g]);
                sl[g] += sc[g];
            }
            const uint32_t vc = codes8(codes + wof[1][c], nwd[1][c], wv, u);
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const float vv = cb[1][c][(vc >> (wv * i)) & mv];
#pragma unroll
                for (int g = 0; g < G; ++g) acc[g][i] = fmaf(sc[g], vv, acc[g][i]);
            }
        }
    }
    // merge the 4 token slots of the wave (lanes 16j' + f share f)
#pragma unroll
    for (int g = 0; g < G; ++g) {
        float M = mx[g];
        M = fmaxf(M, __shfl_xor(M, 16, 64));
        M = fmaxf(M, __shfl_xor(M, 32, 64));
        const float e = mx[g] == -__builtin_huge_valf() ? 0.0f : __expf(mx[g] - M);
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
            const float e2 = xm[w][g] == -__builtin_huge_valf() ? 0.0f : __expf(xm[w][g] - M);
            L = fmaf(xl[w][g], e2, L);
            A = fmaf(xa[w][g][d], e2, A);
        }
        // partial layout: [o][head h * G + g][split][kHD + 2] = (A..., M, L)
        float* pp = part + (((int64_t)o * heads * G + h * G + g) * splits + sp) * (kHD + 2);
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
    float M = -__builtin_huge_valf();
    for (int sp = 0; sp < splits; ++sp) M = fmaxf(M, pp[sp * (kHD + 2) + kHD]);
    float L = 0.0f, A = 0.0f;
    for (int sp = 0; sp < splits; ++sp) {
        const float m = pp[sp * (kHD + 2) + kHD];
        const float e = m == -__builtin_huge_valf() ? 0.0f : __expf(m - M);
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
    switch (group) {
    case 1:
        hipLaunchKernelGGL(attn_split_kernel<1>, grid, dim3(kAT2), 0, st, codes, codebook, m, word_off,
                           nbK, heads, chunks, s, q, scale, part, splits);
        break;
    case 2:
        hipLaunchKernelGGL(attn_split_kernel<2>, grid, dim3(kAT2), 0, st, codes, codebook, m, word_off,
                           nbK, heads, chunks, s, q, scale, part, splits);
        break;
    case 4:
        hipLaunchKernelGGL(attn_split_kernel<4>, grid, dim3(kAT2), 0, st, codes, codebook, m, word_off,
                           nbK, heads, chunks, s, q, scale, part, splits);
        break;
    default:
        return hipErrorInvalidValue;
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(attn_merge_kernel, dim3((unsigned)(outer * heads * group)), dim3(kHD), 0, st,
                       part, splits, out);
    return hipGetLastError();
}

}  // namespace kvq
