// Decode attention over the quantized cache, decoding K and V in registers
// and contracting on the matrix cores.
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
// A workgroup takes (o, h, a split of up to 32 chunks) and up to 4 query
// heads of the group; each of its 4 waves takes every fourth chunk of the
// split and keeps its own online softmax (running maximum, sum of weights,
// weighted V sum per query head).  Per chunk, both products are fp32
// 4x4x1 matrix-core operations over 16 blocks of the wave:
// * scores: block b = 8 hf + tq covers tokens 4 tq .. 4 tq + 3 and the
//   feature half hf; step f (64 steps) multiplies the 4 query heads' q_f
//   (one register per 8 steps, broadcast to each half's 8 blocks) into the
//   decoded k_{t, 64 hf + f} of lane 32 hf + t, so lane l ends with the 4
//   heads' partial scores of token l & 31, and one exchange adds the halves;
// * values: the weights are transposed inside each 4-lane group so that
//   lanes 4q .. 4q + 3 hold the 4 heads' weights of one token; step t (32
//   steps) broadcasts them to all blocks and multiplies them into v_{t, 2l}
//   and v_{t, 2l + 1}, decoded by lane l, into two accumulators.
// Each lane decodes its K codes from registers (its token's 64-feature half
// row is 2 w contiguous words) and its V codes from the chunk's V stream
// staged in the wave's LDS; codepoints come from the chunk's codebooks in
// LDS, two at a time from a table of codepoint pairs for 4-bit codes.  A
// wave's running maximum may trail its scores by a fixed slack, so the sums
// are rescaled on few chunks.  The waves' partials are merged by
// log-sum-exp in LDS into one partial per query head and split; a second
// kernel merges the splits.
#include <math.h>

#include <utility>

#include "kvq_internal.h"

namespace kvq {

namespace {

constexpr int kAT = 256;                      // threads per workgroup
constexpr int kAW = kAT / 64;                 // waves per workgroup
constexpr int kChunksPerWave = 8;
constexpr int kChunkSplit = kAW * kChunksPerWave;  // chunks (32-token blocks) per workgroup
constexpr int kHD = 128;                      // head dim
constexpr int kHeadsPerPass = 4;              // query heads per launch (the matrix rows)
constexpr int kStageWords = 4 * kHD;          // a chunk's V stream at w = 4 bits

typedef float v4f __attribute__((ext_vector_type(4)));

template <int... I, class F>
__device__ __forceinline__ void static_for_impl(std::integer_sequence<int, I...>, F&& f) {
    (f(std::integral_constant<int, I>{}), ...);
}
template <int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
    static_for_impl(std::make_integer_sequence<int, N>{}, f);
}

// 2^x on the transcendental unit (scores live in base-2 units: q is
// pre-scaled by log2 e, so 2^(s - m) is the softmax weight e^(s' - m')).
__device__ __forceinline__ float pow2(float x) { return __builtin_amdgcn_exp2f(x); }

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kDppQuadXor1 = 0xB1;  // quad_perm [1, 0, 3, 2]
constexpr int kDppQuadXor2 = 0x4E;  // quad_perm [2, 3, 0, 1]
// A running maximum may trail the scores by up to this much (base-2 units):
// the weights then stay at most 2^16, and the sums are rescaled only when a
// score passes it, which after a wave's first chunk is rare.
constexpr float kSlack = 16.0f;

template <int CTRL, int RM = 0xF>
__device__ __forceinline__ float dpp_max(float v) {
    return fmaxf(v, __uint_as_float(dpp_u32<CTRL, RM>(__float_as_uint(v), __float_as_uint(v))));
}
// Maximum over the wave, wave-uniform.
__device__ __forceinline__ float wave_max_f32(float v) {
    v = dpp_max<kDppRowShr1>(v);
    v = dpp_max<kDppRowShr2>(v);
    v = dpp_max<kDppRowShr4>(v);
    v = dpp_max<kDppRowShr8>(v);
    v = dpp_max<kDppBcast15, 0xA>(v);
    v = dpp_max<kDppBcast31, 0xC>(v);
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

template <int kCtrl>
__device__ __forceinline__ float quad_swap(float v) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), kCtrl, 0xF, 0xF, false));
}

// 4x4 transpose inside every 4-lane group: lane j of the group, register i
// -> lane i, register j (two butterfly stages, lane bit 0 then bit 1).
__device__ __forceinline__ void quad_transpose(float (&r)[4], int lane) {
    const bool b0 = (lane & 1) != 0, b1 = (lane & 2) != 0;
    {
        const float t0 = quad_swap<kDppQuadXor1>(r[0]), t1 = quad_swap<kDppQuadXor1>(r[1]);
        const float t2 = quad_swap<kDppQuadXor1>(r[2]), t3 = quad_swap<kDppQuadXor1>(r[3]);
        r[0] = b0 ? t1 : r[0];
        r[1] = b0 ? r[1] : t0;
        r[2] = b0 ? t3 : r[2];
        r[3] = b0 ? r[3] : t2;
    }
    {
        const float t0 = quad_swap<kDppQuadXor2>(r[0]), t1 = quad_swap<kDppQuadXor2>(r[1]);
        const float t2 = quad_swap<kDppQuadXor2>(r[2]), t3 = quad_swap<kDppQuadXor2>(r[3]);
        r[0] = b1 ? t2 : r[0];
        r[2] = b1 ? r[2] : t0;
        r[1] = b1 ? t3 : r[1];
        r[3] = b1 ? r[3] : t1;
    }
}

// LDS byte addresses: a codebook row is 64-byte aligned, so a codepoint's
// address is the row's address OR 4 x its code.
typedef __attribute__((address_space(3))) const float lds_cf;
__device__ __forceinline__ uint32_t lds_addr(const float* p) { return (uint32_t)(uintptr_t)(lds_cf*)p; }
__device__ __forceinline__ float lds_at(uint32_t a) { return *(lds_cf*)(uintptr_t)a; }

// Partial scores of the lane's token over its feature half for a chunk of
// K code width W: 64 steps, two accumulator chains (even and odd steps).
// kw: the 2 W code words of the lane's half row; cb: the chunk's K
// codebook in LDS.
template <int W>
__device__ __forceinline__ v4f k_scores(const uint32_t (&kw)[8], const float (&qreg)[8], const float* cb) {
    v4f d0 = {0.0f, 0.0f, 0.0f, 0.0f}, d1 = d0;
    const float k0 = cb[0];
    const uint32_t base = lds_addr(cb);
    static_for<64>([&](auto S) {
        constexpr int s = decltype(S)::value;
        float kv = k0;  // width 0: a one-point codebook
        if constexpr (W > 0) {
            constexpr int bit = W * s, q = bit >> 5, off = bit & 31;
            uint32_t code;
            if constexpr (off + W <= 32)
                code = __builtin_amdgcn_ubfe(kw[q], off, W);
            else
                code = __builtin_amdgcn_ubfe(__builtin_amdgcn_alignbit(kw[q + 1], kw[q], off), 0, W);
            kv = lds_at(base | (code << 2));
        }
        if constexpr ((s & 1) == 0)
            d0 = __builtin_amdgcn_mfma_f32_4x4x1f32(qreg[s >> 3], kv, d0, 3, s & 7, 0);
        else
            d1 = __builtin_amdgcn_mfma_f32_4x4x1f32(qreg[s >> 3], kv, d1, 3, s & 7, 0);
    });
    return d0 + d1;
}

// Weighted V sums of a chunk of V code width W: 32 token steps.  row: the
// lane's first stream word of row 0 in the wave's staging buffer (row t at
// + 4 W t words); sh0, sh1: bit offsets of the lane's two fields in it.
template <int W>
__device__ __forceinline__ void v_accum(const uint32_t* row, uint32_t sh0, uint32_t sh1, const float* cb,
                                        const float (&pt)[4], v4f& a0, v4f& a1) {
    const float c0 = cb[0];
    const uint32_t base = lds_addr(cb);
    static_for<32>([&](auto T) {
        constexpr int t = decltype(T)::value;
        float v0 = c0, v1 = c0;  // width 0: a one-point codebook
        if constexpr (W > 0) {
            uint32_t x;
            if constexpr (W == 3)  // a 6-bit field may straddle two words
                x = __builtin_amdgcn_alignbit(row[4 * W * t + 1], row[4 * W * t], sh0);
            else
                x = row[4 * W * t];
            v0 = lds_at(base | (__builtin_amdgcn_ubfe(x, W == 3 ? 0u : sh0, W) << 2));
            v1 = lds_at(base | (__builtin_amdgcn_ubfe(x, W == 3 ? (uint32_t)W : sh1, W) << 2));
        }
        a0 = __builtin_amdgcn_mfma_f32_4x4x1f32(pt[t & 3], v0, a0, 4, t >> 2, 0);
        a1 = __builtin_amdgcn_mfma_f32_4x4x1f32(pt[t & 3], v1, a1, 4, t >> 2, 0);
    });
}

// 4-bit codes (widths 3 and 4 cover most blocks; 4 where the budget does
// not bind): a byte holds two codes, so a 256-entry table of codepoint pairs
// per chunk, entry y = (cb[y & 15], cb[y >> 4]), decodes two entries with
// one LDS read.  Each lane writes 4 entries.
typedef float f2v __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) const f2v lds_cf2;
__device__ __forceinline__ f2v lds_at2(uint32_t a) { return *(lds_cf2*)(uintptr_t)a; }

__device__ __forceinline__ void build_pairs(float2* tab, const float* cb, int lane) {
    const float lo = cb[lane & 15];
#pragma unroll
    for (int j = 0; j < 4; ++j) tab[lane + 64 * j] = make_float2(lo, cb[(lane >> 4) + 4 * j]);
}

// k_scores<4> through the pair table (tbase: its LDS address, 2 KB aligned):
// byte j of the half row holds features 2 j and 2 j + 1.
__device__ __forceinline__ v4f k_scores_pairs(const uint32_t (&kw)[8], const float (&qreg)[8], uint32_t tbase) {
    v4f d0 = {0.0f, 0.0f, 0.0f, 0.0f}, d1 = d0;
    static_for<32>([&](auto J) {
        constexpr int j = decltype(J)::value;
        const uint32_t y = __builtin_amdgcn_ubfe(kw[j >> 2], 8 * (j & 3), 8);
        const f2v kv = lds_at2(tbase | (y << 3));
        d0 = __builtin_amdgcn_mfma_f32_4x4x1f32(qreg[(2 * j) >> 3], kv.x, d0, 3, (2 * j) & 7, 0);
        d1 = __builtin_amdgcn_mfma_f32_4x4x1f32(qreg[(2 * j + 1) >> 3], kv.y, d1, 3, (2 * j + 1) & 7, 0);
    });
    return d0 + d1;
}

// v_accum<4> through the pair table: the lane's two codes of row t are byte
// lane of the row (rowb: the staged stream's bytes, offset by lane).
__device__ __forceinline__ void v_accum_pairs(const uint8_t* rowb, uint32_t tbase, const float (&pt)[4], v4f& a0,
                                              v4f& a1) {
    static_for<32>([&](auto T) {
        constexpr int t = decltype(T)::value;
        const uint32_t y = rowb[64 * t];
        const f2v v = lds_at2(tbase | (y << 3));
        a0 = __builtin_amdgcn_mfma_f32_4x4x1f32(pt[t & 3], v.x, a0, 4, t >> 2, 0);
        a1 = __builtin_amdgcn_mfma_f32_4x4x1f32(pt[t & 3], v.y, a1, 4, t >> 2, 0);
    });
}

// Words [2 w lane_part, 2 w lane_part + 2 w) of a stream (w <= 4).
__device__ __forceinline__ void load_words(const uint32_t* p, int w, uint32_t (&x)[8]) {
#pragma unroll
    for (int i = 0; i < 8; ++i)
        if (i < 2 * w) x[i] = p[i];
}

}  // namespace

// (5 waves per SIMD: the chains of LDS reads and matrix steps are latency-
// bound, so occupancy pays more than registers)
__global__ void __launch_bounds__(kAT, 5)
attn_split_kernel(const uint32_t* __restrict__ codes, const float* __restrict__ codebook,
                  const uint8_t* __restrict__ m_in, const uint64_t* __restrict__ word_off,
                  int64_t nbK, int heads, int chunks, int s, const float* __restrict__ q,
                  float scale, float* __restrict__ part, int splits, int gtot, int goff, int gcount) {
    __shared__ alignas(64) float cb[2][kChunkSplit][kMaxS];  // 64-byte rows: base | 4 code
    __shared__ int wdt[2][kChunkSplit];
    __shared__ uint64_t wof[2][kChunkSplit];
    __shared__ float xm[kAW][kHeadsPerPass], xl[kAW][kHeadsPerPass];
    __shared__ alignas(2048) float2 pairs[kAW][2][256];  // per wave: K and V pair tables
    __shared__ union {
        uint32_t st[kAW][kStageWords];            // per wave: the current chunk's V stream
        float xa[kAW][kHeadsPerPass][kHD];        // per wave: weighted V sums, for the merge
    } buf;
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int sp = blockIdx.x, h = blockIdx.y, o = blockIdx.z;
    const int c0 = sp * kChunkSplit, c1 = min(c0 + kChunkSplit, chunks);
    const int64_t rbase = ((int64_t)o * heads + h) * chunks;
    // codebooks, widths and word offsets of the split's K and V blocks, and
    // the query registers (lane 32 hf + 4 k + i holds, in register g8, head
    // i's q at feature 64 hf + 8 g8 + k, scaled into base-2 units; heads past
    // gcount are zero).  Every load is issued first, unconditionally (block
    // and entry indices clamped into their arrays), and selected afterwards:
    // loads under conditions were each waited on in turn, a dozen memory
    // round trips before the first chunk.
    constexpr int kSetup = 2 * kChunkSplit * kMaxS / kAT;  // table entries per thread
    static_assert(kSetup * kAT == 2 * kChunkSplit * kMaxS, "whole rounds");
    uint8_t mv[kSetup];
    float cv[kSetup];
    uint64_t ov[kSetup];
#pragma unroll
    for (int u = 0; u < kSetup; ++u) {
        const int e = tid + u * kAT;
        const int t = e / (kChunkSplit * kMaxS), rem = e % (kChunkSplit * kMaxS);
        const int c = rem / kMaxS, k = rem % kMaxS;
        const int64_t r = rbase + min(c0 + c, c1 - 1) + (t ? nbK : 0);
        mv[u] = m_in[r];
        cv[u] = codebook[r * s + min(k, s - 1)];
        ov[u] = word_off[r];
    }
    const int hf = lane >> 5, hi = lane & 3, kq = (lane >> 2) & 7;
    float qv[8];
    {
        const float* qp = q + ((int64_t)o * heads * gtot + (int64_t)h * gtot + goff + min(hi, gcount - 1)) * kHD +
                          64 * hf + kq;
#pragma unroll
        for (int g8 = 0; g8 < 8; ++g8) qv[g8] = qp[8 * g8];
    }
#pragma unroll
    for (int u = 0; u < kSetup; ++u) {
        const int e = tid + u * kAT;
        const int t = e / (kChunkSplit * kMaxS), rem = e % (kChunkSplit * kMaxS);
        const int c = rem / kMaxS, k = rem % kMaxS;
        if (c0 + c < c1) {
            const int mm = min(max((int)mv[u], 1), s);
            cb[t][c][k] = k < mm ? cv[u] : 0.0f;
            if (k == 0) {
                wdt[t][c] = code_width(mm);
                wof[t][c] = ov[u];
            }
        }
    }
    float qreg[8];
    {
        const float c = scale * kLog2e;
#pragma unroll
        for (int g8 = 0; g8 < 8; ++g8) qreg[g8] = hi < gcount ? c * qv[g8] : 0.0f;
    }
    __syncthreads();

    float mrun[4], lsum[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        mrun[i] = -__builtin_huge_valf();
        lsum[i] = 0.0f;
    }
    v4f acc0 = {0.0f, 0.0f, 0.0f, 0.0f}, acc1 = acc0;
    // the lane's K words: token lane & 31, feature half hf of the chunk's
    // K stream, words [w (4 t + 2 hf), + 2 w); its V share of the staging
    // copy: words [2 w lane, + 2 w)
    const int tok = lane & 31;
    uint32_t kw[8] = {}, vw[8] = {}, kn[8] = {}, vn[8] = {};
    auto load = [&](int c, uint32_t (&kx)[8], uint32_t (&vx)[8]) {
        const int wk = __builtin_amdgcn_readfirstlane(wdt[0][c]);
        const int wv = __builtin_amdgcn_readfirstlane(wdt[1][c]);
        load_words(codes + wof[0][c] + wk * (4 * tok + 2 * hf), wk, kx);
        load_words(codes + wof[1][c] + 2 * wv * lane, wv, vx);
    };
    uint32_t* stage = buf.st[wave];
    int c = c0 + wave;
    if (c < c1) load(c - c0, kn, vn);
    for (; c < c1; c += kAW) {
        const int ci = c - c0;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            kw[i] = kn[i];
            vw[i] = vn[i];
        }
        if (c + kAW < c1) load(ci + kAW, kn, vn);
        const int wk = __builtin_amdgcn_readfirstlane(wdt[0][ci]);
        const int wv = __builtin_amdgcn_readfirstlane(wdt[1][ci]);
        // this chunk's V stream into the wave's staging buffer (the wave's
        // own earlier reads of it are ordered before these writes)
#pragma unroll
        for (int i = 0; i < 8; ++i)
            if (i < 2 * wv) stage[2 * wv * lane + i] = vw[i];
        // scores of token tok, both halves added (the two halves of the
        // wave then hold the same values)
        if (wk == 4 || wv == 4) {
            if (wk == 4) build_pairs(pairs[wave][0], cb[0][ci], lane);
            if (wv == 4) build_pairs(pairs[wave][1], cb[1][ci], lane);
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        }
        v4f d;
        switch (wk) {
            case 0: d = k_scores<0>(kw, qreg, cb[0][ci]); break;
            case 1: d = k_scores<1>(kw, qreg, cb[0][ci]); break;
            case 2: d = k_scores<2>(kw, qreg, cb[0][ci]); break;
            case 3: d = k_scores<3>(kw, qreg, cb[0][ci]); break;
            default: d = k_scores_pairs(kw, qreg, lds_addr(&pairs[wave][0][0].x)); break;
        }
        float sc[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) sc[i] = d[i] + __shfl_xor(d[i], 32, 64);
        // a score more than kSlack above its head's running maximum (every
        // score of a wave's first chunk): move every head's maximum up to
        // the chunk's and rescale the running sums
        bool rise = false;
#pragma unroll
        for (int i = 0; i < 4; ++i) rise |= sc[i] > mrun[i] + kSlack;
        if (__any(rise)) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float mx = wave_max_f32(sc[i]);
                const float mn = fmaxf(mrun[i], mx);
                const float corr = mrun[i] == -__builtin_huge_valf() ? 0.0f : pow2(mrun[i] - mn);
                mrun[i] = mn;
                lsum[i] *= corr;
                acc0[i] *= corr;
                acc1[i] *= corr;
            }
        }
        float pt[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            pt[i] = pow2(sc[i] - mrun[i]);
            lsum[i] += hf ? 0.0f : pt[i];  // each token counted once
        }
        quad_transpose(pt, lane);
        // the staged V stream is read by other lanes: keep the writes above
        // ahead of the reads (the wave's LDS operations complete in order)
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        {
            // the lane's V fields: features 2 lane, 2 lane + 1 of each row,
            // bits [2 w lane, 2 w lane + 2 w) of the row
            const uint32_t bit = 2u * (uint32_t)wv * (uint32_t)lane;
            const uint32_t* row = stage + (bit >> 5);
            const uint32_t sh0 = bit & 31u, sh1 = sh0 + (uint32_t)wv;
            switch (wv) {
                case 0: v_accum<0>(row, sh0, sh1, cb[1][ci], pt, acc0, acc1); break;
                case 1: v_accum<1>(row, sh0, sh1, cb[1][ci], pt, acc0, acc1); break;
                case 2: v_accum<2>(row, sh0, sh1, cb[1][ci], pt, acc0, acc1); break;
                case 3: v_accum<3>(row, sh0, sh1, cb[1][ci], pt, acc0, acc1); break;
                default:
                    v_accum_pairs(reinterpret_cast<const uint8_t*>(stage) + lane, lds_addr(&pairs[wave][1][0].x), pt,
                                  acc0, acc1);
                    break;
            }
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
    // the wave's totals: sums of weights over its lanes; weighted V sums of
    // head i at features 2 lane (acc0[i]) and 2 lane + 1 (acc1[i])
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        float L = lsum[i];
#pragma unroll
        for (int k = 1; k < 64; k <<= 1) L += __shfl_xor(L, k, 64);
        lsum[i] = L;
    }
    __syncthreads();  // every wave is done with its staging buffer
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        buf.xa[wave][i][2 * lane] = acc0[i];
        buf.xa[wave][i][2 * lane + 1] = acc1[i];
    }
    if (lane == 0) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            xm[wave][i] = mrun[i];
            xl[wave][i] = lsum[i];
        }
    }
    __syncthreads();
    // merge the waves: thread -> (query head g, feature d)
    for (int e = tid; e < gcount * kHD; e += kAT) {
        const int g = e / kHD, dd = e % kHD;
        float M = xm[0][g];
#pragma unroll
        for (int w = 1; w < kAW; ++w) M = fmaxf(M, xm[w][g]);
        float L = 0.0f, A = 0.0f;
#pragma unroll
        for (int w = 0; w < kAW; ++w) {
            const float e2 = xm[w][g] == -__builtin_huge_valf() ? 0.0f : pow2(xm[w][g] - M);
            L = fmaf(xl[w][g], e2, L);
            A = fmaf(buf.xa[w][g][dd], e2, A);
        }
        // partial layout: [o][query head h * gtot + goff + g][split][kHD + 2]
        // = (A..., M, L), M in base-2 units
        float* pp = part + (((int64_t)o * heads * gtot + h * gtot + goff + g) * splits + sp) * (kHD + 2);
        pp[dd] = A;
        if (dd == 0) {
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
    if (group < 1) return hipErrorInvalidValue;
    const int splits = (chunks + kChunkSplit - 1) / kChunkSplit;
    const dim3 grid((unsigned)splits, (unsigned)heads, (unsigned)outer);
    float* part = (float*)work;
    // a group of any size runs as launches over up to 4 of its query heads
    // (each reads the codes once)
    for (int goff = 0; goff < group; goff += kHeadsPerPass) {
        const int gcount = min(kHeadsPerPass, group - goff);
        hipLaunchKernelGGL(attn_split_kernel, grid, dim3(kAT), 0, st, codes, codebook, m, word_off, nbK, heads,
                           chunks, s, q, scale, part, splits, group, goff, gcount);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(attn_merge_kernel, dim3((unsigned)(outer * heads * group)), dim3(kHD), 0, st,
                       part, splits, out);
    return hipGetLastError();
}

}  // namespace kvq
