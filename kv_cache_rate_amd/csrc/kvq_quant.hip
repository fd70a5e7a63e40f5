// Stochastic interpolation + packing (kvq_quantize_pack) and decode
// (kvq_dequantize).
//
// Page "Rate-adaptive KV-cache quantizer", Key formulas (3): an entry x in
// [q_i, q_{i+1}] becomes q_{i+1} with probability p = (x - q_i)/(q_{i+1} - q_i)
// and q_i otherwise, so its conditional mean is x; Implementation notes: the
// codebook, the symbol stream and the block lengths are stored, and decoding
// happens before attention.
//
// Each thread owns 32 consecutive entries of a block, so with w-bit codes it
// writes exactly w whole 32-bit words (no code straddles two threads).  The
// draw of entry t of block r is word t & 3 of Philox4x32-10 on counter
// (t >> 2, r lo, r hi, 0) under key (seed lo, seed hi): one generator call
// serves four consecutive entries.
#include <stdlib.h>

#include "kvq_internal.h"
#include "kvq_quant_block.h"

namespace kvq {

constexpr int kQuantThreads = 128;  // 128 x 32 entries = 4096

__global__ void __launch_bounds__(kQuantThreads)
quantize_kernel(Geom g, int s, const float* __restrict__ codebook, const uint8_t* __restrict__ m_in,
                const uint64_t* __restrict__ off, uint32_t k0, uint32_t k1,
                uint32_t* __restrict__ codes) {
    __shared__ float q[kMaxS];
    const int64_t r = blockIdx.x;
    const int m = min(max((int)m_in[r], 1), s);
    if (threadIdx.x < s) q[threadIdx.x] = codebook[r * s + threadIdx.x];
    __syncthreads();
    const int w = code_width(m);
    const int n = g.n;
    const int t0 = threadIdx.x * 32;
    if (w == 0 || t0 >= n) return;
    const int cnt = min(32, n - t0);
    int ti;
    const int64_t base = block_base(g, r, ti);
    const uint32_t rlo = (uint32_t)r;
    const uint32_t rhi = (uint32_t)((uint64_t)r >> 32);
    uint64_t acc = 0;
    int nb = 0;
    uint64_t wi = off[r] + (uint64_t)threadIdx.x * (uint64_t)w;
    // the thread's entries, every load first and unconditional (positions
    // past its last entry re-read that entry, unused): loads under the
    // position test were waited on one by one
    float xs[32];
    {
        int64_t ofs[32];
#pragma unroll
        for (int e = 0; e < 32; ++e) ofs[e] = base + entry_off(g, ti, t0 + min(e, cnt - 1));
        if (g.dtype == KVQ_F16) {
            const __half* src = reinterpret_cast<const __half*>(g.data[ti]);
#pragma unroll
            for (int e = 0; e < 32; ++e) xs[e] = __half2float(src[ofs[e]]);
        } else {
            const float* src = reinterpret_cast<const float*>(g.data[ti]);
#pragma unroll
            for (int e = 0; e < 32; ++e) xs[e] = src[ofs[e]];
        }
    }
#pragma unroll
    for (int gq = 0; gq < 8; ++gq) {
        const int tg = t0 + 4 * gq;
        if (tg >= t0 + cnt) continue;
        uint32_t c0 = (uint32_t)(tg >> 2), c1 = rlo, c2 = rhi, c3 = 0u;
        philox4x32_10(c0, c1, c2, c3, k0, k1);
        const uint32_t wd[4] = {c0, c1, c2, c3};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int t = tg + e;
            if (t < t0 + cnt) {
                const float x = xs[4 * gq + e];
                int i = 0;
                for (int j = 1; j < m - 1; ++j) i += (q[j] <= x) ? 1 : 0;
                const float a = q[i];
                const float b = q[i + 1];
                float p = (x - a) / (b - a);
                p = fminf(fmaxf(p, 0.0f), 1.0f);
                const float u = (float)(wd[e] >> 8) * 0x1p-24f;
                const uint32_t code = (uint32_t)i + (u < p ? 1u : 0u);
                acc |= (uint64_t)code << nb;
                nb += w;
                if (nb >= 32) {
                    codes[wi++] = (uint32_t)acc;
                    acc >>= 32;
                    nb -= 32;
                }
            }
        }
    }
    if (nb > 0) codes[wi] = (uint32_t)acc;
}

__global__ void __launch_bounds__(kQuantThreads)
dequantize_kernel(int n, int s, const uint32_t* __restrict__ codes, const float* __restrict__ codebook,
                  const uint8_t* __restrict__ m_in, const uint64_t* __restrict__ off,
                  float* __restrict__ xhat) {
    __shared__ float q[kMaxS];
    const int64_t r = blockIdx.x;
    const int m = min(max((int)m_in[r], 1), s);
    if (threadIdx.x < s) q[threadIdx.x] = codebook[r * s + threadIdx.x];
    __syncthreads();
    const int w = code_width(m);
    const int t0 = threadIdx.x * 32;
    if (t0 >= n) return;
    const int cnt = min(32, n - t0);
    float* out = xhat + r * (int64_t)n + t0;
    if (w == 0) {
        for (int e = 0; e < cnt; ++e) out[e] = q[0];
        return;
    }
    const uint64_t mask = (1ull << w) - 1ull;
    uint64_t wi = off[r] + (uint64_t)threadIdx.x * (uint64_t)w;
    uint64_t acc = 0;
    int nb = 0;
    for (int e = 0; e < cnt; ++e) {
        if (nb < w) {
            acc |= (uint64_t)codes[wi++] << nb;
            nb += 32;
        }
        int code = (int)(acc & mask);
        acc >>= w;
        nb -= w;
        code = code < m ? code : m - 1;
        out[e] = q[code];
    }
}

// ---------------------------------------------------------------------------
// Blocks of 4096 contiguous entries.  In the quantizer lane t of the block's
// wave owns the 8-entry chunks t, t + 64, ..., t + 448.  A chunk's eight
// w-bit codes are exactly w bytes of the block's little-endian stream (chunk
// c at byte w c), so loads are 16-byte coalesced and stores are
// byte-granular with no cross-lane packing.  Codepoints live in LDS padded with +inf to 16 slots, so the
// interval search is a fixed four-step binary search; p uses the reciprocal
// of the interval width.

// quantize: one wave per block, 8 chunks of 8 entries per lane, when the
// launch has blocks enough to fill the GPU (256 threads with 2 chunks each
// was 10% slower there: the per-block set-up is paid per wave); 256 threads
// for small launches (a decode step), where a block's latency dominates.
// dequantize: 128 threads, lane t writing float4s t, t + 128, ..., t + 896 of
// its block, so each wave store writes 1 KB without gaps; the stores are
// non-temporal (the output is not read back by this pass).  256 threads with
// 4 stores per lane, and ordinary stores, were 9% slower on 2^19 blocks.
constexpr int kQT = 64;
constexpr int kQTSmall = 256;
constexpr int64_t kQSmallLaunch = 16384;  // blocks below which kQTSmall is used
constexpr int kDQT = 128;
typedef float f32x4 __attribute__((ext_vector_type(4)));

// One block per workgroup: small launches (a decode step, 256 threads so
// the few blocks finish soon) and fp32 input.
template <int kThreads, int kDt>
__global__ void __launch_bounds__(kThreads)
quantize4096_kernel(const void* __restrict__ x0, const void* __restrict__ x1, int64_t nb0,
                    int s, const float* __restrict__ codebook, const uint8_t* __restrict__ m_in,
                    const uint64_t* __restrict__ off, uint32_t k0, uint32_t k1,
                    uint32_t* __restrict__ codes) {
    __shared__ QuantLds L;
    const int64_t r = blockIdx.x;
    const int tid = threadIdx.x;
    // issue the block's independent loads before anything waits on one: the
    // codebook row (whole, s points), the size m and this lane's chunks
    const float cbv = tid < s ? codebook[r * s + tid] : __builtin_huge_valf();
    const int mraw = m_in[r];
    const uint64_t ob = off[r];
    const void* src = r < nb0 ? x0 : x1;
    const int64_t e_base = (r < nb0 ? r : r - nb0) * 4096;
    // fp16: every chunk of the lane is loaded here, before any code store
    // (one counter tracks loads and stores, so a load waited on after a
    // store would wait for that store too); fp32 chunks are twice the
    // registers and are loaded one step ahead instead
    constexpr int kNH = 512 / kThreads;
    uint4 all[kNH][2] = {};
    if (kDt == KVQ_F16) {
#pragma unroll
        for (int h = 0; h < kNH; ++h) load_raw8<kDt>(src, e_base + 8 * (tid + h * kThreads), all[h]);
    }
    quantize_block4096<kThreads, kDt>(L, r, s, cbv, mraw, ob, all, src, e_base, k0, k1, codes);
}

__global__ void __launch_bounds__(kDQT)
dequantize4096_kernel(int s, const uint32_t* __restrict__ codes, const float* __restrict__ codebook,
                      const uint8_t* __restrict__ m_in, const uint64_t* __restrict__ off,
                      float* __restrict__ xhat) {
    __shared__ float q[kMaxS];
    const int64_t r = blockIdx.x;
    const int tid = threadIdx.x;
    // m, the word offset and the codebook row are requested together
    const float cbv = tid < s ? codebook[r * s + tid] : 0.0f;
    const int mraw = m_in[r];
    const uint64_t ob = off[r];
    const int m = min(max(mraw, 1), s);
    if (tid < kMaxS) q[tid] = tid < m ? cbv : 0.0f;
    __syncthreads();
    const int w = code_width(m);
    const uint32_t* cw = codes + ob;
    const uint32_t mask = (1u << w) - 1u;
    float4* o = reinterpret_cast<float4*>(xhat + r * 4096);
    // every code word first: a load waited on between two stores would also
    // wait for the earlier store (one counter serves both).  The second word
    // is needed only when a group straddles a word boundary, never in the
    // block's last word (128 w words), so its index is clamped and both loads
    // are unconditional.
    constexpr int kIt = 1024 / kDQT;
    uint32_t wa[kIt] = {}, wb[kIt] = {};
    if (w) {
        const uint32_t last = 128u * (uint32_t)w - 1u;
#pragma unroll
        for (int k = 0; k < kIt; ++k) {
            const uint32_t q0 = (4u * (uint32_t)w * (uint32_t)(tid + k * kDQT)) >> 5;
            wa[k] = cw[q0];
            wb[k] = cw[min(q0 + 1u, last)];
        }
    }
#pragma unroll
    for (int k = 0; k < kIt; ++k) {
        const int j = tid + k * kDQT;           // float4 j = entries 4j .. 4j + 3
        uint32_t bits = 0;
        if (w) {
            const uint32_t sh = (4u * (uint32_t)w * (uint32_t)j) & 31u;
            bits = (uint32_t)((((uint64_t)wb[k] << 32) | wa[k]) >> sh);
        }
        float v[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            int code = (int)((bits >> (w * e)) & mask);
            code = code < m ? code : m - 1;
            v[e] = q[code];
        }
        __builtin_nontemporal_store((f32x4){v[0], v[1], v[2], v[3]}, reinterpret_cast<f32x4*>(&o[j]));
    }
}

static bool fast_layout(const Geom& g) {
    if (getenv("KVQ_FORCE_GENERIC")) return false;
    if (g.n != 4096 || !g.contig) return false;
    for (int i = 0; i < KVQ_MAX_TENSORS; ++i) {
        if (!g.data[i]) continue;
        // whole tensor contiguous: block r of a tensor starts at entry 4096 r
        if (g.stride[i][1] != (int64_t)g.chunks * g.Tb * g.Db * g.groups) return false;
        if (g.stride[i][0] != (int64_t)g.heads * g.stride[i][1]) return false;
        if (g.groups != 1) return false;
        if (((uintptr_t)g.data[i]) & 15u) return false;
    }
    return true;
}

hipError_t launch_quantize(const Geom& g, int64_t R, int s, const float* codebook, const uint8_t* m,
                           const uint64_t* off, uint64_t seed, uint32_t* codes, hipStream_t st) {
    if (R == 0) return hipSuccess;
    if (fast_layout(g)) {
        const void* x1 = g.data[1] ? g.data[1] : g.data[0];
        const bool f16 = g.dtype == KVQ_F16;
        const uint32_t k0 = (uint32_t)seed, k1 = (uint32_t)(seed >> 32);
        if (R < kQSmallLaunch) {
            if (f16)
                hipLaunchKernelGGL((quantize4096_kernel<kQTSmall, KVQ_F16>), dim3((unsigned)R), dim3(kQTSmall), 0,
                                   st, g.data[0], x1, g.nb0, s, codebook, m, off, k0, k1, codes);
            else
                hipLaunchKernelGGL((quantize4096_kernel<kQTSmall, KVQ_F32>), dim3((unsigned)R), dim3(kQTSmall), 0,
                                   st, g.data[0], x1, g.nb0, s, codebook, m, off, k0, k1, codes);
        } else {
            if (f16)
                hipLaunchKernelGGL((quantize4096_kernel<kQT, KVQ_F16>), dim3((unsigned)R), dim3(kQT), 0, st,
                                   g.data[0], x1, g.nb0, s, codebook, m, off, k0, k1, codes);
            else
                hipLaunchKernelGGL((quantize4096_kernel<kQT, KVQ_F32>), dim3((unsigned)R), dim3(kQT), 0, st,
                                   g.data[0], x1, g.nb0, s, codebook, m, off, k0, k1, codes);
        }
    } else {
        hipLaunchKernelGGL(quantize_kernel, dim3((unsigned)R), dim3(kQuantThreads), 0, st, g, s,
                           codebook, m, off, (uint32_t)seed, (uint32_t)(seed >> 32), codes);
    }
    return hipGetLastError();
}

hipError_t launch_dequantize(int64_t R, int n, int s, const uint32_t* codes, const float* codebook,
                             const uint8_t* m, const uint64_t* off, float* xhat, hipStream_t st) {
    if (R == 0) return hipSuccess;
    if (n == 4096 && !getenv("KVQ_FORCE_GENERIC") && !(((uintptr_t)xhat) & 15u)) {
        hipLaunchKernelGGL(dequantize4096_kernel, dim3((unsigned)R), dim3(kDQT), 0, st, s, codes,
                           codebook, m, off, xhat);
    } else {
        hipLaunchKernelGGL(dequantize_kernel, dim3((unsigned)R), dim3(kQuantThreads), 0, st, n, s,
                           codes, codebook, m, off, xhat);
    }
    return hipGetLastError();
}

}  // namespace kvq
