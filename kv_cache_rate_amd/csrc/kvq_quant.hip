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
#include "kvq_internal.h"

namespace kvq {

constexpr int kQuantThreads = 128;  // 128 x 32 entries = 4096

__global__ void __launch_bounds__(kQuantThreads)
quantize_kernel(Geom g, int s, const float* __restrict__ codebook, const uint8_t* __restrict__ m_in,
                const uint64_t* __restrict__ off, uint32_t k0, uint32_t k1,
                uint32_t* __restrict__ codes) {
    __shared__ float q[kMaxS];
    const int64_t r = blockIdx.x;
    const int m = m_in[r];
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
    for (int gq = 0; gq < 8; ++gq) {
        const int tg = t0 + 4 * gq;
        if (tg >= t0 + cnt) break;
        uint32_t c0 = (uint32_t)(tg >> 2), c1 = rlo, c2 = rhi, c3 = 0u;
        philox4x32_10(c0, c1, c2, c3, k0, k1);
        const uint32_t wd[4] = {c0, c1, c2, c3};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int t = tg + e;
            if (t < t0 + cnt) {
                const float x = load_entry(g, ti, base + entry_off(g, ti, t));
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
    const int m = m_in[r];
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

hipError_t launch_quantize(const Geom& g, int64_t R, int s, const float* codebook, const uint8_t* m,
                           const uint64_t* off, uint64_t seed, uint32_t* codes, hipStream_t st) {
    if (R == 0) return hipSuccess;
    hipLaunchKernelGGL(quantize_kernel, dim3((unsigned)R), dim3(kQuantThreads), 0, st, g, s, codebook,
                       m, off, (uint32_t)seed, (uint32_t)(seed >> 32), codes);
    return hipGetLastError();
}

hipError_t launch_dequantize(int64_t R, int n, int s, const uint32_t* codes, const float* codebook,
                             const uint8_t* m, const uint64_t* off, float* xhat, hipStream_t st) {
    if (R == 0) return hipSuccess;
    hipLaunchKernelGGL(dequantize_kernel, dim3((unsigned)R), dim3(kQuantThreads), 0, st, n, s, codes,
                       codebook, m, off, xhat);
    return hipGetLastError();
}

}  // namespace kvq
