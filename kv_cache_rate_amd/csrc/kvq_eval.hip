// Candidate scoring (kvq_eval_candidates), generic path.
//
// Page "Rate-adaptive KV-cache quantizer": Implementation notes (candidate
// alphabet from the block's minimum, maximum and quantiles; D_r from interval
// statistics; H_r from expected symbol frequencies) and Key formulas (3)
// (interpolation probabilities, conditional MSE (q_{i+1}-x)(x-q_i)).
//
// One workgroup scores one block.  The block's entries are sorted in LDS
// (bitonic network on order-preserving 32-bit keys), so every order
// statistic is an LDS read and every codepoint's rank is a binary search.
// Interval statistics come from fp64 prefix sums over the sorted entries:
// for the entries of [a, b) with count C, sum S1 and sum of squares S2,
//     D_int = sum (b - x)(x - a) = -S2 + (a + b) S1 - a b C,
//     mass to b = sum (x - a)/(b - a) = (S1 - a C)/(b - a),  mass to a = C - that.
// The last interval of a codebook is closed (it also takes the entries equal
// to the maximum).  Per-thread partial sums plus a short in-thread tail give
// the prefix at any rank, so no 4096-entry fp64 array is held in LDS.
#include "kvq_internal.h"

namespace kvq {

constexpr int kEvalThreads = 256;

__global__ void ws_reset_kernel(WsHeader* h) {
    if (threadIdx.x == 0) {
        h->status = 0;
        h->phase = 0;
        h->done = 0;
        h->err = 0;
        h->nlam = 0;
    }
}

hipError_t launch_ws_reset(void* ws, hipStream_t st) {
    hipLaunchKernelGGL(ws_reset_kernel, dim3(1), dim3(64), 0, st, (WsHeader*)ws);
    return hipGetLastError();
}

// Bitonic sort of one block's NP keys (NP a power of two), thread t
// holding positions [E t, E t + E) in registers.  A stage whose partner
// distance j is below E stays inside the thread; one with j below 64 E
// exchanges across the wave by lane shuffles; only the stages with j >= 64 E
// (two or three per sort) pass through LDS and a barrier.
template <int E>
__device__ void bitonic_regs(uint32_t (&v)[E], int NP, uint32_t* buf) {
    const int t = threadIdx.x;
    for (int k = 2; k <= NP; k <<= 1) {
        for (int j = k >> 1; j >= E; j >>= 1) {
            // partner of position E t + e is E (t ^ tj) + e; the pair takes
            // the direction of its lower position, (E t) & k (k > j >= E)
            const int tj = j / E;
            const bool take_min = ((t & tj) == 0) == (((E * t) & k) == 0);
            uint32_t p[E];
            if (tj < 64) {
#pragma unroll
                for (int e = 0; e < E; ++e) p[e] = __shfl_xor(v[e], tj, 64);
            } else {
#pragma unroll
                for (int e = 0; e < E; ++e) buf[E * t + e] = v[e];
                __syncthreads();
#pragma unroll
                for (int e = 0; e < E; ++e) p[e] = buf[E * (t ^ tj) + e];
                __syncthreads();
            }
#pragma unroll
            for (int e = 0; e < E; ++e) v[e] = take_min ? min(v[e], p[e]) : max(v[e], p[e]);
        }
#pragma unroll
        for (int jj = E / 2; jj >= 1; jj >>= 1) {
            if (jj < k) {
#pragma unroll
                for (int e = 0; e < E; ++e) {
                    if ((e & jj) == 0) {
                        const bool asc = ((E * t + e) & k) == 0;
                        const uint32_t a = v[e], b = v[e | jj];
                        const uint32_t lo = min(a, b), hi = max(a, b);
                        v[e] = asc ? lo : hi;
                        v[e | jj] = asc ? hi : lo;
                    }
                }
            }
        }
    }
}

// Load block r as order-preserving keys (padding keys sort last), flag
// non-finite entries, sort ascending, and leave the sorted values in LDS
// as fp32 (position i at xs[i], i < NP).
template <int E>
__device__ void load_and_sort_e(const Geom& g, int64_t r, int NP, uint32_t* keys, WsHeader* ws) {
    int ti;
    const int64_t base = block_base(g, r, ti);
    const int n = g.n;
    const int t0 = E * (int)threadIdx.x;
    // every load first, unconditionally (positions past the block read its
    // last entry and are dropped): a load under the position test was
    // waited on by itself, one memory round trip per key
    int64_t ofs[E];
#pragma unroll
    for (int e = 0; e < E; ++e) ofs[e] = base + entry_off(g, ti, min(t0 + e, n - 1));
    float xv[E];
    if (g.dtype == KVQ_F16) {
        const __half* src = reinterpret_cast<const __half*>(g.data[ti]);
#pragma unroll
        for (int e = 0; e < E; ++e) xv[e] = __half2float(src[ofs[e]]);
    } else {
        const float* src = reinterpret_cast<const float*>(g.data[ti]);
#pragma unroll
        for (int e = 0; e < E; ++e) xv[e] = src[ofs[e]];
    }
    uint32_t v[E];
    bool bad = false;
#pragma unroll
    for (int e = 0; e < E; ++e) {
        uint32_t k = 0xffffffffu;
        if (t0 + e < n) {
            float x = xv[e];
            if (x == 0.0f) x = 0.0f;  // -0 -> +0
            if (!isfinite(x)) bad = true;
            k = f32_key(x);
        }
        v[e] = k;
    }
    if (__syncthreads_or(bad)) {
        if (threadIdx.x == 0) atomicOr(&ws->status, kStatusNonFinite);
    }
    bitonic_regs<E>(v, NP, keys);
    float* xs = reinterpret_cast<float*>(keys);
#pragma unroll
    for (int e = 0; e < E; ++e)
        if (t0 + e < NP) xs[t0 + e] = key_f32(v[e]);
    __syncthreads();
}

// NP = next power of two of the block size, 2 .. kMaxBlock; each of the
// kEvalThreads threads holds NP / kEvalThreads keys (at least one).
__device__ void load_and_sort(const Geom& g, int64_t r, int NP, uint32_t* keys, WsHeader* ws) {
    static_assert(kMaxBlock == 16 * kEvalThreads, "16 keys per thread at most");
    switch (NP / kEvalThreads) {
        case 16: load_and_sort_e<16>(g, r, NP, keys, ws); break;
        case 8: load_and_sort_e<8>(g, r, NP, keys, ws); break;
        case 4: load_and_sort_e<4>(g, r, NP, keys, ws); break;
        case 2: load_and_sort_e<2>(g, r, NP, keys, ws); break;
        default: load_and_sort_e<1>(g, r, NP, keys, ws); break;
    }
}

__device__ __forceinline__ double wave_incl_scan(double v) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const double o = __shfl_up(v, off, 64);
        if (lane >= off) v += o;
    }
    return v;
}

// Exclusive per-thread prefix of (x, x^2) over chunks of CH sorted entries.
// tp1/tp2 get kEvalThreads + 1 entries (the last one is the block total).
__device__ void chunk_prefix(const float* xs, int n, int CH, double* tp1, double* tp2,
                             double* wt1, double* wt2) {
    const int tid = threadIdx.x;
    double s1 = 0.0, s2 = 0.0;
    for (int k = 0; k < CH; ++k) {
        const int i = tid * CH + k;
        if (i < n) {
            const double x = xs[i];
            s1 += x;
            s2 += x * x;
        }
    }
    const double i1 = wave_incl_scan(s1);
    const double i2 = wave_incl_scan(s2);
    const int wave = tid >> 6;
    if ((tid & 63) == 63) {
        wt1[wave] = i1;
        wt2[wave] = i2;
    }
    __syncthreads();
    double o1 = 0.0, o2 = 0.0;
    for (int w = 0; w < wave; ++w) {
        o1 += wt1[w];
        o2 += wt2[w];
    }
    tp1[tid] = o1 + i1 - s1;
    tp2[tid] = o2 + i2 - s2;
    if (tid == kEvalThreads - 1) {
        tp1[kEvalThreads] = o1 + i1;
        tp2[kEvalThreads] = o2 + i2;
    }
    __syncthreads();
}

__device__ __forceinline__ void prefix_at(int q, const float* xs, int CH, const double* tp1,
                                          const double* tp2, double& p1, double& p2) {
    const int c = q / CH;
    p1 = tp1[c];
    p2 = tp2[c];
    for (int i = c * CH; i < q; ++i) {
        const double x = xs[i];
        p1 += x;
        p2 += x * x;
    }
}

// First index i in [0, n) with xs[i] >= v (n if none).
__device__ __forceinline__ int lower_bound(const float* xs, int n, float v) {
    int lo = 0, hi = n;
    while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (xs[mid] < v) lo = mid + 1;
        else hi = mid;
    }
    return lo;
}

// Interval [a, b) (closed when it is the last) with count C, sums S1, S2.
__device__ __forceinline__ void interval_terms(double a, double b, double C, double S1, double S2,
                                               double& Dint, double& ma, double& mb) {
    Dint = -S2 + (a + b) * S1 - a * b * C;
    mb = (S1 - a * C) / (b - a);
    mb = fmin(fmax(mb, 0.0), C);
    ma = C - mb;
}

__global__ void __launch_bounds__(kEvalThreads)
eval_grids_kernel(Geom g, int s, int NP, RankTable rt, double* __restrict__ D,
                  double* __restrict__ H, float* __restrict__ stats, WsHeader* ws) {
    __shared__ uint32_t keys[kMaxBlock];
    __shared__ double tp1[kEvalThreads + 1], tp2[kEvalThreads + 1];
    __shared__ double wt1[kEvalThreads / 64], wt2[kEvalThreads / 64];
    __shared__ float cq[kMaxCand][kMaxS];
    __shared__ int cm[kMaxCand];
    __shared__ int crank[kMaxCand][kMaxS];
    __shared__ double cp1[kMaxCand][kMaxS], cp2[kMaxCand][kMaxS];

    const int64_t r = xcd_block(blockIdx.x, gridDim.x);
    const int n = g.n;
    const int C = 1 + 2 * (s - 2);
    const int tid = threadIdx.x;
    load_and_sort(g, r, NP, keys, ws);
    const float* xs = reinterpret_cast<const float*>(keys);
    const int CH = (NP + kEvalThreads - 1) / kEvalThreads;
    chunk_prefix(xs, n, CH, tp1, tp2, wt1, wt2);

    const int64_t R = gridDim.x;
    for (int k = tid; k < rt.n_stats; k += blockDim.x) stats[k * R + r] = xs[rt.rank[k]];

    const float mn = xs[0];
    const float mx = xs[n - 1];
    if (tid < C) {
        const int c = tid;
        int k;
        bool uni = false;
        if (c == 0) {
            k = 2;
        } else {
            k = 3 + (c - 1) / 2;
            uni = ((c - 1) & 1) == 0;
        }
        int m = 0;
        for (int j = 0; j < k; ++j) {
            float v;
            if (c == 0) v = j == 0 ? mn : mx;
            else if (uni) v = uniform_point(mn, mx, j, k);
            else v = xs[quantile_rank(j, k, n)];
            if (m == 0 || v != cq[c][m - 1]) cq[c][m++] = v;
        }
        cm[c] = m;
    }
    __syncthreads();
    for (int sl = tid; sl < C * kMaxS; sl += blockDim.x) {
        const int c = sl / kMaxS;
        const int j = sl - c * kMaxS;
        const int m = cm[c];
        if (j < m) {
            const int q = (j == m - 1) ? n : lower_bound(xs, n, cq[c][j]);
            crank[c][j] = q;
            double p1, p2;
            prefix_at(q, xs, CH, tp1, tp2, p1, p2);
            cp1[c][j] = p1;
            cp2[c][j] = p2;
        }
    }
    __syncthreads();
    if (tid < C) {
        const int c = tid;
        const int m = cm[c];
        double Dc = 0.0, Hc = 0.0;
        if (m >= 2) {
            double carry = 0.0;  // mass already sent to point j from its left interval
            const double inv_n = 1.0 / (double)n;
            for (int j = 0; j + 1 < m; ++j) {
                const double a = cq[c][j];
                const double b = cq[c][j + 1];
                const int lo = j == 0 ? 0 : crank[c][j];
                const double Cn = (double)(crank[c][j + 1] - lo);
                const double S1 = cp1[c][j + 1] - (j == 0 ? 0.0 : cp1[c][j]);
                const double S2 = cp2[c][j + 1] - (j == 0 ? 0.0 : cp2[c][j]);
                double Dint, ma, mb;
                interval_terms(a, b, Cn, S1, S2, Dint, ma, mb);
                Dc += Dint;
                const double pj = (carry + ma) * inv_n;
                if (pj > 0.0) Hc -= pj * log2(pj);
                carry = mb;
            }
            const double pl = carry * inv_n;
            if (pl > 0.0) Hc -= pl * log2(pl);
        }
        D[c * R + r] = fmax(Dc, 0.0);
        H[c * R + r] = fmax(Hc, 0.0);
    }
}

__global__ void __launch_bounds__(kEvalThreads)
eval_alphabet_kernel(Geom g, int alpha_m, int NP, double* __restrict__ D, double* __restrict__ H,
                     float* __restrict__ stats, WsHeader* ws) {
    __shared__ uint32_t keys[kMaxBlock];
    __shared__ double tp1[kEvalThreads + 1], tp2[kEvalThreads + 1];
    __shared__ double wt1[kEvalThreads / 64], wt2[kEvalThreads / 64];
    __shared__ float A[kAlpha];
    __shared__ int arank[kAlpha];
    __shared__ double ap1[kAlpha], ap2[kAlpha];
    __shared__ int am;

    const int64_t r = blockIdx.x;
    const int n = g.n;
    const int tid = threadIdx.x;
    load_and_sort(g, r, NP, keys, ws);
    const float* xs = reinterpret_cast<const float*>(keys);
    const int CH = (NP + kEvalThreads - 1) / kEvalThreads;
    chunk_prefix(xs, n, CH, tp1, tp2, wt1, wt2);

    if (tid < alpha_m) stats[r * alpha_m + tid] = xs[quantile_rank(tid, alpha_m, n)];
    if (tid == 0) {
        int m = 0;
        for (int j = 0; j < alpha_m; ++j) {
            const float v = xs[quantile_rank(j, alpha_m, n)];
            if (m == 0 || v != A[m - 1]) A[m++] = v;
        }
        am = m;
    }
    __syncthreads();
    const int m = am;
    if (tid < m) {
        const int q = tid == 0 ? 0 : (tid == m - 1 ? n : lower_bound(xs, n, A[tid]));
        arank[tid] = q;
        double p1, p2;
        prefix_at(q, xs, CH, tp1, tp2, p1, p2);
        ap1[tid] = p1;
        ap2[tid] = p2;
    }
    __syncthreads();
    const int P = n_pairs(alpha_m);
    for (int p = tid; p < P; p += kEvalThreads) {
        // decode pair index -> (i, j) of the alpha_m-point triangle
        int i = 0, rem = p;
        while (rem >= alpha_m - 1 - i) {
            rem -= alpha_m - 1 - i;
            ++i;
        }
        const int j = i + 1 + rem;
        double Dp = 0.0, ML = 0.0, MR = 0.0;
        if (j < m) {
            // entries of [A_i, A_j), closed at the last alphabet point
            const int lo = arank[i];
            double p1lo = ap1[i], p2lo = ap2[i];
            if (i == 0) { p1lo = 0.0; p2lo = 0.0; }
            const int hi_rank = (j == m - 1) ? n : arank[j];
            double p1hi, p2hi;
            if (j == m - 1) {
                p1hi = tp1[kEvalThreads];
                p2hi = tp2[kEvalThreads];
            } else {
                p1hi = ap1[j];
                p2hi = ap2[j];
            }
            const double Cn = (double)(hi_rank - (i == 0 ? 0 : lo));
            interval_terms((double)A[i], (double)A[j], Cn, p1hi - p1lo, p2hi - p2lo, Dp, ML, MR);
            Dp = fmax(Dp, 0.0);
        }
        D[r * P + p] = Dp;
        H[(r * P + p) * 2 + 0] = ML;
        H[(r * P + p) * 2 + 1] = MR;
    }
}

static int next_pow2(int n) {
    int p = 1;
    while (p < n) p <<= 1;
    return p;
}

hipError_t launch_eval_grids(const Geom& g, int64_t R, int s, const RankTable& rt, double* D,
                             double* H, float* stats, void* ws, hipStream_t st) {
    if (R == 0) return hipSuccess;
    const int NP = next_pow2(g.n);
    hipLaunchKernelGGL(eval_grids_kernel, dim3((unsigned)R), dim3(kEvalThreads), 0, st, g, s, NP,
                       rt, D, H, stats, (WsHeader*)ws);
    return hipGetLastError();
}

hipError_t launch_eval_alphabet(const Geom& g, int64_t R, int alpha_m, double* D, double* H,
                                float* stats, void* ws, hipStream_t st) {
    if (R == 0) return hipSuccess;
    const int NP = next_pow2(g.n);
    hipLaunchKernelGGL(eval_alphabet_kernel, dim3((unsigned)R), dim3(kEvalThreads), 0, st, g,
                       alpha_m, NP, D, H, stats, (WsHeader*)ws);
    return hipGetLastError();
}

}  // namespace kvq
