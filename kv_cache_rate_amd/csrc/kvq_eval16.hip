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
// exactly by (count, sum of f) packed in one 32-bit LDS word.  Sweep 1 fills
// these; a prefix over bins gives counts and exact fp64 sums at bin edges
// (fp16 sums of 4096 entries are exact in fp64).  The coarse bins that hold
// a wanted order statistic or a uniform-grid threshold get per-key counts in
// sweep 2 (packed 16-bit counters), and one lane per threshold finishes its
// prefix inside the bin.  Order statistics are therefore exact data values
// and every prefix is exact; only the final per-interval algebra rounds.
//
// Workgroup = one block, 256 threads x 16 entries kept in registers.
#include <string.h>

#include "kvq_internal.h"

namespace kvq {

namespace {

constexpr int kT = 256;            // threads per block
constexpr int kPer = 16;           // entries per thread
constexpr int kNC = 1024;          // coarse bins
constexpr int kFine = 64;          // keys per coarse bin
constexpr int kSlotWords = kFine / 2;
constexpr int kMaxSlots = 128;     // coarse bins resolved per batch
constexpr int kNU = 71;            // distinct interior uniform fractions, s = 16
constexpr int kNQ = 73;            // order statistics, s = 16, n = 4096
constexpr uint16_t kNoSlot = 0xffff;

struct Phase1 {
    uint32_t cnt[kNC];        // sweep 1 payload: count | sum(f) << 13
    uint32_t pc[kNC + 1];     // exclusive prefix counts
    double ps1[kNC + 1];      // exclusive prefix sums
    uint16_t slot[kNC];       // resolved-bin slot or kNoSlot
    uint32_t fine[kMaxSlots][kSlotWords];
};

struct Phase2 {
    float pval[kMaxCand][kMaxS];   // candidate codepoints
    uint32_t pcnt[kMaxCand][kMaxS];  // entries below the codepoint (n at the closed end)
    double ps1[kMaxCand][kMaxS];   // their sum
    double ma[kMaxCand][kMaxS];    // mass of interval j sent to its left end
    double mb[kMaxCand][kMaxS];    // ... and to its right end
    double qm[kMaxCand][kMaxS];    // q_j^2 M_j
    double hb[kMaxCand][kMaxS];    // -pi_j log2 pi_j
    int cm[kMaxCand];
};

struct Shared {
    union {
        Phase1 p1;
        Phase2 p2;
    } u;
    // order statistics (targets) and uniform thresholds
    uint16_t tbin[kNQ];
    uint16_t tloc[kNQ];
    float tval[kNQ];
    uint32_t tcnt[kNQ];
    double ts1[kNQ];
    uint16_t ukey[kNU];
    float uval[kNU];
    uint32_t ucnt[kNU];
    double us1[kNU];
    // reductions
    uint32_t kmin[kT / 64], kmax[kT / 64];
    double wsq[kT / 64];
    uint32_t wtot[kT / 64];
    double wts1[kT / 64];
    int nslots;
    int bad;
};

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

__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = min(v, (uint32_t)__shfl_xor((int)v, o, 64));
    return v;
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = max(v, (uint32_t)__shfl_xor((int)v, o, 64));
    return v;
}
__device__ __forceinline__ double wave_sum_f64(double v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}
__device__ __forceinline__ uint32_t wave_incl_u32(uint32_t v) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const uint32_t t = (uint32_t)__shfl_up((int)v, o, 64);
        if (lane >= o) v += t;
    }
    return v;
}
__device__ __forceinline__ double wave_incl_f64(double v) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const double t = __shfl_up(v, o, 64);
        if (lane >= o) v += t;
    }
    return v;
}

}  // namespace

// Threshold tables from the host: quantile ranks / stats columns and the
// reduced fractions of the uniform grids.
struct Eval16Tables {
    RankTable rt;
    uint8_t unum[kNU];   // numerator of distinct fraction u
    uint8_t uden[kNU];   // denominator
    uint8_t ucol[kMaxS + 1][kMaxS];  // fraction index of U_k point j (interior j)
};

__global__ void __launch_bounds__(kT)
eval16_kernel(const __half* __restrict__ x0, const __half* __restrict__ x1, int64_t nb0,
              Eval16Tables tb, double* __restrict__ Dout, double* __restrict__ Hout,
              float* __restrict__ stats, WsHeader* ws) {
    __shared__ Shared sh;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int64_t r = blockIdx.x;
    const __half* src = r < nb0 ? x0 + r * 4096 : x1 + (r - nb0) * 4096;

    // ---- load: thread owns entries [8 tid, 8 tid + 8) and [2048 + 8 tid, ...)
    uint32_t hw[8];
    {
        const uint4 a = reinterpret_cast<const uint4*>(src)[tid];
        const uint4 b = reinterpret_cast<const uint4*>(src)[256 + tid];
        hw[0] = a.x; hw[1] = a.y; hw[2] = a.z; hw[3] = a.w;
        hw[4] = b.x; hw[5] = b.y; hw[6] = b.z; hw[7] = b.w;
    }
    for (int i = tid; i < kNC; i += kT) sh.u.p1.cnt[i] = 0u;
    if (tid == 0) sh.bad = 0;
    __syncthreads();

    // ---- sweep 1: keys, coarse histogram, min/max, sum of squares
    uint32_t kmin = 0xffffu, kmax = 0u;
    double sq = 0.0;
    bool bad = false;
    uint32_t keys[kPer];
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
        uint32_t h = (hw[i >> 1] >> ((i & 1) * 16)) & 0xffffu;
        if (h == 0x8000u) h = 0u;  // -0 -> +0
        bad |= (h & 0x7c00u) == 0x7c00u;
        const uint32_t key = half_key(h);
        keys[i] = key;
        kmin = min(kmin, key);
        kmax = max(kmax, key);
        const float v = __half2float(__ushort_as_half((unsigned short)h));
        sq += (double)v * (double)v;
        atomicAdd(&sh.u.p1.cnt[key >> 6], 1u | ((key & 63u) << 13));
    }
    if (bad) sh.bad = 1;
    kmin = wave_min_u32(kmin);
    kmax = wave_max_u32(kmax);
    sq = wave_sum_f64(sq);
    if (lane == 0) {
        sh.kmin[wave] = kmin;
        sh.kmax[wave] = kmax;
        sh.wsq[wave] = sq;
    }
    __syncthreads();
    if (sh.bad && tid == 0) atomicOr(&ws->status, kStatusNonFinite);
    kmin = min(min(sh.kmin[0], sh.kmin[1]), min(sh.kmin[2], sh.kmin[3]));
    kmax = max(max(sh.kmax[0], sh.kmax[1]), max(sh.kmax[2], sh.kmax[3]));
    const double sumsq = (sh.wsq[0] + sh.wsq[1]) + (sh.wsq[2] + sh.wsq[3]);
    const float mn = key_value(kmin);
    const float mx = key_value(kmax);

    // ---- coarse prefix: thread owns bins [4 tid, 4 tid + 4)
    {
        uint32_t c[4];
        double s[4];
        uint32_t ct = 0;
        double st = 0.0;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const uint32_t bin = 4 * tid + k;
            const uint32_t p = sh.u.p1.cnt[bin];
            const uint32_t C = p & 0x1fffu;
            const uint32_t SF = p >> 13;
            const float B = key_value(bin << 6);
            const float U = key_value((bin << 6) | 1u) - B;
            c[k] = C;
            // empty bins add exactly 0 (the Inf/NaN code bins have no finite base)
            s[k] = C ? (double)C * (double)B + (double)U * (double)SF : 0.0;
            ct += C;
            st += s[k];
        }
        const uint32_t ic = wave_incl_u32(ct);
        const double is = wave_incl_f64(st);
        if (lane == 63) {
            sh.wtot[wave] = ic;
            sh.wts1[wave] = is;
        }
        __syncthreads();
        uint32_t oc = 0;
        double os = 0.0;
        for (int w = 0; w < wave; ++w) {
            oc += sh.wtot[w];
            os += sh.wts1[w];
        }
        uint32_t runc = oc + ic - ct;
        double runs = os + (is - st);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            sh.u.p1.pc[4 * tid + k] = runc;
            sh.u.p1.ps1[4 * tid + k] = runs;
            runc += c[k];
            runs += s[k];
        }
        if (tid == kT - 1) {
            sh.u.p1.pc[kNC] = runc;
            sh.u.p1.ps1[kNC] = runs;
        }
        for (int i = tid; i < kNC; i += kT) sh.u.p1.slot[i] = kNoSlot;
    }
    __syncthreads();

    // ---- targets (order statistics) and uniform thresholds
    const int nq = tb.rt.n_stats;  // 73
    if (tid < nq) {
        const uint32_t rank = (uint32_t)tb.rt.rank[tid];
        int lo = 0, hi = kNC - 1;  // last bin with pc[bin] <= rank
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (sh.u.p1.pc[mid] <= rank) lo = mid;
            else hi = mid - 1;
        }
        sh.tbin[tid] = (uint16_t)lo;
        sh.tloc[tid] = (uint16_t)(rank - sh.u.p1.pc[lo]);
        sh.u.p1.slot[lo] = 0;  // mark
    } else if (tid >= 128 && tid < 128 + kNU) {
        const int u = tid - 128;
        float t;
        {
#pragma clang fp contract(off)
            const double dmn = (double)mn;
            const double span = (double)mx - dmn;
            t = (float)(dmn + (span * (double)tb.unum[u]) / (double)tb.uden[u]);
        }
        const uint32_t key = key_ceil(t);
        sh.uval[u] = t;
        sh.ukey[u] = (uint16_t)key;
        sh.u.p1.slot[key >> 6] = 0;  // mark
    }
    __syncthreads();
    // compact marked bins into slots (thread owns 4 bins)
    {
        uint32_t m4 = 0;
#pragma unroll
        for (int k = 0; k < 4; ++k) m4 += sh.u.p1.slot[4 * tid + k] == 0 ? 1u : 0u;
        const uint32_t im = wave_incl_u32(m4);
        if (lane == 63) sh.wtot[wave] = im;
        __syncthreads();
        uint32_t o = 0;
        for (int w = 0; w < wave; ++w) o += sh.wtot[w];
        uint32_t s = o + im - m4;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int bin = 4 * tid + k;
            if (sh.u.p1.slot[bin] == 0) sh.u.p1.slot[bin] = (uint16_t)(s++);
        }
        if (tid == kT - 1) sh.nslots = (int)s;
    }
    __syncthreads();
    const int nslots = sh.nslots;

    // ---- sweep 2 (in batches of kMaxSlots resolved bins) and prefix finish
    for (int base = 0; base < nslots; base += kMaxSlots) {
        for (int i = tid; i < kMaxSlots * kSlotWords; i += kT) (&sh.u.p1.fine[0][0])[i] = 0u;
        __syncthreads();
#pragma unroll
        for (int i = 0; i < kPer; ++i) {
            const uint32_t key = keys[i];
            const uint32_t sl = (uint32_t)sh.u.p1.slot[key >> 6] - (uint32_t)base;
            if (sl < (uint32_t)kMaxSlots) {
                const uint32_t f = key & 63u;
                atomicAdd(&sh.u.p1.fine[sl][f >> 1], 1u << ((f & 1u) * 16));
            }
        }
        __syncthreads();
        if (tid < nq) {
            const uint32_t bin = sh.tbin[tid];
            const uint32_t sl = (uint32_t)sh.u.p1.slot[bin] - (uint32_t)base;
            if (sl < (uint32_t)kMaxSlots) {
                const uint32_t loc = sh.tloc[tid];
                uint32_t N = 0, F1 = 0, f = 0;
                for (int wd = 0; wd < kSlotWords; ++wd) {
                    const uint32_t w = sh.u.p1.fine[sl][wd];
                    const uint32_t c0 = w & 0xffffu, c1 = w >> 16;
                    if (N + c0 > loc) { f = 2 * wd; break; }
                    N += c0;
                    F1 += (2 * wd) * c0;
                    if (N + c1 > loc) { f = 2 * wd + 1; break; }
                    N += c1;
                    F1 += (2 * wd + 1) * c1;
                }
                const float B = key_value(bin << 6);
                const float U = key_value((bin << 6) | 1u) - B;
                sh.tval[tid] = key_value((bin << 6) | f);
                sh.tcnt[tid] = sh.u.p1.pc[bin] + N;
                sh.ts1[tid] = sh.u.p1.ps1[bin] + (double)B * (double)N + (double)U * (double)F1;
            }
        } else if (tid >= 128 && tid < 128 + kNU) {
            const int u = tid - 128;
            const uint32_t key = sh.ukey[u];
            const uint32_t bin = key >> 6;
            const uint32_t sl = (uint32_t)sh.u.p1.slot[bin] - (uint32_t)base;
            if (sl < (uint32_t)kMaxSlots) {
                const uint32_t fstop = key & 63u;
                uint32_t N = 0, F1 = 0;
                for (uint32_t f = 0; f < fstop; ++f) {
                    const uint32_t c = (sh.u.p1.fine[sl][f >> 1] >> ((f & 1u) * 16)) & 0xffffu;
                    N += c;
                    F1 += f * c;
                }
                const float B = key_value(bin << 6);
                const float U = key_value((bin << 6) | 1u) - B;
                sh.ucnt[u] = sh.u.p1.pc[bin] + N;
                sh.us1[u] = sh.u.p1.ps1[bin] + (double)B * (double)N + (double)U * (double)F1;
            }
        }
        __syncthreads();
    }
    const double total_s1 = sh.u.p1.ps1[kNC];
    __syncthreads();  // phase-1 storage is reused below

    // ---- order statistics out
    if (tid < nq) stats[r * nq + tid] = sh.tval[tid];

    // ---- candidate codepoints with their prefixes (closed last interval)
    const int C = kMaxCand;  // s = 16
    Phase2& p2 = sh.u.p2;
    if (tid < C) {
        const int c = tid;
        int k;
        bool uni = false;
        if (c == 0) k = 2;
        else {
            k = 3 + (c - 1) / 2;
            uni = ((c - 1) & 1) == 0;
        }
        int m = 0;
        for (int j = 0; j < k; ++j) {
            float v;
            uint32_t cn;
            double s1;
            if (j == 0) {
                v = mn; cn = 0; s1 = 0.0;
            } else if (j == k - 1) {
                v = mx; cn = 4096; s1 = total_s1;
            } else if (uni) {
                const int u = tb.ucol[k][j];
                v = sh.uval[u]; cn = sh.ucnt[u]; s1 = sh.us1[u];
            } else {
                const int q = tb.rt.col[k][j];
                v = sh.tval[q]; cn = sh.tcnt[q]; s1 = sh.ts1[q];
            }
            if (m > 0 && v == p2.pval[c][m - 1]) {
                if (j == k - 1) {  // the maximum keeps the closed end
                    p2.pcnt[c][m - 1] = cn;
                    p2.ps1[c][m - 1] = s1;
                }
                continue;
            }
            p2.pval[c][m] = v;
            p2.pcnt[c][m] = cn;
            p2.ps1[c][m] = s1;
            ++m;
        }
        p2.cm[c] = m;
    }
    __syncthreads();
    // interval masses: slot (c, j) for interval [q_j, q_{j+1}]
    for (int sl = tid; sl < C * kMaxS; sl += kT) {
        const int c = sl / kMaxS, j = sl - c * kMaxS;
        const int m = p2.cm[c];
        if (j + 1 < m) {
            const double a = p2.pval[c][j], b = p2.pval[c][j + 1];
            const double Cn = (double)(p2.pcnt[c][j + 1] - p2.pcnt[c][j]);
            const double S1 = p2.ps1[c][j + 1] - p2.ps1[c][j];
            double mbv = (S1 - a * Cn) / (b - a);
            mbv = fmin(fmax(mbv, 0.0), Cn);
            p2.mb[c][j] = mbv;
            p2.ma[c][j] = Cn - mbv;
        }
    }
    __syncthreads();
    // point terms: q_j^2 M_j and -pi_j log2 pi_j
    for (int sl = tid; sl < C * kMaxS; sl += kT) {
        const int c = sl / kMaxS, j = sl - c * kMaxS;
        const int m = p2.cm[c];
        if (j < m && m >= 2) {
            double M = 0.0;
            if (j > 0) M += p2.mb[c][j - 1];
            if (j + 1 < m) M += p2.ma[c][j];
            const double q = p2.pval[c][j];
            p2.qm[c][j] = q * q * M;
            const double pi = M * (1.0 / 4096.0);
            p2.hb[c][j] = pi > 0.0 ? -pi * log2(pi) : 0.0;
        }
    }
    __syncthreads();
    if (tid < C) {
        const int c = tid;
        const int m = p2.cm[c];
        double Dc = 0.0, Hc = 0.0;
        if (m >= 2) {
            double qs = 0.0;
            for (int j = 0; j < m; ++j) {
                qs += p2.qm[c][j];
                Hc += p2.hb[c][j];
            }
            Dc = qs - sumsq;
        }
        Dout[r * C + c] = fmax(Dc, 0.0);
        Hout[r * C + c] = fmax(Hc, 0.0);
    }
}

hipError_t launch_eval16(const void* x0, const void* x1, int64_t nb0, int64_t R, const RankTable& rt,
                         double* D, double* H, float* stats, void* ws, hipStream_t st) {
    if (R == 0) return hipSuccess;
    Eval16Tables tb;
    memset(&tb, 0, sizeof tb);
    tb.rt = rt;
    // distinct interior fractions j/(k-1), k = 3..16, in order of first appearance
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
            tb.ucol[k][j] = (uint8_t)found;
        }
    if (nu != kNU || rt.n_stats != kNQ) return hipErrorInvalidValue;
    hipLaunchKernelGGL(eval16_kernel, dim3((unsigned)R), dim3(kT), 0, st, (const __half*)x0,
                       (const __half*)x1, nb0, tb, D, H, stats, (WsHeader*)ws);
    return hipGetLastError();
}

}  // namespace kvq
