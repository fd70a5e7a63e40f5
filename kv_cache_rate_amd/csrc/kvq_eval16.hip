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
// sweep 2 (packed 16-bit counters, rows padded to 33 words so lanes reading
// different bins hit different LDS banks) plus totals of each run of 8 keys,
// and one lane per threshold finishes its prefix inside the bin in at most
// 8 + 4 steps.  Order statistics are therefore exact data values and every
// prefix is exact; only the final per-interval algebra rounds (fp64).
//
// Workgroup = one block, 256 threads x 16 entries kept in registers; the
// candidate phase maps one 16-lane row to one candidate so its totals are a
// row reduction.
#include <math.h>
#include <string.h>

#include "kvq_internal.h"

namespace kvq {

namespace {

constexpr int kT = 256;            // threads per block
constexpr int kPer = 16;           // entries per thread
constexpr int kNC = 1024;          // coarse bins
constexpr int kSlotStride = 33;    // 32 words of packed 16-bit counts + pad
constexpr int kGrpStride = 9;      // 8 group words + pad
constexpr int kMaxSlots = 144;     // every target and threshold bin fits
constexpr int kNU = 71;            // distinct interior uniform fractions, s = 16
constexpr int kNQ = 73;            // order statistics, s = 16, n = 4096
constexpr int kPS = kMaxS + 1;     // padded row of per-candidate arrays
constexpr int kSlots = kMaxCand * kMaxS;  // 464 (candidate, point) slots
constexpr uint16_t kNoSlot = 0xffff;
// point sources (per (candidate, point) slot)
constexpr uint16_t kSrcNone = 0xffff, kSrcMin = 0, kSrcMax = 1, kSrcUni = 0x100, kSrcQnt = 0x200;

struct PhaseA {                    // sweep 1 .. threshold search
    uint32_t cnt[kNC + 1];         // payload count | sum(f) << 13, then exclusive prefix counts
    double ps1[kNC + 1];           // exclusive prefix sums
};
struct PhaseB {                    // sweep 2 .. prefix finish
    uint32_t fine[kMaxSlots * kSlotStride];
    uint32_t grp[kMaxSlots * kGrpStride];  // count | sum(f within group) << 16
};
struct PhaseC {                    // candidate points and interval masses
    float pval[kMaxCand * kPS];
    uint32_t pcnt[kMaxCand * kPS];
    double ps1[kMaxCand * kPS];
    double ma[kMaxCand * kPS];
    double mb[kMaxCand * kPS];
};

struct Shared {
    union {
        PhaseA a;
        PhaseB b;
        PhaseC c;
    } u;
    uint16_t slot[kNC];            // resolved bin -> slot * kSlotStride, or kNoSlot
    uint16_t src[kSlots];          // point source of slot (c, j)
    uint16_t tbin[kNQ];
    uint16_t tloc[kNQ];
    float tval[kNQ];
    uint32_t tcnt[kNQ];
    double ts1[kNQ];
    uint16_t ukey[kNU];
    float uval[kNU];
    uint32_t ucnt[kNU];
    double us1[kNU];
    double lg_c[32];
    double lg_inv[32];
    uint32_t wmin[kT / 64], wmax[kT / 64], wamax[kT / 64];
    double wsq[kT / 64];
    uint32_t wtot[kT / 64];
    double wts1[kT / 64];
    int nslots;
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

// 1/x to ~1 ulp: hardware reciprocal estimate and two Newton steps.
__device__ __forceinline__ double recip(double x) {
    double r = __builtin_amdgcn_rcp(x);
    double e = fma(-x, r, 1.0);
    r = fma(r, e, r);
    e = fma(-x, r, 1.0);
    return fma(r, e, r);
}

// log2 of x in (0, 1], relative error ~1e-15: x = m 2^e with m in [1, 2);
// c = 1 + (2i + 1)/64 is the centre of the 1/32-wide cell of m, so
// log2 m = log2 c + log1p(t)/ln 2 with t = (m - c)/c, |t| < 1/64, and a
// degree-8 series for log1p.
__device__ __forceinline__ double log2_unit(double x, const double* lg_c, const double* lg_inv) {
    int e;
    double m = frexp(x, &e);  // [0.5, 1)
    m *= 2.0;
    e -= 1;
    const int i = (int)((__double_as_longlong(m) >> 47) & 31);
    const double c = 1.0 + (double)(2 * i + 1) * (1.0 / 64.0);
    const double t = (m - c) * lg_inv[i];
    double p = -1.0 / 8.0;
    p = fma(p, t, 1.0 / 7.0);
    p = fma(p, t, -1.0 / 6.0);
    p = fma(p, t, 1.0 / 5.0);
    p = fma(p, t, -1.0 / 4.0);
    p = fma(p, t, 1.0 / 3.0);
    p = fma(p, t, -1.0 / 2.0);
    p = fma(p, t, 1.0);
    const double l1p = p * t;
    return ((double)e + lg_c[i]) + l1p * 1.4426950408889634;  // 1/ln 2
}

}  // namespace

// Threshold tables from the host.
struct Eval16Tables {
    RankTable rt;
    uint8_t unum[kNU];              // numerator of distinct fraction u
    uint8_t uden[kNU];              // denominator
    uint16_t src[kSlots];           // point source of (candidate, point) slot
    double lg_c[32];                // log2(1 + (2i+1)/64)
    double lg_inv[32];              // 1 / (1 + (2i+1)/64)
};

__global__ void __launch_bounds__(kT)
eval16_kernel(const __half* __restrict__ x0, const __half* __restrict__ x1, int64_t nb0,
              Eval16Tables tb, double* __restrict__ Dout, double* __restrict__ Hout,
              float* __restrict__ stats, WsHeader* ws) {
    __shared__ Shared sh;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int64_t R = gridDim.x;
    const int64_t r = xcd_block(blockIdx.x, R);
    const __half* src = r < nb0 ? x0 + r * 4096 : x1 + (r - nb0) * 4096;

    // ---- load: thread owns entries [8 tid, 8 tid + 8) and [2048 + 8 tid, ...)
    uint32_t hw[8];
    {
        const uint4 a = reinterpret_cast<const uint4*>(src)[tid];
        const uint4 b = reinterpret_cast<const uint4*>(src)[256 + tid];
        hw[0] = a.x; hw[1] = a.y; hw[2] = a.z; hw[3] = a.w;
        hw[4] = b.x; hw[5] = b.y; hw[6] = b.z; hw[7] = b.w;
    }
    for (int i = tid; i < kNC; i += kT) sh.u.a.cnt[i] = 0u;
    for (int i = tid; i < kSlots; i += kT) sh.src[i] = tb.src[i];
    if (tid < 32) {
        sh.lg_c[tid] = tb.lg_c[tid];
        sh.lg_inv[tid] = tb.lg_inv[tid];
    }
    __syncthreads();

    // ---- sweep 1 (two entries per 32-bit word): canonical -0, keys,
    //      coarse histogram, min/max keys, max |bits|, sum of squares
    ushort2_t kmin2 = {0xffff, 0xffff}, kmax2 = {0, 0}, amax2 = {0, 0};
    double sq = 0.0;
    uint32_t keys2[kPer / 2];
#pragma unroll
    for (int p = 0; p < kPer / 2; ++p) {
        // x + (+0) maps -0 to +0 and leaves every other value (NaN stays NaN)
        half2_t hv = __builtin_bit_cast(half2_t, hw[p]) + (half2_t){(_Float16)0.0f, (_Float16)0.0f};
        const uint32_t w = __builtin_bit_cast(uint32_t, hv);
        const short2_t sg = __builtin_bit_cast(short2_t, w) >> (short2_t){15, 15};
        const uint32_t msk = (__builtin_bit_cast(uint32_t, sg) & 0x7fff7fffu) | 0x80008000u;
        const uint32_t k2 = w ^ msk;  // order-preserving keys of both halves
        keys2[p] = k2;
        const ushort2_t kv = __builtin_bit_cast(ushort2_t, k2);
        kmin2 = __builtin_elementwise_min(kmin2, kv);
        kmax2 = __builtin_elementwise_max(kmax2, kv);
        amax2 = __builtin_elementwise_max(amax2, __builtin_bit_cast(ushort2_t, w & 0x7fff7fffu));
        const double v0 = (double)(float)hv.x, v1 = (double)(float)hv.y;
        sq = fma(v0, v0, sq);
        sq = fma(v1, v1, sq);
        const uint32_t klo = k2 & 0xffffu, khi = k2 >> 16;
        atomicAdd(&sh.u.a.cnt[klo >> 6], 1u | ((klo & 63u) << 13));
        atomicAdd(&sh.u.a.cnt[khi >> 6], 1u | ((khi & 63u) << 13));
    }
    {
        const uint32_t kmin = wave_min_u32_dpp(min((uint32_t)kmin2.x, (uint32_t)kmin2.y));
        const uint32_t kmax = wave_max_u32_dpp(max((uint32_t)kmax2.x, (uint32_t)kmax2.y));
        const uint32_t amax = wave_max_u32_dpp(max((uint32_t)amax2.x, (uint32_t)amax2.y));
        const double sqw = wave_last_f64(wave_scan_add_f64(sq));
        if (lane == 0) {
            sh.wmin[wave] = kmin;
            sh.wmax[wave] = kmax;
            sh.wamax[wave] = amax;
            sh.wsq[wave] = sqw;
        }
    }
    __syncthreads();
    const uint32_t kmin = min(min(sh.wmin[0], sh.wmin[1]), min(sh.wmin[2], sh.wmin[3]));
    const uint32_t kmax = max(max(sh.wmax[0], sh.wmax[1]), max(sh.wmax[2], sh.wmax[3]));
    if (tid == 0 && max(max(sh.wamax[0], sh.wamax[1]), max(sh.wamax[2], sh.wamax[3])) >= 0x7c00u)
        atomicOr(&ws->status, kStatusNonFinite);
    const double sumsq = (sh.wsq[0] + sh.wsq[1]) + (sh.wsq[2] + sh.wsq[3]);
    const float mn = key_value(kmin);
    const float mx = key_value(kmax);

    // ---- coarse prefix: thread owns bins [4 tid, 4 tid + 4) (one binade,
    //      B_k = B0 + 64 k U), prefix counts written over the payloads
    {
        const uint32_t bin0 = 4 * tid;
        const float B0 = key_value(bin0 << 6);
        const double U = (double)(key_value((bin0 << 6) | 1u) - B0);
        uint32_t c[4], acc[4];
        uint32_t ct = 0, at = 0;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const uint32_t p = sh.u.a.cnt[bin0 + k];
            c[k] = p & 0x1fffu;
            acc[k] = 64u * (uint32_t)k * c[k] + (p >> 13);
            ct += c[k];
            at += acc[k];
        }
        // empty threads add exactly 0 (the Inf/NaN code bins have no finite base)
        const double st = ct ? (double)ct * (double)B0 + U * (double)at : 0.0;
        const uint32_t ic = wave_scan_add_u32(ct);
        const double is = wave_scan_add_f64(st);
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
        const uint32_t base_c = oc + ic - ct;
        const double base_s = os + (is - st);
        uint32_t runc = 0, runa = 0;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            sh.u.a.cnt[bin0 + k] = base_c + runc;
            sh.u.a.ps1[bin0 + k] = runc ? base_s + (double)runc * (double)B0 + U * (double)runa : base_s;
            runc += c[k];
            runa += acc[k];
            sh.slot[bin0 + k] = kNoSlot;
        }
        if (tid == kT - 1) {
            sh.u.a.cnt[kNC] = base_c + ct;
            sh.u.a.ps1[kNC] = base_s + st;
        }
    }
    __syncthreads();

    // ---- targets (order statistics) on threads 0..72, uniform thresholds on
    //      threads 128..198: find the bin, read its prefix, mark it
    const int nq = tb.rt.n_stats;  // 73
    if (tid < nq) {
        const uint32_t rank = (uint32_t)tb.rt.rank[tid];
        int lo = 0, hi = kNC - 1;  // last bin with prefix count <= rank
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (sh.u.a.cnt[mid] <= rank) lo = mid;
            else hi = mid - 1;
        }
        const uint32_t pc = sh.u.a.cnt[lo];
        sh.tbin[tid] = (uint16_t)lo;
        sh.tloc[tid] = (uint16_t)(rank - pc);
        sh.tcnt[tid] = pc;
        sh.ts1[tid] = sh.u.a.ps1[lo];
        sh.slot[lo] = 0;  // mark
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
        const uint32_t bin = key >> 6;
        sh.uval[u] = t;
        sh.ukey[u] = (uint16_t)key;
        sh.ucnt[u] = sh.u.a.cnt[bin];
        sh.us1[u] = sh.u.a.ps1[bin];
        sh.slot[bin] = 0;  // mark
    }
    const double total_s1 = sh.u.a.ps1[kNC];
    __syncthreads();
    // compact marked bins into slots (thread owns 4 bins); at most 73 + 71
    {
        uint32_t m4 = 0;
#pragma unroll
        for (int k = 0; k < 4; ++k) m4 += sh.slot[4 * tid + k] == 0 ? 1u : 0u;
        const uint32_t im = wave_scan_add_u32(m4);
        if (lane == 63) sh.wtot[wave] = im;
        __syncthreads();
        uint32_t o = 0;
        for (int w = 0; w < wave; ++w) o += sh.wtot[w];
        uint32_t s = o + im - m4;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int bin = 4 * tid + k;
            if (sh.slot[bin] == 0) sh.slot[bin] = (uint16_t)(kSlotStride * s++);
        }
        if (tid == kT - 1) sh.nslots = (int)s;
    }
    __syncthreads();
    const int nslots = sh.nslots;  // <= 144 = kMaxSlots
    for (int i = tid; i < nslots * kSlotStride; i += kT) sh.u.b.fine[i] = 0u;
    __syncthreads();

    // ---- sweep 2: per-key counts in resolved bins
#pragma unroll
    for (int p = 0; p < kPer / 2; ++p) {
#pragma unroll
        for (int hpart = 0; hpart < 2; ++hpart) {
            const uint32_t key = hpart ? keys2[p] >> 16 : keys2[p] & 0xffffu;
            const uint32_t sl = sh.slot[key >> 6];
            if (sl != kNoSlot)
                atomicAdd(&sh.u.b.fine[sl + ((key & 63u) >> 1)], 1u << ((key & 1u) * 16));
        }
    }
    __syncthreads();
    // group totals: 8 keys (4 words) per group, 8 groups per slot
    for (int g = tid; g < nslots * 8; g += kT) {
        const int s = g >> 3, gi = g & 7;
        const uint32_t* fw = &sh.u.b.fine[s * kSlotStride + 4 * gi];
        uint32_t cn = 0, fs = 0;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const uint32_t w = fw[q];
            const uint32_t c0 = w & 0xffffu, c1 = w >> 16;
            cn += c0 + c1;
            fs += (2 * q) * c0 + (2 * q + 1) * c1;
        }
        sh.u.b.grp[s * kGrpStride + gi] = cn | (fs << 16);
    }
    __syncthreads();

    // ---- finish the prefixes inside the bins
    if (tid < nq) {
        const uint32_t bin = sh.tbin[tid];
        const uint32_t sbase = sh.slot[bin];
        const uint32_t loc = sh.tloc[tid];
        const uint32_t* gw = &sh.u.b.grp[(sbase / kSlotStride) * kGrpStride];
        uint32_t N = 0, F1 = 0;
        int gi = 0;
        for (; gi < 7; ++gi) {
            const uint32_t g = gw[gi];
            const uint32_t gc = g & 0xffffu;
            if (N + gc > loc) break;
            N += gc;
            F1 += 8u * (uint32_t)gi * gc + (g >> 16);
        }
        const uint32_t* fw = &sh.u.b.fine[sbase + 4 * gi];
        uint32_t f = 8 * gi + 7;
        for (int q = 0; q < 4; ++q) {
            const uint32_t w = fw[q];
            const uint32_t c0 = w & 0xffffu, c1 = w >> 16;
            const uint32_t f0 = 8 * gi + 2 * q;
            if (N + c0 > loc) { f = f0; break; }
            N += c0;
            F1 += f0 * c0;
            if (N + c1 > loc) { f = f0 + 1; break; }
            N += c1;
            F1 += (f0 + 1) * c1;
        }
        const float B = key_value(bin << 6);
        const float U = key_value((bin << 6) | 1u) - B;
        sh.tval[tid] = key_value((bin << 6) | f);
        sh.tcnt[tid] += N;
        if (N) sh.ts1[tid] += (double)B * (double)N + (double)U * (double)F1;
    } else if (tid >= 128 && tid < 128 + kNU) {
        const int u = tid - 128;
        const uint32_t key = sh.ukey[u];
        const uint32_t bin = key >> 6;
        const uint32_t sbase = sh.slot[bin];
        const uint32_t fstop = key & 63u;
        const uint32_t* gw = &sh.u.b.grp[(sbase / kSlotStride) * kGrpStride];
        uint32_t N = 0, F1 = 0;
        const int gstop = (int)(fstop >> 3);
        for (int gi = 0; gi < gstop; ++gi) {
            const uint32_t g = gw[gi];
            const uint32_t gc = g & 0xffffu;
            N += gc;
            F1 += 8u * (uint32_t)gi * gc + (g >> 16);
        }
        const uint32_t* fw = &sh.u.b.fine[sbase + 4 * gstop];
        for (uint32_t f = 8u * gstop; f < fstop; ++f) {
            const uint32_t c = (fw[(f >> 1) - 4u * gstop] >> ((f & 1u) * 16)) & 0xffffu;
            N += c;
            F1 += f * c;
        }
        const float B = key_value(bin << 6);
        const float U = key_value((bin << 6) | 1u) - B;
        sh.ucnt[u] += N;
        if (N) sh.us1[u] += (double)B * (double)N + (double)U * (double)F1;
    }
    __syncthreads();  // phase-B storage is reused below

    // ---- order statistics out
    if (tid < nq) stats[tid * R + r] = sh.tval[tid];

    // ---- raw candidate points: slot (c, j), repeats kept
    PhaseC& pc = sh.u.c;
    for (int sl = tid; sl < kSlots; sl += kT) {
        const uint16_t sc = sh.src[sl];
        if (sc != kSrcNone) {
            float v;
            uint32_t cn;
            double s1;
            if (sc == kSrcMin) {
                v = mn; cn = 0; s1 = 0.0;
            } else if (sc == kSrcMax) {
                v = mx; cn = 4096; s1 = total_s1;
            } else if (sc < kSrcQnt) {
                const int u = sc - kSrcUni;
                v = sh.uval[u]; cn = sh.ucnt[u]; s1 = sh.us1[u];
            } else {
                const int q = sc - kSrcQnt;
                v = sh.tval[q]; cn = sh.tcnt[q]; s1 = sh.ts1[q];
            }
            const int i0 = (sl >> 4) * kPS + (sl & 15);
            pc.pval[i0] = v;
            pc.pcnt[i0] = cn;
            pc.ps1[i0] = s1;
        }
    }
    __syncthreads();
    // interval masses; an interval between two equal points carries the
    // entries equal to that point (possible only at the closed maximum)
    for (int sl = tid; sl < kSlots; sl += kT) {
        if ((sl & 15) < 15 && sh.src[sl + 1] != kSrcNone) {
            const int i0 = (sl >> 4) * kPS + (sl & 15);
            const double a = pc.pval[i0], b = pc.pval[i0 + 1];
            const double Cn = (double)(pc.pcnt[i0 + 1] - pc.pcnt[i0]);
            double mbv = Cn;
            if (b > a) {
                const double S1 = pc.ps1[i0 + 1] - pc.ps1[i0];
                mbv = (S1 - a * Cn) * recip(b - a);
                mbv = fmin(fmax(mbv, 0.0), Cn);
            }
            pc.mb[i0] = mbv;
            pc.ma[i0] = Cn - mbv;
        }
    }
    __syncthreads();
    // point terms, then one 16-lane row per candidate: D = sum q^2 M - sum x^2
    // and H = sum over distinct values of -pi log2 pi
#pragma unroll
    for (int round = 0; round < 2; ++round) {
        const int sl = tid + round * kT;
        const int c = sl >> 4, j = sl & 15;
        double qm = 0.0, hb = 0.0;
        if (sl < kSlots && sh.src[sl] != kSrcNone) {
            const int i0 = c * kPS + j;
            const bool has_right = j < 15 && sh.src[sl + 1] != kSrcNone;
            double M = 0.0;
            if (j > 0) M += pc.mb[i0 - 1];
            if (has_right) M += pc.ma[i0];
            const double q = pc.pval[i0];
            qm = q * q * M;
            if (j == 0 || pc.pval[i0 - 1] != pc.pval[i0]) {
                double Mv = M;
                for (int jj = j + 1; jj < 16 && sh.src[c * kMaxS + jj] != kSrcNone &&
                                     pc.pval[c * kPS + jj] == pc.pval[i0];
                     ++jj) {
                    Mv += pc.mb[c * kPS + jj - 1];
                    if (jj < 15 && sh.src[c * kMaxS + jj + 1] != kSrcNone) Mv += pc.ma[c * kPS + jj];
                }
                const double pi = Mv * (1.0 / 4096.0);
                if (pi > 0.0) hb = -pi * log2_unit(pi, sh.lg_c, sh.lg_inv);
            }
        }
        qm = row_sum_f64(qm);
        hb = row_sum_f64(hb);
        if (j == 15 && c < kMaxCand) {
            double Dc = 0.0, Hc = 0.0;
            if (mx > mn) {
                Dc = qm - sumsq;
                Hc = hb;
            }
            Dout[c * R + r] = fmax(Dc, 0.0);
            Hout[c * R + r] = fmax(Hc, 0.0);
        }
    }
}

hipError_t launch_eval16(const void* x0, const void* x1, int64_t nb0, int64_t R, const RankTable& rt,
                         double* D, double* H, float* stats, void* ws, hipStream_t st) {
    if (R == 0) return hipSuccess;
    Eval16Tables tb;
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
    // point sources: candidate 0 is {min, max}; then U_k, E_k for k = 3..16
    for (int c = 0; c < kMaxCand; ++c) {
        const int k = c == 0 ? 2 : 3 + (c - 1) / 2;
        const bool uni = c > 0 && ((c - 1) & 1) == 0;
        for (int j = 0; j < kMaxS; ++j) {
            uint16_t v = kSrcNone;
            if (j == 0) v = kSrcMin;
            else if (j == k - 1) v = kSrcMax;
            else if (j < k) v = uni ? (uint16_t)(kSrcUni + ucol[k][j]) : (uint16_t)(kSrcQnt + rt.col[k][j]);
            tb.src[c * kMaxS + j] = v;
        }
    }
    for (int i = 0; i < 32; ++i) {
        const double c = 1.0 + (double)(2 * i + 1) / 64.0;
        tb.lg_c[i] = log2(c);
        tb.lg_inv[i] = 1.0 / c;
    }
    hipLaunchKernelGGL(eval16_kernel, dim3((unsigned)R), dim3(kT), 0, st, (const __half*)x0,
                       (const __half*)x1, nb0, tb, D, H, stats, (WsHeader*)ws);
    return hipGetLastError();
}

}  // namespace kvq
