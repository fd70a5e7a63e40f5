// The global multiplier and each block's codebook (kvq_solve_lambda).
//
// Page "Rate-adaptive KV-cache quantizer", Key formulas (1)-(2): for a fixed
// lambda every block minimises D_r + lambda d_r H_r on its own, so the
// modelled rate R(lambda) = sum_r d_r H_r(choice_r(lambda)) is a sum of
// independent per-block terms; Key formulas (4) gives the projected
// subgradient step.  The bisection on lambda follows the page "Joint
// Tucker-rank and residual-bit KV allocator" (Mathematical statement).
//
// Device design: a "rates" pass evaluates R at up to 64 multipliers at once
// (one read of the score table per pass).  A one-thread "select" kernel then
// advances the bracket held in the workspace header, so the search runs with
// one host round trip (after lambda = 0, which is probed alone first: when it
// is feasible no further pass is launched):
//   pass 0: lambda in {2^0, ..., 2^62}; the first feasible power gives the
//           doubling bracket exactly as sequential doubling from [0, 1] would;
//   pass 1: {2^63, 2^64} only if none of those was feasible;
//   passes 2..: the 2^b - 1 interior points of a dyadic grid over the
//           bracket (b <= 6); the b halvings of sequential bisection are then
//           replayed on those values (every midpoint it would probe is one of
//           them, and all are exact in fp64), so 40 halvings take 7 passes
//           and give the same final bracket bit for bit.
// Rates are summed as unsigned fixed point (d_r H_r scaled by 2^shift and
// rounded), so the sum is exact and independent of summation order.
#include <algorithm>
#include <type_traits>

#include "kvq_internal.h"
#include "kvq_grid_choice.h"

namespace kvq {

constexpr int kSolveThreads = 256;
constexpr int kScanPer = 4;
constexpr int kScanTile = kSolveThreads * kScanPer;

enum Phase : int32_t {
    kPhaseDouble = 0, kPhaseDouble2 = 1, kPhaseMulti = 2, kPhaseZero = 3, kPhaseSubgrad = 10
};

__device__ __forceinline__ unsigned long long wave_sum_u64(unsigned long long v) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v += __shfl_down(v, off, 64);
    return v;
}

__global__ void solve_init_kernel(WsHeader* h, int mode, double lam_in, unsigned long long Btot_fx,
                                  int iters, int bits_max, int dbl_n) {
    for (int i = threadIdx.x; i < kMaxLam * kRateStripes; i += blockDim.x)
        h->rsum[i / kRateStripes][i % kRateStripes] = 0ull;
    for (int i = threadIdx.x; i < kRateStripes; i += blockDim.x) h->rate_part[i] = 0ull;
    if (threadIdx.x != 0) return;
    h->done = 0;
    h->err = 0;
    h->Btot_fx = Btot_fx;
    h->bits_left = iters;
    h->bits_max = bits_max;
    h->dbl_n = dbl_n;
    h->dbl_base = 0;
    h->rate_final = 0;
    for (int j = 0; j < kMaxLam + 8; ++j) h->sums[j] = 0ull;
    h->pool_n = 0;
    h->pool_overflow = 0;
    h->swaps = 0;
    if (mode == KVQ_SUBGRAD) {  // blocks are chosen at lam_in by the final pass
        h->phase = kPhaseSubgrad;
        h->nlam = 0;
        h->lam_final = lam_in;
        h->done = 1;
    } else {                    // first probe: lambda = 0 alone
        h->phase = kPhaseZero;
        h->nlam = 1;
        h->lam[0] = 0.0;
    }
}

__device__ void setup_multisection(WsHeader* h) {
    if (h->bits_left <= 0) {
        h->lam_final = h->hi;
        h->done = 1;
        h->nlam = 0;
        return;
    }
    const int b = h->bits_left < h->bits_max ? h->bits_left : h->bits_max;
    const int pts = (1 << b) - 1;
    const double lo = h->lo, width = h->hi - h->lo;
    for (int i = 1; i <= pts; ++i) h->lam[i - 1] = lo + (width * (double)i) / (double)(1 << b);
    h->bits_now = b;
    h->nlam = pts;
    h->phase = kPhaseMulti;
}

// rate_final += the final pass's striped rate sums (64 threads).
__global__ void fold_rate_kernel(WsHeader* h) {
    const int k = threadIdx.x;
    unsigned long long v = 0;
    if (k < kRateStripes) {
        v = h->rate_part[k];
        h->rate_part[k] = 0ull;
    }
    v = wave_sum_u64(v);
    if (k == 0) h->rate_final += v;
}

// 64 threads: lane j first folds multiplier j's rate stripes into sums[j]
// (every lane, whether or not the pass probed j or ran at all: unused
// stripes hold zeros, and the loads wait for nothing).
__global__ void solve_select_kernel(WsHeader* h) {
    static_assert(kMaxLam == 64, "one lane per multiplier");
    const int j = threadIdx.x;
    unsigned long long t = 0;
    for (int k = 0; k < kRateStripes; ++k) {
        t += h->rsum[j][k];
        h->rsum[j][k] = 0ull;
    }
    h->sums[j] += t;
    __syncthreads();
    if (threadIdx.x != 0 || h->done) return;
    const unsigned long long B = h->Btot_fx;
    switch (h->phase) {
    case kPhaseZero:
        if (h->sums[0] <= B) {
            h->lam_final = 0.0;
            h->done = 1;
        } else {  // bracket doubling: 2^0, 2^1, ... dbl_n per pass, up to 2^62
            h->phase = kPhaseDouble;
            h->dbl_base = 0;
            h->nlam = h->dbl_n;
            for (int j = 0; j < h->nlam; ++j) h->lam[j] = ldexp(1.0, j);
        }
        break;
    case kPhaseDouble: {
        int first = -1;
        for (int j = 0; j < h->nlam; ++j)
            if (h->sums[j] <= B) {
                first = j;
                break;
            }
        const int e0 = h->dbl_base;
        if (first >= 0) {
            h->hi = ldexp(1.0, e0 + first);
            h->lo = e0 + first == 0 ? 0.0 : ldexp(1.0, e0 + first - 1);
            setup_multisection(h);
        } else if (e0 + h->nlam < kMaxLam - 1) {  // next powers of two
            const int base = e0 + h->nlam;
            const int cnt = min(h->dbl_n, kMaxLam - 1 - base);
            h->dbl_base = base;
            h->nlam = cnt;
            for (int j = 0; j < cnt; ++j) h->lam[j] = ldexp(1.0, base + j);
        } else {
            h->phase = kPhaseDouble2;
            h->nlam = 2;
            h->lam[0] = ldexp(1.0, 63);
            h->lam[1] = ldexp(1.0, 64);
        }
        break;
    }
    case kPhaseDouble2:
        if (h->sums[0] <= B) {
            h->lo = ldexp(1.0, 62);
            h->hi = ldexp(1.0, 63);
            setup_multisection(h);
        } else if (h->sums[1] <= B) {
            h->lo = ldexp(1.0, 63);
            h->hi = ldexp(1.0, 64);
            setup_multisection(h);
        } else {
            h->err = KVQ_EINFEASIBLE;
            h->done = 1;
            h->nlam = 0;
        }
        break;
    case kPhaseMulti: {
        const int b = h->bits_now;
        int l = 0, u = 1 << b;
        for (int step = 0; step < b; ++step) {
            const int mid = (l + u) >> 1;
            if (h->sums[mid - 1] <= B) u = mid;
            else l = mid;
        }
        const double lo = h->lo, width = h->hi - h->lo;
        h->lo = lo + (width * (double)l) / (double)(1 << b);
        h->hi = lo + (width * (double)u) / (double)(1 << b);
        h->bits_left -= b;
        setup_multisection(h);
        break;
    }
    default:
        h->err = KVQ_EINVAL;
        h->done = 1;
    }
    for (int j = 0; j < kMaxLam + 8; ++j) h->sums[j] = 0ull;
}

// ---------------------------------------------------------------- grids ----

// kZero: the bisection's first pass, lambda = 0 alone (the host launches
// this instance for it and the general one for the others).
template <bool kZero>
__global__ void __launch_bounds__(kSolveThreads)
rates_grids_kernel(const double* __restrict__ D, const double* __restrict__ H,
                   const double* __restrict__ wgt, int64_t R, int C, double d, int shift,
                   WsHeader* h) {
    __shared__ unsigned long long part[kSolveThreads / 64][kMaxLam];
    const int nlam = h->nlam;
    if (h->done || nlam == 0) return;
    const int64_t r = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int wave = threadIdx.x >> 6;
    if constexpr (kZero) {
        // lambda = 0: the objective is the weighted D plus (+0) (0 H = +0 for
        // the finite, non-negative H), so only D is read for the choice and
        // H only at the chosen candidate
        unsigned long long v = 0;
        if (r < R) {
            const double wr = wgt ? wgt[r] : 1.0;
            double Dr[kMaxCand];
#pragma unroll
            for (int c = 0; c < kMaxCand; ++c) {
                // unconditional loads (candidate clamped into the table):
                // a load under the c < C condition was waited on by itself
                const double dv = D[(c < C ? c : C - 1) * R + r];
                Dr[c] = c < C ? wr * dv : 0.0;
            }
            double best = Dr[0] + 0.0;
            int bc = 0;
#pragma unroll
            for (int c = 1; c < kMaxCand; ++c) {
                if (c < C) {
                    const double o = Dr[c] + 0.0;
                    if (o < best) {
                        best = o;
                        bc = c;
                    }
                }
            }
            v = rate_fx(d, H[bc * R + r], shift);
        }
        v = wave_sum_u64(v);
        if ((threadIdx.x & 63) == 0) part[wave][0] = v;
        __syncthreads();
        if (threadIdx.x == 0) {
            unsigned long long t = 0;
            for (int w = 0; w < kSolveThreads / 64; ++w) t += part[w][0];
            atomicAdd(&h->rsum[0][blockIdx.x % kRateStripes], t);
        }
        return;
    } else {
    double Dr[kMaxCand], Hr[kMaxCand];
    if (r < R) {
        const double wr = wgt ? wgt[r] : 1.0;  // distortion weight (1: exact identity)
        // every load unconditional (candidate clamped into the table), so
        // all are in flight together; under the c < C condition each was
        // waited on by itself
#pragma unroll
        for (int c = 0; c < kMaxCand; ++c) {
            const int cc = c < C ? c : C - 1;
            Dr[c] = wr * D[cc * R + r];
            Hr[c] = H[cc * R + r];
        }
    }
    for (int j = 0; j < nlam; ++j) {
        unsigned long long v = 0;
        if (r < R) {
            const double lamd = h->lam[j] * d;
            double best = objective(Dr[0], Hr[0], lamd);
            double bh = Hr[0];
#pragma unroll
            for (int c = 1; c < kMaxCand; ++c) {
                if (c < C) {
                    const double o = objective(Dr[c], Hr[c], lamd);
                    if (o < best) {
                        best = o;
                        bh = Hr[c];
                    }
                }
            }
            v = rate_fx(d, bh, shift);
        }
        v = wave_sum_u64(v);
        if ((threadIdx.x & 63) == 0) part[wave][j] = v;
    }
    __syncthreads();
    for (int j = threadIdx.x; j < nlam; j += blockDim.x) {
        unsigned long long t = 0;
        for (int w = 0; w < kSolveThreads / 64; ++w) t += part[w][j];
        atomicAdd(&h->rsum[j][blockIdx.x % kRateStripes], t);
    }
    }
}

// One block's choice at multiplier lam (grid search) from its table row
// (Dv[c], Hv[c] for c < C, already loaded): candidate, codebook, levels and
// code words; returns the block's fixed-point rate.  Ties go to the lowest
// candidate index.
template <int kN>
__device__ __forceinline__ unsigned long long choose_grid_block(
    int64_t r, const double (&Dv)[kN], const double (&Hv)[kN], int C, double wr, double lamd, float mn,
    float mx, const float* __restrict__ stats, int64_t R, int s, int n, int shift, const uint8_t* col,
    int32_t* __restrict__ choice, float* __restrict__ codebook, uint8_t* __restrict__ m_out,
    uint64_t& words) {
    double best = 0.0, bestH = 0.0;
    int bc = -1;
#pragma unroll
    for (int c = 0; c < kN; ++c) {
        if (c < C) {
            const double o = objective(wr * Dv[c], Hv[c], lamd);
            if (bc < 0 || o < best) {
                best = o;
                bestH = Hv[c];
                bc = c;
            }
        }
    }
    const int m = write_grid_codebook(bc, mn, mx, stats + r, R, col, s, codebook + r * s);
    choice[r] = bc;
    m_out[r] = (uint8_t)m;
    words = ((uint64_t)n * (uint64_t)code_width(m) + 31u) / 32u;
    return rate_fx((double)n, bestH, shift);
}

// A block with no feasible multiplier: a well-formed empty result.
__device__ __forceinline__ void empty_grid_block(int64_t r, int s, int32_t* __restrict__ choice,
                                                 float* __restrict__ codebook, uint8_t* __restrict__ m_out) {
    choice[r] = -1;
    m_out[r] = 1;
    for (int j = 0; j < s; ++j) codebook[r * s + j] = 0.0f;
}

// The same, loading the table row in chunks of 15 candidates whose loads are
// in flight together (a loop bounded by the run-time C waits out one load
// latency per candidate).
template <bool kZero>  // the multiplier is 0
__device__ unsigned long long final_grid_block(int64_t r, const double* __restrict__ D,
                                               const double* __restrict__ H, const double* __restrict__ wgt,
                                               const float* __restrict__ stats, int64_t R, int C, int s,
                                               int n, int shift, const uint8_t* col, int n_stats,
                                               bool err, double lam,
                                               int32_t* __restrict__ choice, float* __restrict__ codebook,
                                               uint8_t* __restrict__ m_out, uint64_t& words) {
    if (err) {
        empty_grid_block(r, s, choice, codebook, m_out);
        words = 0;
        return 0;
    }
    const double wr = wgt ? wgt[r] : 1.0;
    const float mn = stats[r];
    const float mx = stats[(int64_t)(n_stats - 1) * R + r];
    if constexpr (kZero) {
        // the objective is the weighted D plus (+0) (0 H = +0 for the
        // finite, non-negative H): D is read for the choice, H only at the
        // chosen candidate, and the choice is choose_grid_block's
        double Dv[kMaxCand];
#pragma unroll
        for (int c = 0; c < kMaxCand; ++c) Dv[c] = c < C ? D[c * R + r] : 0.0;
        double best = 0.0;
        int bc = -1;
#pragma unroll
        for (int c = 0; c < kMaxCand; ++c) {
            if (c < C) {
                const double o = wr * Dv[c] + 0.0;
                if (bc < 0 || o < best) {
                    best = o;
                    bc = c;
                }
            }
        }
        const double Hc = H[bc * R + r];
        const int m = write_grid_codebook(bc, mn, mx, stats + r, R, col, s, codebook + r * s);
        choice[r] = bc;
        m_out[r] = (uint8_t)m;
        words = ((uint64_t)n * (uint64_t)code_width(m) + 31u) / 32u;
        return rate_fx((double)n, Hc, shift);
    } else {
    double Dv[kMaxCand], Hv[kMaxCand];
    constexpr int kChunk = 15;
#pragma unroll
    for (int c0 = 0; c0 < kMaxCand; c0 += kChunk) {
#pragma unroll
        for (int c = c0; c < c0 + kChunk && c < kMaxCand; ++c) {
            Dv[c] = c < C ? D[c * R + r] : 0.0;
            Hv[c] = c < C ? H[c * R + r] : 0.0;
        }
    }
    return choose_grid_block(r, Dv, Hv, C, wr, lam * (double)n, mn, mx, stats, R, s, n, shift, col, choice,
                             codebook, m_out, words);
    }
}

// kZero: the multiplier is 0 (the host knows it from the bisection's first
// pass).
template <bool kZero>
__global__ void __launch_bounds__(kSolveThreads)
final_grids_kernel(const double* __restrict__ D, const double* __restrict__ H,
                   const double* __restrict__ wgt, const float* __restrict__ stats, int64_t R,
                   int C, int s, int n, int shift,
                   RankTable rt, WsHeader* h, int32_t* __restrict__ choice,
                   float* __restrict__ codebook, uint8_t* __restrict__ m_out,
                   uint64_t* __restrict__ off) {
    __shared__ unsigned long long part[kSolveThreads / 64];
    __shared__ uint8_t col[(kMaxS + 1) * kMaxS];
    for (int i = threadIdx.x; i < (kMaxS + 1) * kMaxS; i += blockDim.x) col[i] = (&rt.col[0][0])[i];
    __syncthreads();
    const int64_t r = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (r == 0) off[0] = 0;
    unsigned long long v = 0;
    if (r < R) {
        uint64_t words;
        v = final_grid_block<kZero>(r, D, H, wgt, stats, R, C, s, n, shift, col, rt.n_stats, h->err != 0,
                             h->lam_final, choice, codebook, m_out, words);
        off[r + 1] = words;
    }
    v = wave_sum_u64(v);
    if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = v;
    __syncthreads();
    if (threadIdx.x == 0) {
        unsigned long long t = 0;
        for (int w = 0; w < kSolveThreads / 64; ++w) t += part[w];
        atomicAdd(&h->rate_part[blockIdx.x % kRateStripes], t);
    }
}

// ------------------------------------------------------------ exact DP ----

__device__ __forceinline__ double hbits(double p) { return p > 0.0 ? -p * log2(p) : 0.0; }

// Triples i < j < l of an M-point alphabet: those of pair (j, l) are
// i = 0 .. j - 1 from tri_base(j, l), pairs in their triangle order, so
// tri_base(j, l) = S(j) + j (l - j - 1) with S(j) = sum over j' < j of
// j' (M - 1 - j').
__host__ __device__ __forceinline__ int n_triples(int M) { return M * (M - 1) * (M - 2) / 6; }
__device__ __forceinline__ int tri_first(int j, int M) {
    return (M - 1) * j * (j - 1) / 2 - (j - 1) * j * (2 * j - 1) / 6;
}
__device__ __forceinline__ int tri_base(int j, int l, int M) { return tri_first(j, M) + j * (l - j - 1); }

constexpr int kDpThreads = 256;
// beam arrivals at one destination, (l - 1) width <= 30 x 8, over 64 lanes
constexpr int kArrivalsPerLane = ((kAlpha - 2) * kMaxBeam + 63) / 64;

// Pair-state dynamic program over the distinct alphabet A (m points, pairs
// indexed in the M-point triangle), one workgroup per (block, multiplier):
//   f_2[0][l]     = Dp(0,l) + w h(ML(0,l)/n)
//   f_{c+1}[j][l] = min_{i<j} (f_c[i][j] + Dp(j,l)) + w h((MR(i,j) + ML(j,l))/n)
//   best          = min over c, i of f_c[i][m-1] + w h(MR(i,m-1)/n)
// with w = lambda n and h(p) = -p log2 p: f_c[i][j] is the best cost of a
// chain from point 0 with c points ending in i < j, holding the distortion
// of its closed intervals and the entropy of every point before j (a
// point's frequency needs both neighbours).  Chains that reach the last
// point are complete.  Ties: lowest i, and across completions the smallest
// c, then the lowest i.  One thread per state (j, l) per layer, layers
// double-buffered in LDS; the chain's points ride along as a bitmask.
// LDS of one alphabet-search workgroup, carved from dynamic shared memory
// and sized by the alphabet (P pairs) and the beam width W (0: the DP):
//   Dp [P] (fp64)  pair distortions
//   DP:   hl, hr [P], h3 [T] (fp64)  entropy terms, independent of the
//         multiplier: h(ML(j,l)/n), h(MR(j,l)/n) and, for every triple
//         i < j < l, h((MR(i,j) + ML(j,l))/n) (T = M(M-1)(M-2)/6 triples,
//         those of pair (j, l) consecutive from tri_base(j, l));
//         f[2][P] (fp64), mk[2][P] (u32)       two layers of chain costs / masks
//   beam: ML, MR [P] (fp64) pair masses; cand[P][W] (fp64), g[2][M][W],
//         cnt[2][M]  arrivals and kept groups
//   A[M] (fp32) distinct alphabet, m (its size)
struct BeamEntry {
    double cost;
    uint32_t mask;   // the chain's points
    uint32_t prev;   // the point before the last
};

struct AlphaLds {
    double *Dp, *ML, *MR, *hl, *hr, *h3, *f, *cand;
    uint32_t* mk;
    BeamEntry* g;
    int* cnt;
    float* A;
    int* m;
};

// The DP keeps its entropy terms in tables while its LDS stays within
// kDpTableLds (at least five workgroups per CU); with larger alphabets
// (32 points: a 39.7 KB triple table, two workgroups per CU) and in the
// beam it evaluates them per transition.
constexpr size_t kDpTableLds = 32768;

__host__ __device__ inline size_t alpha_lds_layout(int M, int W, bool tab, AlphaLds* v, unsigned char* base) {
    const size_t P = (size_t)n_pairs(M);
    size_t o = 0;
    auto take = [&](size_t bytes) {
        const size_t at = o;
        o = (o + bytes + 15) & ~(size_t)15;
        return base ? base + at : nullptr;
    };
    AlphaLds t{};
    t.Dp = (double*)take(P * 8);
    if (tab) {
        t.hl = (double*)take(P * 8);
        t.hr = (double*)take(P * 8);
        t.h3 = (double*)take((size_t)n_triples(M) * 8 + 8);
    } else {
        t.ML = (double*)take(P * 8);
        t.MR = (double*)take(P * 8);
    }
    if (W == 0) {
        t.f = (double*)take(2 * P * 8);
        t.mk = (uint32_t*)take(2 * P * 4);
    } else {
        t.cand = (double*)take(P * (size_t)W * 8);
        t.g = (BeamEntry*)take(2 * (size_t)M * W * sizeof(BeamEntry));
        t.cnt = (int*)take(2 * (size_t)M * 4);
    }
    t.A = (float*)take((size_t)M * 4);
    t.m = (int*)take(4);
    if (v) *v = t;
    return o;
}

__host__ __device__ inline bool alpha_dp_tables(int M, int W) {
    return W == 0 && alpha_lds_layout(M, 0, true, nullptr, nullptr) <= kDpTableLds;
}
__host__ __device__ inline size_t alpha_lds_bytes(int M, int W, AlphaLds* v, unsigned char* base) {
    return alpha_lds_layout(M, W, alpha_dp_tables(M, W), v, base);
}

// Alphabet searches, one kernel instance each (their register needs
// differ): the beam, the DP evaluating its entropy terms per transition,
// the DP reading them from tables.
constexpr int kSearchBeam = 0, kSearchDp = 1, kSearchDpTables = 2;
inline int alpha_search_kind(int M, int W) {
    return W ? kSearchBeam : (alpha_dp_tables(M, W) ? kSearchDpTables : kSearchDp);
}

// Load one block's pair statistics and distinct alphabet into LDS.  The DP
// takes its entropy terms from tables: each point frequency's term depends
// on the point and its two neighbours only, not on the multiplier, so it is
// evaluated once per triple here instead of once per transition and layer.
__device__ void load_pairs(const AlphaLds& t, const double* __restrict__ Dg, const double* __restrict__ Mg,
                           const float* __restrict__ st, int M, int n) {
    const int P = n_pairs(M);
    const double dn = (double)n;
    for (int p = threadIdx.x; p < P; p += blockDim.x) {
        t.Dp[p] = Dg[p];
        if (t.h3) {
            t.hl[p] = hbits(Mg[2 * p] / dn);
            t.hr[p] = hbits(Mg[2 * p + 1] / dn);
        } else {
            t.ML[p] = Mg[2 * p];
            t.MR[p] = Mg[2 * p + 1];
        }
    }
    if (t.h3) {
        // triple x: find its middle point j (the S(j) it lies past), then
        // l and i; points at or past the distinct count m carry zero masses
        const int T = n_triples(M);
        for (int x = threadIdx.x; x < T; x += blockDim.x) {
            int j = 1, b = 0;
            while (x >= b + j * (M - 1 - j)) {
                b += j * (M - 1 - j);
                ++j;
            }
            const int li = (x - b) / j;
            const int i = x - b - li * j;
            const int l = j + 1 + li;
            t.h3[x] = hbits((Mg[2 * pair_index(i, j, M) + 1] + Mg[2 * pair_index(j, l, M)]) / dn);
        }
    }
    // distinct alphabet: the M order statistics are non-decreasing, so a
    // point is new unless it equals the one before; wave 0 keeps lane j's
    // point at the count of kept lanes below it (M <= 32)
    if (threadIdx.x < 64) {
        const int j = threadIdx.x;
        const float v = j < M ? st[j] : 0.0f;
        const float prev = __shfl_up(v, 1, 64);
        const bool keep = j < M && (j == 0 || v != prev);
        const unsigned long long kb = __ballot(keep);
        if (keep) t.A[__popcll(kb & ((1ull << j) - 1ull))] = v;
        if (j == 0) *t.m = __popcll(kb);
    }
}

// Pair index -> (j, l) of the M-point triangle.
__device__ __forceinline__ void pair_of(int p, int M, int& j, int& l) {
    j = 0;
    int rem = p;
    while (rem >= M - 1 - j) {
        rem -= M - 1 - j;
        ++j;
    }
    l = j + 1 + rem;
}

// The block's tables are in LDS (load_pairs, then a barrier).
template <bool tab>  // entropy terms from the tables (t.h3 set) or evaluated per transition
__device__ uint32_t dp_block(const AlphaLds& t, int M, int smax, int n, double w) {
    // each cost is formed as written, (f + D) + w h, each step rounded
#pragma clang fp contract(off)
    const int tid = threadIdx.x;
    const int P = n_pairs(M);
    const double dn = (double)n;
    const double INF = __builtin_huge_val();
    for (int p = tid; p < P; p += blockDim.x) {
        t.f[p] = INF;
        t.mk[p] = 0u;
    }
    __syncthreads();
    const int m = *t.m;
    if (m <= 1) return 1u;
    for (int l = 1 + tid; l < m; l += blockDim.x) {
        const int p = pair_index(0, l, M);
        t.f[p] = t.Dp[p] + w * (tab ? t.hl[p] : hbits(t.ML[p] / dn));
        t.mk[p] = 1u | (1u << l);
    }
    double best = INF;  // wave 0's running completion
    uint32_t best_mask = 0u;
    const int cmax = smax < m ? smax : m;
    int cur = 0;
    for (int c = 2;; ++c) {
        __syncthreads();
        const double* fc = t.f + cur * P;
        const uint32_t* mc = t.mk + cur * P;
        if (tid < 64) {
            // completions (i, m - 1): lane i scores its chain; the minimum
            // wins, ties to the lowest i
            double tot = INF;
            if (tid < m - 1) {
                const int p = pair_index(tid, m - 1, M);
                const double fv = fc[p];
                if (fv < INF) tot = fv + w * (tab ? t.hr[p] : hbits(t.MR[p] / dn));
            }
            double mn = tot;
            for (int o = 32; o > 0; o >>= 1) mn = fmin(mn, __shfl_xor(mn, o, 64));
            const unsigned long long hit = __ballot(tot == mn && mn < INF);
            if (mn < best && hit) {
                const int i = __ffsll((long long)hit) - 1;
                best = mn;
                best_mask = mc[pair_index(i, m - 1, M)];
            }
        }
        if (c >= cmax) break;
        const int nx = cur ^ 1;
        double* fn = t.f + nx * P;
        uint32_t* mn_ = t.mk + nx * P;
        // states (j, l): 1 <= j <= m - 2, j < l <= m - 1; every other entry
        // of the next layer is unreachable
        for (int p = tid; p < P; p += blockDim.x) {
            int j, l;
            pair_of(p, M, j, l);
            double bv = INF;
            uint32_t bm = 0u;
            if (j >= 1 && l < m) {
                const double Djl = t.Dp[p];
                const double* h3 = tab ? t.h3 + tri_base(j, l, M) : nullptr;
                const double MLjl = tab ? 0.0 : t.ML[p];
                for (int i = 0; i < j; ++i) {
                    const int q = pair_index(i, j, M);
                    const double fv = fc[q];
                    if (fv < INF) {
                        const double h = tab ? h3[i] : hbits((t.MR[q] + MLjl) / dn);
                        const double v = (fv + Djl) + w * h;
                        if (v < bv) {
                            bv = v;
                            bm = mc[q];
                        }
                    }
                }
            }
            fn[p] = bv;
            mn_[p] = bv < INF ? (bm | (1u << l)) : 0u;
        }
        cur = nx;
    }
    return best_mask;  // valid in wave 0
}

// a precedes b among chains of equal length: the lowest point where they
// differ belongs to a
__device__ __forceinline__ bool lex_before(uint32_t a, uint32_t b) {
    const uint32_t d = a ^ b;
    return (d & (0u - d) & a) != 0u;
}

// Beam search over ordered codepoints (the same partial cost as the DP):
// chains with the same number of points ending at the same codepoint
// compete, and only the `width` cheapest of each such group are extended,
// ties to the lexicographically smaller chain.  Chains reaching the last
// point are complete; the best completion wins, ties to the shorter, then
// the lexicographically smaller chain.
//   layer step: thread per (source group j, destination l > j) scores the
//   j-group's chains extended by l into cand; then every arrival counts
//   the arrivals at its destination that precede it and the `width` first
//   take the next layer's group; wave 0 picks the best completion
//   (destination m - 1).
__device__ uint32_t beam_block(const AlphaLds& t, int M, int smax, int width, int n, double w) {
    const int tid = threadIdx.x;
    const int P = n_pairs(M);
    const double dn = (double)n;
    const double INF = __builtin_huge_val();
    const int m = *t.m;
    if (m <= 1) return 1u;
    auto grp = [&](int layer, int l) { return t.g + ((size_t)layer * M + l) * width; };
    auto cnt = [&](int layer, int l) -> int& { return t.cnt[layer * M + l]; };
    // length 2: group l holds the chain (0, l); (0, m - 1) is complete
    for (int l = tid; l < m; l += blockDim.x) {
        cnt(0, l) = 0;
        if (l >= 1 && l < m - 1) {
            const int p = pair_index(0, l, M);
            grp(0, l)[0] = BeamEntry{t.Dp[p] + w * hbits(t.ML[p] / dn), 1u | (1u << l), 0u};
            cnt(0, l) = 1;
        }
    }
    // wave 0's running completion, starting from the chain (0, m - 1)
    double best;
    uint32_t best_mask;
    {
        const int p = pair_index(0, m - 1, M);
        best = (t.Dp[p] + w * hbits(t.ML[p] / dn)) + w * hbits(t.MR[p] / dn);
        best_mask = 1u | (1u << (m - 1));
    }
    const int cmax = smax < m ? smax : m;
    int cur = 0;
    for (int c = 2; c < cmax; ++c) {
        __syncthreads();
        // arrivals: chain b of group j extended by l
        for (int p = tid; p < P; p += blockDim.x) {
            int j, l;
            pair_of(p, M, j, l);
            if (j >= 1 && l < m) {
                const int nb = cnt(cur, j);
                const BeamEntry* gj = grp(cur, j);
                const double Djl = t.Dp[p], MLjl = t.ML[p];
                const double fin = l == m - 1 ? w * hbits(t.MR[p] / dn) : 0.0;
                for (int b = 0; b < nb; ++b) {
                    const BeamEntry e = gj[b];
                    const int q = pair_index((int)e.prev, j, M);
                    const double v = (e.cost + Djl) + w * hbits((t.MR[q] + MLjl) / dn);
                    t.cand[(size_t)p * width + b] = l == m - 1 ? v + fin : v;
                }
            }
        }
        __syncthreads();
        const int nx = cur ^ 1;
        // destinations l = 2 .. m - 2 keep their `width` cheapest arrivals
        // (ties: lexicographically smaller), one wave per destination: lane
        // q holds arrivals q, q + 64, ... (arrival x = chain x % width of
        // group 1 + x / width), and `width` rounds extract the wave minimum
        {
            const int lane = tid & 63, nw = (int)blockDim.x >> 6;
            for (int l = 2 + (tid >> 6); l < m - 1; l += nw) {
                double v[kArrivalsPerLane];
                uint32_t pm[kArrivalsPerLane], src[kArrivalsPerLane];
#pragma unroll
                for (int k = 0; k < kArrivalsPerLane; ++k) {
                    const int x = lane + 64 * k;
                    const int j = 1 + x / width, b = x - (j - 1) * width;
                    v[k] = INF;
                    pm[k] = 0u;
                    src[k] = 0u;
                    if (j < l && b < cnt(cur, j)) {
                        v[k] = t.cand[(size_t)pair_index(j, l, M) * width + b];
                        pm[k] = grp(cur, j)[b].mask;
                        src[k] = (uint32_t)j;
                    }
                }
                int kept = 0;
                for (int r = 0; r < width; ++r) {
                    // this lane's first remaining arrival in the order
                    double bv = INF;
                    uint32_t bm = 0u;
#pragma unroll
                    for (int k = 0; k < kArrivalsPerLane; ++k)
                        if (pm[k] != 0u && (v[k] < bv || (v[k] == bv && (bm == 0u || lex_before(pm[k], bm))))) {
                            bv = v[k];
                            bm = pm[k];
                        }
                    // the wave's first: the (cost, chain) order is strict
                    double wv = bv;
                    uint32_t wm = bm;
                    for (int o = 32; o > 0; o >>= 1) {
                        const double ov = __shfl_xor(wv, o, 64);
                        const uint32_t om = __shfl_xor(wm, o, 64);
                        if (om != 0u && (wm == 0u || ov < wv || (ov == wv && lex_before(om, wm)))) {
                            wv = ov;
                            wm = om;
                        }
                    }
                    if (wm == 0u) break;  // no arrival left
#pragma unroll
                    for (int k = 0; k < kArrivalsPerLane; ++k)
                        if (pm[k] == wm && v[k] == wv) {  // the holder records and drops it
                            grp(nx, l)[r] = BeamEntry{wv, wm | (1u << l), src[k]};
                            pm[k] = 0u;
                        }
                    ++kept;
                }
                if (lane == 0) cnt(nx, l) = kept;
            }
        }
        for (int l = tid; l < m; l += blockDim.x)
            if (l < 2 || l == m - 1) cnt(nx, l) = 0;
        // completions at the last point: lane j scores group j's chains,
        // then the wave keeps the cheapest (ties: lexicographically smaller)
        if (tid < 64) {
            double tot = INF;
            uint32_t tm = 0u;
            if (tid >= 1 && tid < m - 1) {
                const int nb = cnt(cur, tid);
                const BeamEntry* gj = grp(cur, tid);
                const double* cp = t.cand + (size_t)pair_index(tid, m - 1, M) * width;
                for (int b2 = 0; b2 < nb; ++b2) {
                    const double v = cp[b2];
                    const uint32_t mk = gj[b2].mask | (1u << (m - 1));
                    if (v < tot || (v == tot && lex_before(mk, tm))) {
                        tot = v;
                        tm = mk;
                    }
                }
            }
            for (int o = 32; o > 0; o >>= 1) {
                const double ot = __shfl_xor(tot, o, 64);
                const uint32_t om = __shfl_xor(tm, o, 64);
                if (ot < tot || (ot == tot && om != 0u && (tm == 0u || lex_before(om, tm)))) {
                    tot = ot;
                    tm = om;
                }
            }
            if (tm != 0u && (tot < best || (tot == best && __popc(tm) == __popc(best_mask) &&
                                            lex_before(tm, best_mask)))) {
                best = tot;
                best_mask = tm;
            }
        }
        cur = nx;
    }
    return best_mask;  // valid in wave 0
}

// Entropy (bits per entry) of the subset given by mask: each point's mass
// is what the interval on its left sends right plus what the interval on
// its right sends left.
__device__ double subset_entropy(const AlphaLds& t, int M, uint32_t mask, int n) {
    const int m = *t.m;
    int pts[kAlpha];
    int k = 0;
    for (int i = 0; i < m; ++i)
        if (mask & (1u << i)) pts[k++] = i;
    if (k <= 1) return 0.0;
    double Hs = 0.0;
    if (t.h3) {  // the DP's tables hold exactly these terms
        for (int q = 0; q < k; ++q)
            Hs += q == 0       ? t.hl[pair_index(pts[0], pts[1], M)]
                  : q == k - 1 ? t.hr[pair_index(pts[k - 2], pts[k - 1], M)]
                               : t.h3[tri_base(pts[q], pts[q + 1], M) + pts[q - 1]];
        return Hs;
    }
    for (int q = 0; q < k; ++q) {
        double mass = 0.0;
        if (q > 0) mass += t.MR[pair_index(pts[q - 1], pts[q], M)];
        if (q + 1 < k) mass += t.ML[pair_index(pts[q], pts[q + 1], M)];
        Hs += hbits(mass / (double)n);
    }
    return Hs;
}

// One search at multiplier w / n over the block whose tables load_pairs
// put in LDS (a barrier between; the previous search, if any, finished).
template <int kSearch>
__device__ __forceinline__ uint32_t alpha_search(const AlphaLds& t, int M, int smax, int width, int n, double w) {
    if constexpr (kSearch == kSearchBeam) return beam_block(t, M, smax, width, n, w);
    else return dp_block<kSearch == kSearchDpTables>(t, M, smax, n, w);
}

// Rate of every multiplier of the pass (up to 8 per doubling pass, one per
// bisection pass).  The DP with tables runs one workgroup per block, which
// loads the tables once and searches at the multipliers in turn: its
// searches are short and share the tables.  The others (each search costs
// far more than the load) run one workgroup per block and multiplier y.
// Width 0 runs the exact DP, else the beam.
template <int kSearch>
__global__ void __launch_bounds__(kDpThreads)
rates_alpha_kernel(const double* __restrict__ Dp, const double* __restrict__ Mlr,
                   const float* __restrict__ stats, int64_t R, int alpha_m, int smax, int width, int n,
                   int shift, WsHeader* h) {
    extern __shared__ __align__(16) unsigned char lds[];
    const int nlam = h->nlam;
    if (h->done || (int)blockIdx.y >= nlam) return;
    AlphaLds t;
    alpha_lds_bytes(alpha_m, width, &t, lds);
    const int64_t r = blockIdx.x;
    const int P = n_pairs(alpha_m);
    load_pairs(t, Dp + r * P, Mlr + r * P * 2, stats + r * alpha_m, alpha_m, n);
    auto search = [&](int j) {
        const double w = h->lam[j] * (double)n;
        const uint32_t mask = alpha_search<kSearch>(t, alpha_m, smax, width, n, w);
        if (threadIdx.x == 0) {
            const double Hs = subset_entropy(t, alpha_m, mask, n);
            atomicAdd(&h->rsum[j][blockIdx.x % kRateStripes], rate_fx((double)n, Hs, shift));
        }
    };
    if constexpr (kSearch == kSearchDpTables) {
        for (int j = 0; j < nlam; ++j) {
            __syncthreads();  // tables loaded; the previous search done with its layers
            search(j);
        }
    } else {  // one multiplier per workgroup (a loop here costs these kernels registers)
        __syncthreads();
        search(blockIdx.y);
    }
}

// The blocks' choice at the final multiplier: workgroup = block.
template <int kSearch>
__global__ void __launch_bounds__(kDpThreads)
final_alpha_kernel(const double* __restrict__ Dp, const double* __restrict__ Mlr,
                   const float* __restrict__ stats, int64_t R, int alpha_m, int smax, int width, int s,
                   int n, int shift, WsHeader* h, int32_t* __restrict__ choice, float* __restrict__ codebook,
                   uint8_t* __restrict__ m_out, uint64_t* __restrict__ off) {
    extern __shared__ __align__(16) unsigned char lds[];
    const int64_t r = blockIdx.x;
    const int tid = threadIdx.x;
    if (r == 0 && tid == 0) off[0] = 0;
    if (h->err) {
        if (tid == 0) {
            choice[r] = -1;
            m_out[r] = 1;
            off[r + 1] = 0;
        }
        for (int j = tid; j < s; j += blockDim.x) codebook[r * s + j] = 0.0f;
        return;
    }
    AlphaLds t;
    alpha_lds_bytes(alpha_m, width, &t, lds);
    const int P = n_pairs(alpha_m);
    const double w = h->lam_final * (double)n;
    load_pairs(t, Dp + r * P, Mlr + r * P * 2, stats + r * alpha_m, alpha_m, n);
    __syncthreads();
    const uint32_t mask = alpha_search<kSearch>(t, alpha_m, smax, width, n, w);
    if (tid == 0) {
        const double Hs = subset_entropy(t, alpha_m, mask, n);
        atomicAdd(&h->rate_part[blockIdx.x % kRateStripes], rate_fx((double)n, Hs, shift));
        const int m = *t.m;
        int k = 0;
        for (int i = 0; i < m; ++i)
            if (mask & (1u << i)) codebook[r * s + k++] = t.A[i];
        for (int j = k; j < s; ++j) codebook[r * s + j] = 0.0f;
        choice[r] = (int32_t)mask;
        m_out[r] = (uint8_t)k;
        off[r + 1] = ((uint64_t)n * (uint64_t)code_width(k) + 31u) / 32u;
    }
}

// --------------------------------------------------------- offsets scan ----

__device__ __forceinline__ uint64_t wave_incl_scan_u64(uint64_t v) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const uint64_t t = __shfl_up(v, o, 64);
        if (lane >= o) v += t;
    }
    return v;
}

// Block-wide inclusive scan of one value per thread; returns the inclusive
// value and the block total.
__device__ uint64_t block_incl_scan(uint64_t v, uint64_t& total) {
    __shared__ uint64_t wsum[kSolveThreads / 64];
    const uint64_t inc = wave_incl_scan_u64(v);
    const int wave = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 63) wsum[wave] = inc;
    __syncthreads();
    uint64_t pre = 0, tot = 0;
    for (int w = 0; w < kSolveThreads / 64; ++w) {
        if (w < wave) pre += wsum[w];
        tot += wsum[w];
    }
    __syncthreads();
    total = tot;
    return pre + inc;
}

// Inclusive scan of off[1..R] inside tiles of kScanTile entries.
__global__ void __launch_bounds__(kSolveThreads)
scan_tiles_kernel(uint64_t* off, int64_t R, uint64_t* tile_sums) {
    const int64_t base = (int64_t)blockIdx.x * kScanTile;
    uint64_t vals[kScanPer];
    uint64_t run = 0;
    for (int k = 0; k < kScanPer; ++k) {
        const int64_t i = base + threadIdx.x * kScanPer + k;
        vals[k] = i < R ? off[i + 1] : 0;
        run += vals[k];
        vals[k] = run;
    }
    uint64_t total;
    const uint64_t inc = block_incl_scan(run, total);
    const uint64_t pre = inc - run;
    for (int k = 0; k < kScanPer; ++k) {
        const int64_t i = base + threadIdx.x * kScanPer + k;
        if (i < R) off[i + 1] = pre + vals[k];
    }
    if (threadIdx.x == 0) tile_sums[blockIdx.x] = total;
}

// Exclusive scan of the tile sums (one workgroup, any count).
__global__ void __launch_bounds__(kSolveThreads)
scan_sums_kernel(uint64_t* tile_sums, int64_t T) {
    uint64_t carry = 0;
    for (int64_t base = 0; base < T; base += kSolveThreads) {
        const int64_t i = base + threadIdx.x;
        const uint64_t v = i < T ? tile_sums[i] : 0;
        uint64_t total;
        const uint64_t inc = block_incl_scan(v, total);
        if (i < T) tile_sums[i] = carry + inc - v;
        carry += total;
        __syncthreads();
    }
}

__global__ void __launch_bounds__(kSolveThreads)
scan_add_kernel(uint64_t* off, int64_t R, const uint64_t* tile_sums) {
    const int64_t tile = blockIdx.x;
    const uint64_t add = tile_sums[tile];
    for (int k = 0; k < kScanPer; ++k) {
        const int64_t i = tile * kScanTile + threadIdx.x * kScanPer + k;
        if (i < R) off[i + 1] += add;
    }
}

// ------------------------------------------------------- greedy fill ----
// Post-pass after bisection (page "Joint Tucker-rank and residual-bit KV
// allocator", Implementation notes: swap candidates with the best distortion
// reduction per added byte).  Bits are the fixed-point rates of the bisection
// (rate_fx), so the slack and every step are exact integers.

__device__ __forceinline__ double wdist(const double* D, const double* wgt, int64_t R, int64_t r, int c) {
    return (wgt ? wgt[r] : 1.0) * D[c * R + r];
}

// Every (block, candidate) upgrade that fits the slack left by the final
// pass (the slack only shrinks, so later steps draw from this pool).
__global__ void __launch_bounds__(kSolveThreads)
greedy_pool_kernel(const double* __restrict__ D, const double* __restrict__ H,
                   const double* __restrict__ wgt, int64_t R, int C, double d, int shift,
                   WsHeader* h, const int32_t* __restrict__ choice, uint2* __restrict__ pool) {
    const int64_t r = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (r >= R || h->err) return;
    const int cur = choice[r];
    if (cur < 0) return;
    const unsigned long long slack = h->Btot_fx - h->rate_final;
    const unsigned long long rc = rate_fx(d, H[cur * R + r], shift);
    const double dc = wdist(D, wgt, R, r, cur);
    for (int c = 0; c < C; ++c) {
        const unsigned long long rn = rate_fx(d, H[c * R + r], shift);
        if (rn > rc && rn - rc <= slack && dc - wdist(D, wgt, R, r, c) > 0.0) {
            const uint32_t i = atomicAdd(&h->pool_n, 1u);
            if (i < kGreedyPool) pool[i] = make_uint2((uint32_t)r, (uint32_t)c);
            else h->pool_overflow = 1u;
        }
    }
}

// Pools of up to this many upgrades take greedy_apply_fast_kernel.
constexpr int kGreedyFast = 1024;

// One workgroup applies upgrades one at a time: the best efficiency
// (D_cur - D_c) / (d H_c - d H_cur) among pool entries that still improve
// their block and fit; ties to the lowest block, then candidate.  The chosen
// block's codebook, level count and word count are rebuilt in place.
__global__ void __launch_bounds__(kSolveThreads)
greedy_apply_kernel(const double* __restrict__ D, const double* __restrict__ H,
                    const double* __restrict__ wgt, const float* __restrict__ stats, int64_t R,
                    int s, int n, int shift, RankTable rt, WsHeader* h, int32_t* choice,
                    float* __restrict__ codebook, uint8_t* __restrict__ m_out,
                    uint64_t* __restrict__ off, const uint2* __restrict__ pool) {
    __shared__ double be[kSolveThreads];
    __shared__ uint32_t bi[kSolveThreads];
    __shared__ unsigned long long slack;
    __shared__ int found;
    const int tid = threadIdx.x;
    if (h->err || h->pool_overflow) return;
    const uint32_t np = min(h->pool_n, kGreedyPool);
    if (np <= (uint32_t)kGreedyFast) return;  // greedy_apply_fast_kernel's
    const double d = (double)n;
    if (tid == 0) slack = h->Btot_fx - h->rate_final;
    __syncthreads();
    for (uint32_t step = 0; step < np * (uint32_t)kMaxCand; ++step) {
        double best = -1.0;
        uint32_t bidx = 0xffffffffu;
        for (uint32_t i = tid; i < np; i += kSolveThreads) {
            const uint2 e = pool[i];
            const int64_t r = e.x;
            const int c = (int)e.y;
            const int cur = __hip_atomic_load(&choice[r], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            const double hc = H[c * R + r], hu = H[cur * R + r];
            const unsigned long long rn = rate_fx(d, hc, shift), ru = rate_fx(d, hu, shift);
            const double dd = wdist(D, wgt, R, r, cur) - wdist(D, wgt, R, r, c);
            if (rn > ru && rn - ru <= slack && dd > 0.0) {
                const double eff = dd / (d * hc - d * hu);
                // larger efficiency first; then lower block, lower candidate
                const bool take = eff > best ||
                                  (eff == best && (r < (int64_t)pool[bidx].x ||
                                                   (r == (int64_t)pool[bidx].x && c < (int)pool[bidx].y)));
                if (take) {
                    best = eff;
                    bidx = i;
                }
            }
        }
        be[tid] = best;
        bi[tid] = bidx;
        __syncthreads();
        for (int w = kSolveThreads / 2; w > 0; w >>= 1) {
            if (tid < w) {
                const double eb = be[tid + w];
                const uint32_t ib = bi[tid + w];
                bool take = false;
                if (ib != 0xffffffffu) {
                    if (bi[tid] == 0xffffffffu || eb > be[tid]) {
                        take = true;
                    } else if (eb == be[tid]) {
                        const uint2 a = pool[bi[tid]], b = pool[ib];
                        take = b.x < a.x || (b.x == a.x && b.y < a.y);
                    }
                }
                if (take) {
                    be[tid] = eb;
                    bi[tid] = ib;
                }
            }
            __syncthreads();
        }
        if (tid == 0) {
            found = bi[0] != 0xffffffffu;
            if (found) {
                const uint2 e = pool[bi[0]];
                const int64_t r = e.x;
                const int c = (int)e.y;
                const int cur = __hip_atomic_load(&choice[r], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                const unsigned long long rn = rate_fx(d, H[c * R + r], shift);
                const unsigned long long ru = rate_fx(d, H[cur * R + r], shift);
                slack -= rn - ru;
                h->rate_final += rn - ru;
                h->swaps += 1u;
                __hip_atomic_store(&choice[r], c, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                const int m = write_grid_codebook(c, stats[r], stats[(int64_t)(rt.n_stats - 1) * R + r],
                                                  stats + r, R, &rt.col[0][0], s, codebook + r * s);
                m_out[r] = (uint8_t)m;
                off[r + 1] = ((uint64_t)n * (uint64_t)code_width(m) + 31u) / 32u;
            }
        }
        __threadfence();
        __syncthreads();
        if (!found) break;
    }
}

// The same greedy fill for pools of up to kGreedyFast upgrades by one wave
// with the pool in registers: lane l holds entries l, l + 64, ... of the
// pool ordered by (block, candidate).  Each step every lane scores its
// entries against their blocks' current choices and the remaining slack,
// the wave takes the best by (efficiency, lower entry index, i.e. lower
// block, then candidate), and the entries of the upgraded block take the
// winner's values as their block's current ones.  No barrier is needed, and
// the choices, rates and steps are those of greedy_apply_kernel (which took
// 2.6 ms for the 444 upgrades of the long-context cache at 1.5 bits per
// entry, scanning the pool in memory once per step).  Codebooks, levels and
// word counts of the upgraded blocks are written once at the end.
constexpr int kGreedyPer = kGreedyFast / 64;

// Wave maximum of v (every lane gets it): DPP steps within rows, then
// across rows, the result read from lane 63.
__device__ __forceinline__ unsigned long long wave_max_u64_dpp(unsigned long long v) {
#define KVQ_MAX64_STEP(CTRL, MASK)                                   \
    {                                                                \
        const unsigned long long t = dpp_u64<CTRL, MASK>(0ull, v);   \
        v = t > v ? t : v;                                           \
    }
    KVQ_MAX64_STEP(kDppRowShr1, 0xF)
    KVQ_MAX64_STEP(kDppRowShr2, 0xF)
    KVQ_MAX64_STEP(kDppRowShr4, 0xF)
    KVQ_MAX64_STEP(kDppRowShr8, 0xF)
    KVQ_MAX64_STEP(kDppBcast15, 0xA)
    KVQ_MAX64_STEP(kDppBcast31, 0xC)
#undef KVQ_MAX64_STEP
    const uint32_t lo = __builtin_amdgcn_readlane((uint32_t)v, 63);
    const uint32_t hi = __builtin_amdgcn_readlane((uint32_t)(v >> 32), 63);
    return ((unsigned long long)hi << 32) | lo;
}

__global__ void __launch_bounds__(64)
greedy_apply_fast_kernel(const double* __restrict__ D, const double* __restrict__ H,
                         const double* __restrict__ wgt, const float* __restrict__ stats, int64_t R,
                         int s, int n, int shift, RankTable rt, WsHeader* h, int32_t* choice,
                         float* __restrict__ codebook, uint8_t* __restrict__ m_out,
                         uint64_t* __restrict__ off, const uint2* __restrict__ pool) {
    __shared__ uint64_t sorted[kGreedyFast];
    __shared__ double ent_h[kGreedyFast];   // each entry's H and weighted D, read when it wins
    __shared__ double ent_d[kGreedyFast];
    const int lane = threadIdx.x;
    if (h->err || h->pool_overflow) return;
    const uint32_t np = h->pool_n;
    if (np == 0 || np > (uint32_t)kGreedyFast) return;  // larger pools: greedy_apply_kernel
    const double d = (double)n;
    // the pool ordered by (block, candidate)
    for (int i = lane; i < kGreedyFast; i += 64)
        sorted[i] = i < (int)np ? ((uint64_t)pool[i].x << 8 | pool[i].y) : ~0ull;
    __syncthreads();
    for (int k = 2; k <= kGreedyFast; k <<= 1) {
        for (int j = k >> 1; j > 0; j >>= 1) {
            for (int t = lane; t < kGreedyFast; t += 64) {
                const int p = t ^ j;
                if (p > t) {
                    const uint64_t a = sorted[t], b = sorted[p];
                    if ((a > b) == ((t & k) == 0)) {
                        sorted[t] = b;
                        sorted[p] = a;
                    }
                }
            }
            __syncthreads();
        }
    }
    int64_t r[kGreedyPer];
    int c[kGreedyPer], cur[kGreedyPer];
    double hc[kGreedyPer], dcv[kGreedyPer], hu[kGreedyPer], du[kGreedyPer];
    unsigned long long rc[kGreedyPer], ru[kGreedyPer];
#pragma unroll
    for (int k = 0; k < kGreedyPer; ++k) {
        const int i = lane + 64 * k;
        const bool live = i < (int)np;
        r[k] = live ? (int64_t)(sorted[i] >> 8) : -1;
        c[k] = live ? (int)(sorted[i] & 0xffu) : 0;
        cur[k] = live ? choice[r[k]] : 0;
        hc[k] = live ? H[c[k] * R + r[k]] : 0.0;
        dcv[k] = live ? wdist(D, wgt, R, r[k], c[k]) : 0.0;
        hu[k] = live ? H[cur[k] * R + r[k]] : 0.0;
        du[k] = live ? wdist(D, wgt, R, r[k], cur[k]) : 0.0;
        rc[k] = rate_fx(d, hc[k], shift);
        ru[k] = rate_fx(d, hu[k], shift);
        ent_h[i] = hc[k];
        ent_d[i] = dcv[k];
    }
    int cur0[kGreedyPer];
#pragma unroll
    for (int k = 0; k < kGreedyPer; ++k) cur0[k] = cur[k];
    __syncthreads();
    // each entry's efficiency against its block's current choice (0 where it
    // is no upgrade); it changes only when its block is upgraded.  Positive
    // doubles order as their bit patterns, so the best entry is the maximum
    // of (efficiency bits), then the lowest index among equal ones.
    unsigned long long ekey[kGreedyPer];
#pragma unroll
    for (int k = 0; k < kGreedyPer; ++k) {
        const bool up = r[k] >= 0 && rc[k] > ru[k] && du[k] - dcv[k] > 0.0;
        ekey[k] = up ? (unsigned long long)__double_as_longlong((du[k] - dcv[k]) / (d * hc[k] - d * hu[k])) : 0ull;
    }
    unsigned long long slack = h->Btot_fx - h->rate_final;
    unsigned long long added = 0;
    uint32_t swaps = 0;
    // the steps, compiled for the first K register slots: a pool of np
    // entries fills slots k < ceil(np / 64), the rest hold no entry, and a
    // step's cost grows with the slots it scans (0.59 ms for the long-
    // context cache's 444 upgrades scanning 16 slots, 0.33 ms scanning 8)
    auto steps = [&](auto kc) {
    constexpr int K = decltype(kc)::value;
    for (uint32_t step = 0; step < np * (uint32_t)kMaxCand; ++step) {
        unsigned long long best = 0;
        uint32_t bidx = 0xffffffffu;
#pragma unroll
        for (int k = 0; k < K; ++k) {
            const unsigned long long key = rc[k] - ru[k] <= slack ? ekey[k] : 0ull;
            if (key > best) {  // entries of a lane rise in index with k: the first of equals stays
                best = key;
                bidx = (uint32_t)(lane + 64 * k);
            }
        }
        const unsigned long long top = wave_max_u64_dpp(best);
        if (top == 0ull) break;
        const uint32_t idx = wave_min_u32_dpp(best == top ? bidx : 0xffffffffu);
        const int wl = (int)(idx & 63u), wk_slot = (int)(idx >> 6);
        const uint64_t wk = sorted[idx];
        const int64_t wr = (int64_t)(wk >> 8);
        const int wc = (int)(wk & 0xffu);
        const double wh = ent_h[idx], wd = ent_d[idx];
        const unsigned long long wrt = rate_fx(d, wh, shift);
        // the step's bits: the winner's rate over its block's current one
        unsigned long long wru = 0;
#pragma unroll
        for (int k = 0; k < K; ++k)
            if (k == wk_slot) wru = ru[k];
        const uint32_t wru_lo = __builtin_amdgcn_readlane((uint32_t)wru, wl);
        const uint32_t wru_hi = __builtin_amdgcn_readlane((uint32_t)(wru >> 32), wl);
        const unsigned long long bits = wrt - (((unsigned long long)wru_hi << 32) | wru_lo);
        slack -= bits;
        added += bits;
        ++swaps;
#pragma unroll
        for (int k = 0; k < K; ++k) {
            if (r[k] == wr) {  // the upgraded block's entries take the winner's values
                cur[k] = wc;
                hu[k] = wh;
                du[k] = wd;
                ru[k] = wrt;
                const bool up = rc[k] > ru[k] && du[k] - dcv[k] > 0.0;
                ekey[k] = up ? (unsigned long long)__double_as_longlong((du[k] - dcv[k]) / (d * hc[k] - d * hu[k]))
                             : 0ull;
            }
        }
    }
    };
    const uint32_t kn = (np + 63u) >> 6;  // wave-uniform
    if (kn <= 2)
        steps(std::integral_constant<int, 2>{});
    else if (kn <= 4)
        steps(std::integral_constant<int, 4>{});
    else if (kn <= 8)
        steps(std::integral_constant<int, 8>{});
    else
        steps(std::integral_constant<int, kGreedyPer>{});
    // the upgraded blocks: the entry of the final choice writes its block's
    // choice, codebook, levels and word count
#pragma unroll
    for (int k = 0; k < kGreedyPer; ++k) {
        if (r[k] >= 0 && cur[k] != cur0[k] && c[k] == cur[k]) {
            choice[r[k]] = cur[k];
            const int m = write_grid_codebook(cur[k], stats[r[k]], stats[(int64_t)(rt.n_stats - 1) * R + r[k]],
                                              stats + r[k], R, &rt.col[0][0], s, codebook + r[k] * s);
            m_out[r[k]] = (uint8_t)m;
            off[r[k] + 1] = ((uint64_t)n * (uint64_t)code_width(m) + 31u) / 32u;
        }
    }
    if (lane == 0) {
        h->rate_final += added;
        h->swaps += swaps;
    }
}

// ----------------------------------------------------------------- host ----

// Up to kSmallR blocks (grid search; a decode step): the final choice in
// one 64-thread workgroup per 64 blocks, then one workgroup for the scan of
// the code words, the rate sum and the header.  The choice is a chain of
// dependent memory round trips over a table just written on every XCD, so
// each thread first issues all of its block's table loads and the column
// table is copied to LDS while they are in flight; the codepoints'
// statistics are then gathered in one batch.  Spreading the blocks over
// workgroups (CUs) matters: one workgroup for 512 blocks spent 15 us in its
// CU's memory pipeline on the scattered gathers and row stores.
constexpr int kSmallR = 1024;
constexpr int kSmallWG = 64;
static_assert(kSmallR / kSmallWG <= 16, "WsHeader::part_rate holds one entry per workgroup");

__global__ void __launch_bounds__(kSmallWG)
final_grids_rows_kernel(const double* __restrict__ D, const double* __restrict__ H,
                        const double* __restrict__ wgt, const float* __restrict__ stats, int64_t R, int C,
                        int s, int n, int shift, RankTable rt, WsHeader* h, int subgrad, double lam_in,
                        int32_t* __restrict__ choice, float* __restrict__ codebook,
                        uint8_t* __restrict__ m_out, uint64_t* __restrict__ off) {
    __shared__ uint8_t col[(kMaxS + 1) * kMaxS];
    const int lane = threadIdx.x;
    const bool err = subgrad ? false : h->err != 0;
    const double lam = subgrad ? lam_in : h->lam_final;
    const int64_t r = (int64_t)blockIdx.x * kSmallWG + lane;
    const bool live = r < R;
    double Dv[kMaxCand], Hv[kMaxCand];
    float mn = 0.0f, mx = 0.0f;
    double wr = 1.0;
    if (live && !err) {
        wr = wgt ? wgt[r] : 1.0;
        mn = stats[r];
        mx = stats[(int64_t)(rt.n_stats - 1) * R + r];
#pragma unroll
        for (int c = 0; c < kMaxCand; ++c) {
            Dv[c] = c < C ? D[c * R + r] : 0.0;
            Hv[c] = c < C ? H[c * R + r] : 0.0;
        }
    }
    for (int i = lane; i < (kMaxS + 1) * kMaxS; i += kSmallWG) col[i] = (&rt.col[0][0])[i];
    __syncthreads();
    unsigned long long v = 0;
    if (live) {
        uint64_t words = 0;
        if (err) {
            empty_grid_block(r, s, choice, codebook, m_out);
        } else {
            v = choose_grid_block(r, Dv, Hv, C, wr, lam * (double)n, mn, mx, stats, R, s, n, shift, col, choice,
                                  codebook, m_out, words);
        }
        off[r + 1] = words;  // the scan kernel turns these into offsets
    }
    v = wave_sum_u64(v);
    if (lane == 0) h->part_rate[blockIdx.x] = v;
}

// The offsets scan (R <= kSmallR, one thread per block), the rate sum and
// the header; in the subgradient mode also the header set-up of
// solve_init_kernel.  If `out` is given, the fields the host reads go
// straight into its pinned buffer.
__global__ void __launch_bounds__(kSmallR)
final_grids_tail_kernel(int64_t R, WsHeader* h, int subgrad, double lam_in, uint64_t* __restrict__ off,
                        SolveOut* out) {
    __shared__ uint64_t wsum[kSmallR / 64];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const uint64_t words = tid < R ? off[tid + 1] : 0u;
    const int nwg = (int)((R + kSmallWG - 1) / kSmallWG);
    const uint64_t pr = tid < nwg ? h->part_rate[tid] : 0u;
    const uint64_t inc = wave_incl_scan_u64(words);
    if (lane == 63) wsum[wave] = inc;
    __syncthreads();
    uint64_t pre = 0;
    for (int w = 0; w < wave; ++w) pre += wsum[w];
    if (tid < R) off[tid + 1] = pre + inc;
    if (wave == 0) {
        const unsigned long long t = wave_sum_u64(pr);  // nwg <= 16 workgroups: wave 0 holds them all
        if (lane == 0) {
            off[0] = 0;
            if (subgrad) {
                h->phase = kPhaseSubgrad;
                h->nlam = 0;
                h->done = 1;
                h->err = 0;
                h->lam_final = lam_in;
                h->pool_n = 0;
                h->pool_overflow = 0;
                h->swaps = 0;
            }
            h->rate_final = t;
            if (out) {
                SolveOut o;
                o.status = h->status;
                o.err = subgrad ? 0 : h->err;
                o.pool_overflow = 0u;
                o.pad = 0u;
                o.lam_final = subgrad ? lam_in : h->lam_final;
                o.rate_final = t;
                *out = o;
                __threadfence_system();
            }
        }
    }
}

// Launch the two kernels of the few-block final pass.
static void launch_final_small(const kvq_plan& p, const RankTable& rt, const double* D, const double* H,
                               const double* wgt, const float* stats, int64_t R, int n, int shift, WsHeader* h,
                               int subgrad, double lam_in, int32_t* choice, float* codebook, uint8_t* m,
                               uint64_t* off, SolveOut* out, hipStream_t st) {
    const unsigned wgs = (unsigned)((R + kSmallWG - 1) / kSmallWG);
    hipLaunchKernelGGL(final_grids_rows_kernel, dim3(wgs), dim3(kSmallWG), 0, st, D, H, wgt, stats, R,
                       p.n_cand, p.s, n, shift, rt, h, subgrad, lam_in, choice, codebook, m, off);
    const unsigned threads = (unsigned)((R + 63) / 64 * 64);
    hipLaunchKernelGGL(final_grids_tail_kernel, dim3(1), dim3(threads), 0, st, R, h, subgrad, lam_in, off, out);
}

hipError_t launch_solve(const kvq_plan& p, const RankTable& rt, const double* D, const double* H,
                        const double* wgt, const float* stats, double B, int mode, int iters,
                        double lam_in,
                        int32_t* choice, float* codebook, uint8_t* m, uint64_t* off, void* ws,
                        SolveOut* out, bool* direct, hipStream_t st, bool staging) {
    WsHeader* h = (WsHeader*)ws;
    *direct = false;
    const int64_t R = p.n_blocks;
    const int n = p.d_block;
    const int shift = p.rate_shift;
    const double Btot = B * (double)p.n_entries;
    const double Bfx = ldexp(Btot, shift);
    const unsigned long long Btot_fx =
        Bfx >= 18446744073709551615.0 ? ~0ull : (unsigned long long)floor(Bfx);
    // Multipliers per pass (every split gives the same bisection).  A grid
    // search over fewer than kManyBlocks blocks pays about a launch per pass
    // whatever it probes, so it takes 6 halvings (63 multipliers, and all 63
    // doubling probes) per pass.  Over more, the objective evaluations
    // dominate (on 524288 blocks a 63-multiplier pass took 230 us, a
    // one-multiplier pass 68), so it takes 4 halvings (15 multipliers) and 7
    // doubling probes per pass: 1.33 ms against 2.16 ms for the B = 1.5
    // bisection there.  The alphabet searches cost a dynamic program per
    // block and multiplier, so they take one halving (and 8 doubling
    // probes) per pass.
    const bool grids = p.search == KVQ_GRIDS;
    const bool many = R >= kManyBlocks;
    const int bits_max = grids ? (many ? 4 : 6) : 1;
    const int dbl_n = grids ? (many ? 7 : kMaxLam - 1) : kAlphaLam;
    // few blocks (a decode step): choice, rate and offsets in two small
    // launches (launch_final_small), the result written to `out`
    const bool small = grids && R >= 1 && R <= kSmallR && mode != KVQ_BISECT_GREEDY;

    if (small && mode == KVQ_SUBGRAD) {
        launch_final_small(p, rt, D, H, wgt, stats, R, n, shift, h, 1, lam_in, choice, codebook, m, off, out, st);
        *direct = out != nullptr;
        return hipGetLastError();
    }
    hipLaunchKernelGGL(solve_init_kernel, dim3(1), dim3(64), 0, st, h, mode, lam_in, Btot_fx, iters,
                       bits_max, dbl_n);
    const int width = p.search == KVQ_BEAM ? p.beam_width : 0;
    const size_t alpha_lds = grids ? 0 : alpha_lds_bytes(p.alphabet_m, width, nullptr, nullptr);
    const int kind = grids ? kSearchDp : alpha_search_kind(p.alphabet_m, width);
    const unsigned grid = (unsigned)((R + kSolveThreads - 1) / kSolveThreads);
    // exact DP: one thread per pair state, in whole waves
    const int dp_pairs = p.search != KVQ_GRIDS ? n_pairs(p.alphabet_m) : 0;
    const int dp_waves = (dp_pairs + 63) / 64;
    const unsigned dp_threads = dp_waves < 1 ? 64u : (dp_waves > kDpThreads / 64 ? (unsigned)kDpThreads
                                                                                : 64u * dp_waves);
    auto rates_pass = [&](bool zero) {
        if (p.search == KVQ_GRIDS) {
            hipLaunchKernelGGL(zero ? rates_grids_kernel<true> : rates_grids_kernel<false>, dim3(grid),
                               dim3(kSolveThreads), 0, st, D, H, wgt, R, p.n_cand, (double)n, shift, h);
        } else {
            const auto k = kind == kSearchBeam ? rates_alpha_kernel<kSearchBeam>
                         : kind == kSearchDp   ? rates_alpha_kernel<kSearchDp>
                                               : rates_alpha_kernel<kSearchDpTables>;
            const unsigned ys = kind == kSearchDpTables ? 1u : (unsigned)kAlphaLam;
            hipLaunchKernelGGL(k, dim3((unsigned)R, ys), dim3(dp_threads), alpha_lds,
                               st, D, H, stats, R, p.alphabet_m, p.s, width, n, shift, h);
        }
        hipLaunchKernelGGL(solve_select_kernel, dim3(1), dim3(64), 0, st, h);
    };
    bool lam_zero = false;  // the final multiplier is known to be 0
    if (mode == KVQ_BISECT || mode == KVQ_BISECT_GREEDY) {
        // lambda = 0 first; the bracket passes run only when it is infeasible
        rates_pass(true);
        int32_t done = 0;
        const hipError_t e = read_back(&done, &h->done, sizeof done, st, staging);
        if (e != hipSuccess) return e;
        lam_zero = done != 0;
        if (!done) {
            // doubling passes up to 2^62, the 2^63 / 2^64 pass if needed,
            // then multisection passes of up to bits_max halvings each;
            // passes after the bracket is closed return at once
            const int passes = (kMaxLam - 1 + dbl_n - 1) / dbl_n + 1 + (iters + bits_max - 1) / bits_max;
            for (int ps = 0; ps < passes; ++ps) rates_pass(false);
        }
    }
    if (small) {
        launch_final_small(p, rt, D, H, wgt, stats, R, n, shift, h, 0, 0.0, choice, codebook, m, off, out, st);
        *direct = out != nullptr;
        return hipGetLastError();
    }
    if (p.search == KVQ_GRIDS) {
        hipLaunchKernelGGL(lam_zero ? final_grids_kernel<true> : final_grids_kernel<false>, dim3(grid),
                           dim3(kSolveThreads), 0, st, D, H, wgt, stats, R, p.n_cand, p.s, n, shift, rt, h,
                           choice, codebook, m, off);
    } else {
        const auto k = kind == kSearchBeam ? final_alpha_kernel<kSearchBeam>
                     : kind == kSearchDp   ? final_alpha_kernel<kSearchDp>
                                           : final_alpha_kernel<kSearchDpTables>;
        hipLaunchKernelGGL(k, dim3((unsigned)R), dim3(dp_threads), alpha_lds, st, D, H,
                           stats, R, p.alphabet_m, p.s, width, p.s, n, shift, h, choice, codebook, m, off);
    }
    hipLaunchKernelGGL(fold_rate_kernel, dim3(1), dim3(64), 0, st, h);
    if (mode == KVQ_BISECT_GREEDY && p.search == KVQ_GRIDS) {
        uint2* pool = (uint2*)((char*)ws + ws_pool_offset(R));
        hipLaunchKernelGGL(greedy_pool_kernel, dim3(grid), dim3(kSolveThreads), 0, st, D, H, wgt, R,
                           p.n_cand, (double)n, shift, h, choice, pool);
        // pools of up to kGreedyFast upgrades take the register-resident
        // kernel; larger ones the one-entry-scan kernel (each returns at
        // once when the pool is the other's)
        hipLaunchKernelGGL(greedy_apply_fast_kernel, dim3(1), dim3(64), 0, st, D, H, wgt, stats, R,
                           p.s, n, shift, rt, h, choice, codebook, m, off, pool);
        hipLaunchKernelGGL(greedy_apply_kernel, dim3(1), dim3(kSolveThreads), 0, st, D, H, wgt, stats, R,
                           p.s, n, shift, rt, h, choice, codebook, m, off, pool);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    return launch_offsets_scan(off, R, ws, st);
}

hipError_t launch_offsets_scan(uint64_t* off, int64_t R, void* ws, hipStream_t st) {
    if (R == 0) return hipSuccess;
    const int64_t tiles = (R + kScanTile - 1) / kScanTile;
    uint64_t* tile_sums = (uint64_t*)((char*)ws + kWsHeaderBytes);
    hipLaunchKernelGGL(scan_tiles_kernel, dim3((unsigned)tiles), dim3(kSolveThreads), 0, st, off, R,
                       tile_sums);
    if (tiles == 1) return hipGetLastError();  // one tile: its scan is the result
    hipLaunchKernelGGL(scan_sums_kernel, dim3(1), dim3(kSolveThreads), 0, st, tile_sums, tiles);
    hipLaunchKernelGGL(scan_add_kernel, dim3((unsigned)tiles), dim3(kSolveThreads), 0, st, off, R,
                       tile_sums);
    return hipGetLastError();
}

}  // namespace kvq
