// A block's choice among the grid candidates at a known multiplier: the
// objective and the fixed-point rate (shared by the solve, kvq_solve.hip,
// and the one-launch decode admission, kvq_eval16.hip) and the chosen
// codebook's points (the solve; the one-launch admission computes the same
// points one per lane).
//
// Page "Rate-adaptive KV-cache quantizer", Key formulas (2): at a fixed
// multiplier each block minimises D_r + lambda d_r H_r on its own;
// Implementation notes: the candidates are built from the block's minimum,
// maximum and quantiles.
#pragma once

#include "kvq_internal.h"

namespace kvq {

// Objective D + (lambda * d) * H, evaluated without contraction.
__device__ __forceinline__ double objective(double Dv, double Hv, double lamd) {
#pragma clang fp contract(off)
    const double t = lamd * Hv;
    return Dv + t;
}

__device__ __forceinline__ unsigned long long rate_fx(double d, double Hv, int shift) {
    return __double2ull_rn(ldexp(d * Hv, shift));
}

// Codepoints of grid candidate c of a block from its minimum, maximum and
// order statistics (st: the block's first statistic, `stride` apart; col:
// RankTable::col as a (kMaxS + 1) x kMaxS table, in LDS where it matters),
// written as the block's codebook row (s entries, zero after the m distinct
// points); returns m.  The k points are gathered unrolled to kMaxS with
// unconditional loads (statistic 0 where a point needs none), so the loads
// are in flight together.  The points are non-decreasing, so equal ones are
// adjacent: each distinct point is stored at a running position, straight
// to memory (a register array indexed by a per-lane position compiles into
// long select chains).
__device__ inline int write_grid_codebook(int c, float mn, float mx, const float* st, int64_t stride,
                                   const uint8_t* col, int s, float* row) {
    if ((s & 3) == 0 && ((uintptr_t)row & 15u) == 0) {
#pragma unroll
        for (int j4 = 0; j4 < kMaxS / 4; ++j4)
            if (4 * j4 < s) reinterpret_cast<float4*>(row)[j4] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    } else {
        for (int j = 0; j < s; ++j) row[j] = 0.0f;
    }
    if (mn == mx) {
        row[0] = mn;
        return 1;
    }
    int k;
    bool uni = false;
    if (c == 0) {
        k = 2;
    } else {
        k = 3 + (c - 1) / 2;
        uni = ((c - 1) & 1) == 0;
    }
    const bool quant = c != 0 && !uni;
    int idx[kMaxS];
#pragma unroll
    for (int j = 0; j < kMaxS; ++j) idx[j] = quant && j < k ? (int)col[k * kMaxS + j] : 0;
    float g[kMaxS];
#pragma unroll
    for (int j = 0; j < kMaxS; ++j) g[j] = st[idx[j] * stride];
    int m = 0;
    float prev = 0.0f;
#pragma unroll
    for (int j = 0; j < kMaxS; ++j) {
        float v = c == 0 ? (j == 0 ? mn : mx) : g[j];
        if (uni && j < k) v = uniform_point(mn, mx, j, k);  // fp64 division: only where needed
        const bool keep = j < k && (j == 0 || v != prev);
        if (keep) row[m] = v;
        m += keep ? 1 : 0;
        prev = v;
    }
    return m;
}

}  // namespace kvq
