"""Exact codebook search over a quantile alphabet (oracle; test
infrastructure only).

Page "Rate-adaptive KV-cache quantizer": the Implementation notes choose each
block's codebook as the argmin of D_r + lambda d_r H_r "using a small dynamic
program ... over ordered codepoints" drawn from an alphabet of the block's
minimum, maximum and quantiles; the Mathematical statement scores a codebook
by the closed-form interpolation distortion and the entropy of expected
frequencies (Key formulas (3)).

Reading taken here: the alphabet is the sorted distinct set of the m = 12
order statistics at ranks j (n-1)/11 rounded half up (j = 0..11); a
candidate is any subset S of the alphabet that contains its minimum and
maximum and has 2 <= |S| <= s (s = 8).  The definition of the minimiser is
brute force over all such subsets (:func:`brute_force_tables` + argmin, ties
to the first subset in the order (size, lexicographic index tuple)).  The
pair-state dynamic program (:func:`dp_minimise`) is a second, independent
route to the same minimum and is pinned to brute force in the tests.

Decomposition used by both (an exact regrouping of the per-entry sums of
Key formulas (3)): every entry of the block falls in exactly one interval
[A_i, A_j) between consecutive points of S (the last interval closed), so
D(S) is a sum of per-pair distortions and each point's expected frequency
is the mass sent to it from the interval on its left plus the interval on
its right.
"""

import itertools
import math

import numpy as np

from .ecasq import quantile_rank


def alphabet(xs, m=12):
    """Sorted distinct order statistics at the m alphabet ranks of sorted ``xs``."""
    n = xs.size
    j = np.arange(m, dtype=np.int64)
    return np.unique(xs[quantile_rank(j, m, n)])


def alphabet_ranks(n, m=12):
    return quantile_rank(np.arange(m, dtype=np.int64), m, n)


def pair_stats(x, A):
    """Per pair (i < j) of alphabet points, over the entries x with
    A_i <= x < A_j (x <= A_j when j is the last point):

    * Dp[i, j]  = sum (A_j - x)(x - A_i)
    * ML[i, j]  = sum (A_j - x)/(A_j - A_i)   (mass sent to A_i)
    * MR[i, j]  = sum (x - A_i)/(A_j - A_i)   (mass sent to A_j)

    computed directly entry by entry.  Arrays are [m, m] (upper triangle used).
    """
    x = np.asarray(x, dtype=np.float64)
    m = A.size
    Dp = np.zeros((m, m))
    ML = np.zeros((m, m))
    MR = np.zeros((m, m))
    for i in range(m):
        for j in range(i + 1, m):
            a, b = A[i], A[j]
            if j == m - 1:
                sel = x[(x >= a) & (x <= b)]
            else:
                sel = x[(x >= a) & (x < b)]
            Dp[i, j] = np.sum((b - sel) * (sel - a))
            ML[i, j] = np.sum((b - sel) / (b - a))
            MR[i, j] = np.sum((sel - a) / (b - a))
    return Dp, ML, MR


def subsets(m, smax):
    """Endpoint-containing index subsets of range(m), sizes 2..smax, in
    canonical order (size, then lexicographic)."""
    if m == 1:
        return [(0,)]
    inner = list(range(1, m - 1))
    out = []
    for size in range(2, min(smax, m) + 1):
        for mid in itertools.combinations(inner, size - 2):
            out.append((0,) + mid + (m - 1,))
    return out


def subset_score(Dp, ML, MR, n, S):
    """D(S) and H(S) (bits per entry) from pair statistics."""
    if len(S) == 1:
        return 0.0, 0.0
    D = 0.0
    pis = []
    for t, i in enumerate(S):
        mass = 0.0
        if t > 0:
            mass += MR[S[t - 1], i]
        if t + 1 < len(S):
            mass += ML[i, S[t + 1]]
            D += Dp[i, S[t + 1]]
        pis.append(mass / n)
    H = 0.0
    for p in pis:
        if p > 0:
            H -= p * math.log2(p)
    return D, H


def brute_force_tables(Dp, ML, MR, n, smax):
    """(D(S), H(S)) for every candidate subset, in canonical order."""
    m = Dp.shape[0]
    S_list = subsets(m, smax)
    D = np.empty(len(S_list))
    H = np.empty(len(S_list))
    for c, S in enumerate(S_list):
        D[c], H[c] = subset_score(Dp, ML, MR, n, S)
    return D, H, S_list


def _h(p):
    return -p * math.log2(p) if p > 0 else 0.0


def dp_minimise(Dp, ML, MR, n, d, lam, smax):
    """Pair-state dynamic program for min_S D(S) + lam d H(S).

    State (c, i, j): best cost of a chain that starts at point 0, has c
    points and ends with the two points i < j; the cost holds the distortion
    of every closed interval and the entropy term of every point before j
    (the frequency of q_j needs both of its neighbours).  Returns
    ``(best_value, best_subset)``.
    """
    m = Dp.shape[0]
    if m == 1:
        return 0.0, (0,)
    w = lam * d
    INF = math.inf
    # f[(i, j)] for the current count c, with the chain stored for the argmin.
    f = {}
    for l in range(1, m):
        f[(0, l)] = (Dp[0, l] + w * _h(ML[0, l] / n), (0, l))
    best = (INF, None)
    c = 2
    while True:
        for (i, j), (v, chain) in f.items():
            if j == m - 1:
                tot = v + w * _h(MR[i, j] / n)
                if tot < best[0]:
                    best = (tot, chain)
        if c == min(smax, m):
            break
        g = {}
        for (i, j), (v, chain) in f.items():
            if j == m - 1:
                continue
            for l in range(j + 1, m):
                cand = v + Dp[j, l] + w * _h((MR[i, j] + ML[j, l]) / n)
                if (j, l) not in g or cand < g[(j, l)][0]:
                    g[(j, l)] = (cand, chain + (l,))
        f = g
        c += 1
    return best
