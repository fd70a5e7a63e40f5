"""Exact codebook search over a quantile alphabet (oracle; test
infrastructure only).

Page "Rate-adaptive KV-cache quantizer": the Implementation notes choose each
block's codebook as the argmin of D_r + lambda d_r H_r "using a small dynamic
program ... over ordered codepoints" drawn from an alphabet of the block's
minimum, maximum and quantiles; the Mathematical statement scores a codebook
by the closed-form interpolation distortion and the entropy of expected
frequencies (Key formulas (3)).

Reading taken here: the alphabet is the sorted distinct set of the M
order statistics at ranks j (n-1)/(M-1) rounded half up (j = 0..M-1; M = 12
for the feature-group workload, up to 32 for the larger alphabets); a
candidate is any subset S of the alphabet that contains its minimum and
maximum and has 2 <= |S| <= s.  The definition of the minimiser is brute
force over all such subsets (:func:`brute_force_tables` + argmin, ties to
the first subset in the order (size, lexicographic index tuple)).  The
pair-state dynamic program (:func:`dp_minimise`) is a second, independent
route to the same minimum and is pinned to brute force in the tests; it is
the route used where brute force is out of reach (large M and s), with
:func:`solve_bisect_dp` running the bisection on its minimisers.

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


def _h_array(P):
    """-p log2 p elementwise (0 where p <= 0)."""
    P = np.asarray(P, dtype=np.float64)
    out = np.zeros_like(P)
    pos = P > 0
    out[pos] = -P[pos] * np.log2(P[pos])
    return out


def dp_minimise(Dp, ML, MR, n, d, lam, smax):
    """Pair-state dynamic program for min_S D(S) + lam d H(S).

    State (c, i, j): best cost of a chain that starts at point 0, has c
    points and ends with the two points i < j; the cost holds the distortion
    of every closed interval and the entropy term of every point before j
    (the frequency of q_j needs both of its neighbours):

        f_2[0, l]     = Dp[0, l] + w h(ML[0, l] / n)
        f_{c+1}[j, l] = min_{i < j} (f_c[i, j] + Dp[j, l]) + w h((MR[i, j] + ML[j, l]) / n)
        value         = min_{c, i} f_c[i, m-1] + w h(MR[i, m-1] / n)

    with w = lam d and h(p) = -p log2 p.  Chains that reached the last point
    are complete and are not extended.  Ties go to the lowest i, and across
    completions to the smallest c, then the lowest i.  Each layer is
    evaluated for all (i, j, l) at once.  Returns ``(best_value,
    best_subset)``.
    """
    m = Dp.shape[0]
    if m == 1:
        return 0.0, (0,)
    w = lam * d
    INF = math.inf
    idx = np.arange(m)
    # valid transitions i < j < l, j not the last point
    valid = (idx[:, None, None] < idx[None, :, None]) & (idx[None, :, None] < idx[None, None, :])
    valid &= (idx[None, :, None] < m - 1)
    # the entropy term of point j given both neighbours i and l
    hmid = w * _h_array((MR[:, :, None] + ML[None, :, :]) / n)
    f = np.full((m, m), INF)
    f[0, 1:] = Dp[0, 1:] + w * _h_array(ML[0, 1:] / n)
    parents = []          # parents[t][j, l]: the i chosen when (j, l) was reached
    best = (INF, None)
    c = 2
    while True:
        for i in range(m - 1):
            if f[i, m - 1] < INF:
                tot = f[i, m - 1] + w * _h(MR[i, m - 1] / n)
                if tot < best[0]:
                    best = (tot, _chain(parents, i, m - 1))
        if c == min(smax, m):
            break
        T = np.where(valid & (f[:, :, None] < INF), (f[:, :, None] + Dp[None, :, :]) + hmid, INF)
        par = np.argmin(T, axis=0)        # first minimum: lowest i
        f = np.min(T, axis=0)
        parents.append(par)
        c += 1
    return best


def _chain(parents, i, j):
    """Indices of the chain whose last two points are (i, j), rebuilt from
    the parent tables of the layers that led to it."""
    out = [j, i]
    for par in reversed(parents):
        i, j = int(par[i, j]), i
        out.append(i)
    return tuple(reversed(out))


def _dp_rate_chunk(args):
    pairs, n, lam, smax, width = args
    out = []
    for Dp, ML, MR in pairs:
        if width is None:
            _, S = dp_minimise(Dp, ML, MR, n, float(n), lam, smax)
        else:
            _, S = beam_minimise(Dp, ML, MR, n, float(n), lam, smax, width)
        out.append((S, float(n) * subset_score(Dp, ML, MR, n, S)[1]))
    return out


def solve_bisect_dp(pairs, n, B, smax, iters=40, processes=None, width=None):
    """The bisection of :func:`ecasq.bisect_multiplier` with every block's
    minimiser at each probed multiplier: the exact pair-state DP
    (:func:`dp_minimise`), or the beam search (:func:`beam_minimise`) of
    the given ``width``.

    ``pairs`` lists (Dp, ML, MR) per block.  Returns ``(lam, subsets,
    rate_bits_total, B_total, probes)``; the rate of a choice is
    sum_r n H_r(S_r) summed exactly (math.fsum).  ``processes`` > 1 spreads
    the blocks of each probe over a process pool (same results).
    """
    from multiprocessing import get_context
    from .ecasq import bisect_multiplier
    R = len(pairs)
    d = float(n)
    Btot = float(B) * math.fsum([d] * R)
    probes = []
    nchunk = max(1, min(R, 4 * (processes or 1)))
    bounds = np.linspace(0, R, nchunk + 1).astype(int)
    chunks = [pairs[bounds[k]:bounds[k + 1]] for k in range(nchunk)]
    pool = get_context("fork").Pool(processes) if processes and processes > 1 and R > 1 else None
    try:
        def rate(lam):
            args = [(c, n, lam, smax, width) for c in chunks]
            res = pool.map(_dp_rate_chunk, args) if pool else [_dp_rate_chunk(a) for a in args]
            flat = [e for part in res for e in part]
            rt = math.fsum([t for _, t in flat])
            probes.append((lam, rt))
            return rt, [S for S, _ in flat]

        lam, subs, rt = bisect_multiplier(rate, Btot, iters)
    finally:
        if pool:
            pool.close()
            pool.join()
    return lam, subs, rt, Btot, probes


def _lex_key(chain):
    return (len(chain), chain)


def beam_minimise(Dp, ML, MR, n, d, lam, smax, width):
    """Beam search over ordered codepoints for min_S D(S) + lam d H(S).

    Codebooks grow left to right over the ordered alphabet.  A partial
    chain (0, ..., j, l) is scored with the cost the DP carries: the
    distortion of its closed intervals and the entropy terms of every point
    before its last (w = lam d, h(p) = -p log2 p):

        cost(0, l)          = Dp[0, l] + w h(ML[0, l] / n)
        cost(..., i, j, l)  = (cost(..., i, j) + Dp[j, l]) + w h((MR[i, j] + ML[j, l]) / n)
        total(..., j, m-1)  = cost(..., j, m-1) + w h(MR[j, m-1] / n)

    The beam: chains with the same number of points that end at the same
    codepoint compete, and only the ``width`` cheapest of each such group
    (ties to the lexicographically smaller chain) are extended, by every
    later codepoint, up to ``smax`` points.  Every chain that reaches the
    last point is complete and scored.  Returns ``(best_total,
    best_chain)``, ties to the shorter, then the lexicographically smaller
    chain.  With an unbounded width every chain is enumerated (brute force);
    with the DP's state (the last two points) in place of the beam it would
    be :func:`dp_minimise`.
    """
    m = Dp.shape[0]
    if m == 1:
        return 0.0, (0,)
    w = lam * d
    best = (math.inf, None)
    arrivals = {}  # end point -> [(cost, chain)] of the current chain length
    for l in range(1, m):
        arrivals.setdefault(l, []).append((Dp[0, l] + w * _h(ML[0, l] / n), (0, l)))
    length = 2
    while True:
        for cost, chain in arrivals.get(m - 1, []):
            tot = cost + w * _h(MR[chain[-2], m - 1] / n)
            if best[1] is None or (tot, _lex_key(chain)) < (best[0], _lex_key(best[1])):
                best = (tot, chain)
        if length >= min(smax, m):
            break
        nxt = {}
        for j in range(1, m - 1):
            for cost, chain in sorted(arrivals.get(j, []))[:width]:
                i = chain[-2]
                for l in range(j + 1, m):
                    c2 = (cost + Dp[j, l]) + w * _h((MR[i, j] + ML[j, l]) / n)
                    nxt.setdefault(l, []).append((c2, chain + (l,)))
        arrivals = nxt
        length += 1
    return best
