"""Candidate codebooks, closed-form scoring and the dual solve (oracle;
test infrastructure only).

Everything is fp64 and follows the page "Rate-adaptive KV-cache quantizer"
(synthcore idea 2502):

* Mathematical statement / Key formulas (3): for x in [q_i, q_{i+1}] the
  unbiased stochastic interpolation goes to q_i with probability
  (q_{i+1}-x)/(q_{i+1}-q_i) and to q_{i+1} with probability
  (x-q_i)/(q_{i+1}-q_i); its conditional mean is x and its conditional MSE is
  (q_{i+1}-x)(x-q_i); the block distortion D_r sums that MSE over the block.
* Mathematical statement: H_r is the entropy in bits of the expected symbol
  frequencies pi_{r,j} (never of one random draw, Implementation notes).
* Key formulas (1)-(2): minimise sum_r D_r subject to sum_r d_r H_r <= B; for
  a fixed multiplier lambda each block independently minimises
  D_r + lambda d_r H_r.
* Key formulas (4) and Implementation notes: the multiplier may be moved by a
  projected subgradient step; page "Joint Tucker-rank and residual-bit KV
  allocator", Mathematical statement / Implementation notes: a binary search
  on the multiplier finds a budget-feasible allocation.
* Implementation notes: the candidate alphabet of a block is built from its
  minimum, maximum and quantiles, for codebook sizes k <= s.

Readings taken where the pages are silent:

* D_r is a sum over the block; H_r is bits per entry, so d_r H_r is bits per
  block and a per-entry budget B means a total of B * sum_r d_r.
* Candidate family for codebook limit s: {min, max}, then for k = 3..s the
  uniform grid U_k and the empirical-quantile grid E_k, in that order.
* U_k point j is computed in fp64 round-to-nearest as
  mn + ((mx - mn) * j) / (k - 1) with no fused multiply-add, then rounded to
  fp32; codepoints are stored in fp32 and unbiasedness holds for the stored
  values.
* E_k point j is the order statistic of rank floor((2 j (n-1) + k - 1) /
  (2 (k - 1))), i.e. j (n-1)/(k-1) rounded half up.
* Each candidate is reduced to its sorted distinct values (ties in the data
  or coinciding grid points give fewer than k levels).
* An entry equal to a codepoint is interpolated in the interval to its right
  (the last interval is closed); every convention gives the same D, pi and
  code because the formulas are continuous there.
* argmin ties go to the lowest candidate index.
"""

import math
from fractions import Fraction

import numpy as np


def n_candidates(s):
    """Number of grid candidates for codebook limit ``s`` (k = 2 counted once)."""
    return 1 + 2 * (s - 2)


def quantile_rank(j, k, n):
    """Rank of the j-th point of the k-point empirical-quantile grid of n
    sorted entries: j (n-1)/(k-1) rounded half up (integer arithmetic)."""
    return (2 * j * (n - 1) + (k - 1)) // (2 * (k - 1))


def quantile_ranks(n, s):
    """Sorted distinct ranks used by every quantile grid with k = 2..s."""
    ranks = set()
    for k in range(2, s + 1):
        for j in range(k):
            ranks.add(quantile_rank(j, k, n))
    return np.array(sorted(ranks), dtype=np.int64)


def uniform_points(mn, mx, k):
    """k equally spaced codepoints from mn to mx (fp64 ops, then fp32)."""
    mn = np.float64(mn)
    mx = np.float64(mx)
    j = np.arange(k, dtype=np.float64)
    v = mn + ((mx - mn) * j) / np.float64(k - 1)
    return v.astype(np.float32).astype(np.float64)


def quantile_points(xs, k):
    """k empirical-quantile codepoints (order statistics) of sorted ``xs``."""
    n = xs.size
    j = np.arange(k, dtype=np.int64)
    return xs[quantile_rank(j, k, n)]


def grid_candidates(xs, s):
    """Candidate codebooks of one block, in canonical order.

    ``xs`` is the block sorted ascending.  Returns a list of
    ``n_candidates(s)`` sorted arrays of distinct fp64 values.
    """
    mn, mx = xs[0], xs[-1]
    cands = [np.unique(np.array([mn, mx], dtype=np.float64))]
    for k in range(3, s + 1):
        cands.append(np.unique(uniform_points(mn, mx, k)))
        cands.append(np.unique(quantile_points(xs, k)))
    return cands


def interval_index(Q, x):
    """Index i of the interval [Q_i, Q_{i+1}] that interpolates x."""
    m = Q.size
    i = np.searchsorted(Q, x, side="right") - 1
    return np.clip(i, 0, m - 2)


def entropy_bits(pi):
    """-sum pi log2 pi over the positive entries (0 log 0 = 0)."""
    pi = np.asarray(pi, dtype=np.float64)
    pos = pi[pi > 0]
    return float(-np.sum(pos * np.log2(pos)))


def score_codebook(x, Q):
    """Closed-form distortion, expected-frequency entropy and frequencies.

    For each entry x_t: interval i(t), probability p_t of rounding up,
    distortion (q_{i+1}-x_t)(x_t-q_i); pi_j collects the probability mass
    each entry sends to q_j, divided by the block length.
    Returns ``(D, H, pi)`` with D a block sum and H in bits per entry.
    """
    x = np.asarray(x, dtype=np.float64)
    Q = np.asarray(Q, dtype=np.float64)
    n = x.size
    m = Q.size
    if m == 1:
        return 0.0, 0.0, np.ones(1)
    i = interval_index(Q, x)
    a = Q[i]
    b = Q[i + 1]
    p = (x - a) / (b - a)
    D = float(np.sum((b - x) * (x - a)))
    pi = (np.bincount(i, weights=1.0 - p, minlength=m)
          + np.bincount(i + 1, weights=p, minlength=m)) / n
    return D, entropy_bits(pi), pi


def eval_block(x, s):
    """Score every grid candidate of one block.

    Returns ``(D[C], H[C], stats, cands)`` where ``stats`` holds the order
    statistics at :func:`quantile_ranks` (minimum first, maximum last).
    """
    xs = np.sort(np.asarray(x, dtype=np.float64))
    C = n_candidates(s)
    stats = xs[quantile_ranks(xs.size, s)]
    if xs[0] == xs[-1]:
        cands = [np.array([xs[0]])] * C
        return np.zeros(C), np.zeros(C), stats, cands
    cands = grid_candidates(xs, s)
    D = np.empty(C)
    H = np.empty(C)
    for c, Q in enumerate(cands):
        D[c], H[c], _ = score_codebook(x, Q)
    return D, H, stats, cands


def choose(D, H, d, lam, w=None):
    """Per-block argmin of D + lambda d H (ties to the lowest index).

    ``D``, ``H`` are ``[R, C]``; ``d`` is the block length (scalar or [R]).
    The objective is evaluated as D + ((lambda * d) * H) in fp64.  With
    per-block weights ``w`` ([R], the page's optional attention-sensitivity
    weighting of D_r, Implementation notes) it is (w_r D) + ((lambda d) H).
    """
    D = np.asarray(D, dtype=np.float64)
    H = np.asarray(H, dtype=np.float64)
    if w is not None:
        D = np.asarray(w, dtype=np.float64)[:, None] * D
    scale = np.float64(lam) * np.asarray(d, dtype=np.float64)
    if np.ndim(scale):
        scale = scale[:, None]
    return np.argmin(D + scale * H, axis=1)


def total_rate(H, d, choice):
    """sum_r d_r H_r of a choice, in bits, summed exactly (math.fsum)."""
    H = np.asarray(H, dtype=np.float64)
    R = H.shape[0]
    dr = np.broadcast_to(np.asarray(d, dtype=np.float64), (R,))
    return math.fsum((dr * H[np.arange(R), choice]).tolist())


class Infeasible(Exception):
    """No multiplier up to 2**64 meets the budget."""


def bisect_multiplier(rate_at, Btot, iters=40):
    """Bisection on the multiplier for any per-multiplier allocation.

    ``rate_at(lam)`` returns ``(rate_bits_total, choice)`` of the blocks'
    minimisers at ``lam``.  Bracket: lambda = 0 if it is already feasible;
    otherwise lo = 0, hi = 1 and hi doubles (lo following) while infeasible,
    up to 2**64; then ``iters`` halvings.  The feasible end ``hi`` is
    returned with its choice and rate: ``(lam, choice, rate_bits_total)``.
    """
    r0, c0 = rate_at(0.0)
    if r0 <= Btot:
        return 0.0, c0, r0
    lo, hi = 0.0, 1.0
    while True:
        rh, ch = rate_at(hi)
        if rh <= Btot:
            break
        if hi >= 2.0 ** 64:
            raise Infeasible("budget below the least-entropy allocation")
        lo, hi = hi, hi * 2.0
    for _ in range(iters):
        mid = (lo + hi) / 2.0
        rm, cm = rate_at(mid)
        if rm <= Btot:
            hi, rh, ch = mid, rm, cm
        else:
            lo = mid
    return hi, ch, rh


def solve_bisect(D, H, d, B, iters=40, w=None):
    """Bisection on the multiplier until sum_r d_r H_r <= B * sum_r d_r, over
    the candidate tables ``D``, ``H`` ([R, C]); see :func:`bisect_multiplier`.
    Returns ``(lam, choice, rate_bits_total, B_total, probes)`` where
    ``probes`` lists every (lambda, rate) evaluated, in order.
    """
    R = np.asarray(D).shape[0]
    dr = np.broadcast_to(np.asarray(d, dtype=np.float64), (R,))
    Btot = float(B) * math.fsum(dr.tolist())
    probes = []

    def rate(lam):
        c = choose(D, H, dr, lam, w)
        rt = total_rate(H, dr, c)
        probes.append((lam, rt))
        return rt, c

    lam, choice, rt = bisect_multiplier(rate, Btot, iters)
    return lam, choice, rt, Btot, probes


def subgrad_step(D, H, d, B, lam_prev, eta, w=None):
    """One decode-time dual step.

    The blocks are chosen at the known multiplier ``lam_prev``; the modelled
    rate per entry Rbar = sum d_r H_r / sum d_r is compared with the per-entry
    budget B and lambda <- max(0, lam_prev + eta (Rbar - B)).
    Returns ``(choice, Rbar, lam_next)``.
    """
    R = np.asarray(D).shape[0]
    dr = np.broadcast_to(np.asarray(d, dtype=np.float64), (R,))
    c = choose(D, H, dr, lam_prev, w)
    rbar = total_rate(H, dr, c) / math.fsum(dr.tolist())
    lam_next = max(0.0, float(lam_prev) + float(eta) * (rbar - float(B)))
    return c, rbar, lam_next


def greedy_fill(D, H, d, Btot, choice, w=None):
    """Post-pass after a feasible multiplier (the page "Joint Tucker-rank and
    residual-bit KV allocator", Implementation notes: after the multiplier
    search, improve the allocation by swapping candidates with the best
    distortion reduction per added byte).

    While some block has a candidate with more bits (dR > 0), less
    (weighted) distortion (dD > 0) and dR no larger than the remaining
    budget, switch the block with the largest dD / dR (fp64), ties to the
    lowest block then the lowest candidate.  Rates are d H_{r,c} (fp64
    products); the remaining budget and each dR are compared exactly
    (rational arithmetic).  Returns ``(choice, rate_bits, swaps)``.
    """
    D = np.asarray(D, dtype=np.float64)
    H = np.asarray(H, dtype=np.float64)
    Dw = D if w is None else np.asarray(w, dtype=np.float64)[:, None] * D
    R, C = D.shape
    dr = float(d)
    rates = dr * H                      # fp64 products, as the budget counts them
    ch = np.array(choice, dtype=np.int64).copy()
    rows = np.arange(R)
    slack = Fraction(float(Btot)) - sum(Fraction(float(v)) for v in rates[rows, ch])
    swaps = []
    while True:
        cur_r = rates[rows, ch][:, None]
        cur_d = Dw[rows, ch][:, None]
        dR = rates - cur_r              # fp64 screen; exact check below
        dD = cur_d - Dw
        ok = (dR > 0) & (dD > 0) & (dR <= float(slack) * (1 + 1e-12) + 1e-300)
        best = None
        for r, c in zip(*np.nonzero(ok)):
            exact = Fraction(float(rates[r, c])) - Fraction(float(rates[r, ch[r]]))
            if exact <= 0 or exact > slack:
                continue
            e = (Dw[r, ch[r]] - Dw[r, c]) / (rates[r, c] - rates[r, ch[r]])
            key = (e, -int(r), -int(c))
            if best is None or key > best[0]:
                best = (key, int(r), int(c), exact)
        if best is None:
            break
        _, r, c, exact = best
        swaps.append((r, int(ch[r]), c))
        ch[r] = c
        slack -= exact
    return ch, total_rate(H, dr, ch), swaps
