"""Pins of the oracle's dual solve (CPU only).

Page "Rate-adaptive KV-cache quantizer", Key formulas (1), (2), (4) and the
Verification section (choice transitions occur at analytically predicted
multiplier crossings); page "Joint Tucker-rank and residual-bit KV
allocator", Mathematical statement (binary search on the multiplier finds a
budget-feasible allocation).
"""

import itertools
import math

import numpy as np
import pytest

from oracle import ecasq, pipeline
from oracle import blocks as oblocks
from kv_cache_rate_amd import workloads as W


@pytest.fixture(scope="module")
def tiny_tables():
    t = W.generate(W.TINY_K_FP32)
    b = oblocks.partition(t, 32, 128)
    D, H, S, books = pipeline.eval_grids(b, 8)
    return D, H


def test_lambda_zero_and_infinity(tiny_tables):
    """lambda = 0 picks the least distortion; a huge lambda picks the least
    entropy (not necessarily k = 2: with heavy tails {min, median, max}
    carries less entropy than {min, max})."""
    D, H = tiny_tables
    c0 = ecasq.choose(D, H, 4096.0, 0.0)
    assert np.array_equal(c0, np.argmin(D, axis=1))
    cinf = ecasq.choose(D, H, 4096.0, 1e30)
    for r in range(D.shape[0]):
        hmin = H[r].min()
        ties = np.flatnonzero(H[r] <= hmin * (1 + 1e-12))
        assert cinf[r] in ties
    # on this workload the least-entropy candidate is the 3-point quantile grid
    assert np.all(cinf == 2)


def test_bisection_feasible_and_tight(tiny_tables):
    D, H = tiny_tables
    R = D.shape[0]
    for B in (0.8, 1.0, 1.2):
        lam, choice, rate, Btot, probes = ecasq.solve_bisect(D, H, 4096.0, B, 40)
        assert rate <= Btot
        assert rate == ecasq.total_rate(H, 4096.0, choice)
        # bracket: the last infeasible probe is within hi * 2^-39 below lam
        infeasible = [l for l, rt in probes if rt > Btot]
        lo = max(infeasible)
        assert lo < lam <= lo + lam * 2.0 ** -39
        # a choice transition of some block lies in (lo, lam]: the analytic
        # crossing (D_a - D_b) / (d (H_b - H_a)) of its two choices
        c_lo = ecasq.choose(D, H, 4096.0, lo)
        changed = np.flatnonzero(c_lo != choice)
        assert changed.size >= 1
        for r in changed:
            a, b = choice[r], c_lo[r]
            cross = (D[r, a] - D[r, b]) / (4096.0 * (H[r, b] - H[r, a]))
            assert lo * (1 - 1e-12) <= cross <= lam * (1 + 1e-12)


def test_lambda_transitions_at_analytic_crossings(tiny_tables):
    """Sweeping lambda, every block's choice changes exactly where the
    lower envelope of the lines D_c + lambda d H_c predicts."""
    D, H = tiny_tables
    d = 4096.0
    lams = np.geomspace(1e-3, 1e3, 3000)
    for r in range(0, D.shape[0], 7):
        prev = ecasq.choose(D[r:r + 1], H[r:r + 1], d, lams[0])[0]
        for lo, hi in zip(lams[:-1], lams[1:]):
            cur = ecasq.choose(D[r:r + 1], H[r:r + 1], d, hi)[0]
            if cur != prev:
                cross = (D[r, prev] - D[r, cur]) / (d * (H[r, cur] - H[r, prev]))
                assert lo <= cross <= hi
                assert H[r, cur] < H[r, prev]  # entropy falls as lambda grows
            prev = cur


def test_everett_brute_force(tiny_tables):
    """Lagrangian sufficiency (Everett 1963): the choice at the bisection's
    multiplier has the least total distortion among ALL allocations whose
    rate does not exceed its own.  Brute force over 13^4 allocations."""
    D, H = tiny_tables
    blocks = [3, 17, 40, 61]
    Ds, Hs = D[blocks], H[blocks]
    d = 4096.0
    for B in (0.7, 0.9, 1.1):
        lam, choice, rate, Btot, _ = ecasq.solve_bisect(Ds, Hs, d, B, 40)
        dsum = Ds[np.arange(4), choice].sum()
        best = math.inf
        for combo in itertools.product(range(Ds.shape[1]), repeat=4):
            rt = sum(d * Hs[i, c] for i, c in enumerate(combo))
            if rt <= rate * (1 + 1e-12):
                best = min(best, sum(Ds[i, c] for i, c in enumerate(combo)))
        assert dsum <= best * (1 + 1e-12)


def test_infeasible_budget():
    D = np.array([[1.0, 2.0], [1.0, 3.0]])
    H = np.array([[1.0, 0.5], [2.0, 0.25]])
    with pytest.raises(ecasq.Infeasible):
        ecasq.solve_bisect(D, H, 1.0, 0.1, 40)


def test_slack_budget_gives_zero():
    D = np.array([[1.0, 2.0], [1.0, 3.0]])
    H = np.array([[1.0, 0.5], [2.0, 0.25]])
    lam, choice, rate, Btot, _ = ecasq.solve_bisect(D, H, 1.0, 1.5, 40)
    assert lam == 0.0 and list(choice) == [0, 0] and rate == 3.0


def test_subgradient_worked_example():
    """Hand-worked numbers (tests/golden/subgrad_example.txt)."""
    path = __file__.replace("test_oracle_solve.py", "golden/subgrad_example.txt")
    vals = {}
    for line in open(path):
        line = line.split("#")[0].strip()
        if line:
            k, v = line.split("=")
            vals[k.strip()] = v.strip()
    D = np.array(eval(vals["D"]))
    H = np.array(eval(vals["H"]))
    c, rbar, lam = ecasq.subgrad_step(D, H, float(vals["d"]), float(vals["B"]),
                                      float(vals["lam_prev"]), float(vals["eta"]))
    assert list(c) == eval(vals["choice"])
    assert rbar == pytest.approx(float(vals["Rbar"]), rel=1e-15)
    assert lam == pytest.approx(float(vals["lam_next"]), rel=1e-15)
    _, _, lam2 = ecasq.subgrad_step(D, H, float(vals["d"]), 3.0,
                                    float(vals["lam_prev"]), float(vals["eta"]))
    assert lam2 == pytest.approx(float(vals["lam_next_b3"]), rel=1e-15)
    _, _, lam3 = ecasq.subgrad_step(D, H, float(vals["d"]), 10.0,
                                    float(vals["lam_prev"]), float(vals["eta"]))
    assert lam3 == float(vals["lam_next_projected"])


def test_two_block_mechanism():
    """Qualitative analogue of the page's toy (Verification): with a low-
    and a high-variance block and equally spaced min/max alphabets, the
    adaptive allocation gives fewer levels to the low-variance block and less
    total distortion than 4 levels everywhere, at no more modelled rate."""
    rng = np.random.default_rng(7)
    xa = rng.standard_normal(4096) * 0.2
    xb = rng.standard_normal(4096) * 2.0
    ks = list(range(2, 9))
    D = np.zeros((2, len(ks)))
    H = np.zeros((2, len(ks)))
    for r, x in enumerate((xa, xb)):
        for c, k in enumerate(ks):
            Q = np.unique(ecasq.uniform_points(x.min(), x.max(), k))
            D[r, c], H[r, c], _ = ecasq.score_codebook(x, Q)
    c4 = ks.index(4)
    rate4 = 4096 * (H[0, c4] + H[1, c4])
    lam, choice, rate, Btot, _ = ecasq.solve_bisect(D, H, 4096.0, rate4 / 8192, 40)
    assert rate <= rate4
    assert ks[choice[0]] < ks[choice[1]]
    assert D[0, choice[0]] + D[1, choice[1]] < D[0, c4] + D[1, c4]


# ------------------------------------------------ weighted distortion ---

def _tables(rng, R=40, C=9):
    D = rng.uniform(0.1, 10.0, size=(R, C))
    H = rng.uniform(0.0, 4.0, size=(R, C))
    return D, H


def test_unit_weights_are_the_unweighted_problem(rng):
    D, H = _tables(rng)
    w = np.ones(D.shape[0])
    for lam in (0.0, 1e-3, 0.37, 5.0):
        assert np.array_equal(ecasq.choose(D, H, 64.0, lam, w), ecasq.choose(D, H, 64.0, lam))
    a = ecasq.solve_bisect(D, H, 64.0, 1.5, 30, w)
    b = ecasq.solve_bisect(D, H, 64.0, 1.5, 30)
    assert a[0] == b[0] and np.array_equal(a[1], b[1])


def test_weight_scaling_is_a_multiplier_scaling(rng):
    """argmin (4w) D + lam d H = argmin w D + (lam / 4) d H exactly (powers of
    two scale every rounded term exactly)."""
    D, H = _tables(rng)
    w = rng.lognormal(0.0, 0.5, size=D.shape[0])
    for lam in (1e-3, 0.37, 5.0):
        assert np.array_equal(ecasq.choose(D, H, 64.0, lam, 4.0 * w),
                              ecasq.choose(D, H, 64.0, lam / 4.0, w))


def test_heavier_weight_never_raises_a_blocks_distortion(rng):
    """Exchange argument: w' > w implies D(choice at w') <= D(choice at w)."""
    D, H = _tables(rng, R=200)
    w = rng.lognormal(0.0, 0.5, size=200)
    for lam in (0.01, 0.2, 1.0):
        c1 = ecasq.choose(D, H, 64.0, lam, w)
        c2 = ecasq.choose(D, H, 64.0, lam, 1.7 * w)
        r = np.arange(200)
        assert np.all(D[r, c2] <= D[r, c1])


def test_weighted_bisection_is_feasible_and_tight(rng):
    D, H = _tables(rng, R=60)
    w = rng.lognormal(0.0, 0.5, size=60)
    lam, c, rate, Btot, probes = ecasq.solve_bisect(D, H, 64.0, 1.2, 40, w)
    assert rate <= Btot
    assert np.array_equal(c, ecasq.choose(D, H, 64.0, lam, w))
    # the closest probe below lambda was infeasible, within the bracket width
    lo = max((p for p, r in probes if p < lam), default=0.0)
    assert dict(probes)[lo] > Btot
    assert lam - lo <= 2.0 ** -40 * max(1.0, 2.0 * lam)
    below = ecasq.choose(D, H, 64.0, lo, w)
    assert ecasq.total_rate(H, 64.0, below) > Btot


# --------------------------------------------------- greedy post-pass ---

def test_greedy_fill_hand_example():
    """Three blocks, d = 1.  Budget 4.0; bisection picks (H, D) = (1, 10)
    for every block (rate 3).  Slack 1.0.  Upgrades: block 0 to (1.5, 6)
    saves 4 for 0.5 bits (8 per bit); block 1 to (2, 5) saves 5 for 1 bit
    (5 per bit); block 2 to (1.25, 9) saves 1 for 0.25 (4 per bit).
    Greedy: block 0 (8/bit, slack 0.5 left), then block 2 (0.25 <= 0.5,
    slack 0.25); block 1's step (1 bit) no longer fits."""
    H = np.array([[1.0, 1.5], [1.0, 2.0], [1.0, 1.25]])
    D = np.array([[10.0, 6.0], [10.0, 5.0], [10.0, 9.0]])
    ch, rate, swaps = ecasq.greedy_fill(D, H, 1.0, 4.0, np.zeros(3, dtype=int))
    assert swaps == [(0, 0, 1), (2, 0, 1)]
    assert ch.tolist() == [1, 0, 1] and rate == 3.75


def test_greedy_fill_properties(rng):
    for trial in range(20):
        R, C = 30, 8
        H = np.sort(rng.uniform(0.0, 4.0, size=(R, C)), axis=1)
        D = np.sort(rng.uniform(0.1, 10.0, size=(R, C)), axis=1)[:, ::-1].copy()
        B = rng.uniform(0.8, 2.5)
        lam, c0, r0, Btot, _ = ecasq.solve_bisect(D, H, 64.0, B, 30)
        c1, r1, swaps = ecasq.greedy_fill(D, H, 64.0, Btot, c0)
        r = np.arange(R)
        assert r1 <= Btot                                  # still within budget
        assert D[r, c1].sum() <= D[r, c0].sum()           # never worse
        slack = Btot - r1
        rates = 64.0 * H
        up = (rates - rates[r, c1][:, None] > 0) & (D[r, c1][:, None] - D > 0)
        assert not np.any(up & (rates - rates[r, c1][:, None] <= slack * (1 - 1e-12)))  # maximal
        eff = [(D[b, a] - D[b, c]) / (rates[b, c] - rates[b, a]) for b, a, c in swaps]
        assert all(x > 0 for x in eff)
