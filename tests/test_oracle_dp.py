"""Pins of the exact codebook search over a quantile alphabet (CPU only).

Page "Rate-adaptive KV-cache quantizer", Implementation notes (a small
dynamic program over ordered codepoints drawn from the block's minimum,
maximum and quantiles) and Key formulas (3) (the scores).
"""

import math

import numpy as np
import pytest

from oracle import ecasq, exact_dp
from oracle import blocks as oblocks
from kv_cache_rate_amd import workloads as W


def test_subset_count():
    # sum_{i=0..6} C(10, i) endpoint-containing subsets of 12 points, |S| <= 8
    assert len(exact_dp.subsets(12, 8)) == sum(math.comb(10, i) for i in range(7)) == 848
    assert exact_dp.subsets(2, 8) == [(0, 1)]
    assert exact_dp.subsets(1, 8) == [(0,)]


def _blocks(count, n_tok=256):
    t = W.generate(W.FEATURE_GROUP_EXACT_FP32)
    return oblocks.partition(t, 256, 16)[:count]


def test_pair_decomposition_equals_direct_scoring(rng):
    """D(S), H(S) assembled from pair statistics equal the per-entry scoring
    of the subset's codebook."""
    for x in _blocks(4):
        xs = np.sort(x)
        A = exact_dp.alphabet(xs, 12)
        Dp, ML, MR = exact_dp.pair_stats(x, A)
        S_list = exact_dp.subsets(A.size, 8)
        for idx in rng.choice(len(S_list), size=40, replace=False):
            S = S_list[idx]
            D, H = exact_dp.subset_score(Dp, ML, MR, x.size, S)
            D2, H2, _ = ecasq.score_codebook(x, A[list(S)])
            assert D == pytest.approx(D2, rel=1e-10)
            assert H == pytest.approx(H2, rel=1e-12)


@pytest.mark.parametrize("lam", [0.0, 1e-4, 3e-3, 0.05, 1.0, 1e6])
def test_dp_equals_brute_force(lam):
    d = 4096.0
    for x in _blocks(6):
        xs = np.sort(x)
        A = exact_dp.alphabet(xs, 12)
        Dp, ML, MR = exact_dp.pair_stats(x, A)
        Dt, Ht, S_list = exact_dp.brute_force_tables(Dp, ML, MR, x.size, 8)
        obj = Dt + (lam * d) * Ht
        bf = int(np.argmin(obj))
        val, S = exact_dp.dp_minimise(Dp, ML, MR, x.size, d, lam, 8)
        assert val == pytest.approx(obj[bf], rel=1e-12, abs=1e-12)
        if S != S_list[bf]:
            # a different subset is allowed only on an exact tie
            other = S_list.index(S)
            assert obj[other] == pytest.approx(obj[bf], rel=1e-12)


def test_dp_on_tied_alphabet():
    """fp16-like ties collapse alphabet points (m < 12); the search still
    matches brute force."""
    rng = np.random.default_rng(3)
    x = np.round(rng.standard_normal(4096), 1)
    x[:2000] = 0.0
    A = exact_dp.alphabet(np.sort(x), 12)
    assert A.size < 12
    Dp, ML, MR = exact_dp.pair_stats(x, A)
    Dt, Ht, S_list = exact_dp.brute_force_tables(Dp, ML, MR, x.size, 8)
    for lam in (0.0, 0.01, 10.0):
        obj = Dt + (lam * 4096.0) * Ht
        val, S = exact_dp.dp_minimise(Dp, ML, MR, x.size, 4096.0, lam, 8)
        assert val == pytest.approx(obj.min(), rel=1e-12, abs=1e-12)


def test_dp_limited_size():
    """With |S| <= 3 only {A0, Aj, Am-1} chains are searched."""
    x = _blocks(1)[0]
    A = exact_dp.alphabet(np.sort(x), 12)
    Dp, ML, MR = exact_dp.pair_stats(x, A)
    Dt, Ht, S_list = exact_dp.brute_force_tables(Dp, ML, MR, x.size, 3)
    assert len(S_list) == 1 + 10
    val, S = exact_dp.dp_minimise(Dp, ML, MR, x.size, 4096.0, 0.0, 3)
    assert val == pytest.approx(Dt.min(), rel=1e-12)
    assert len(S) <= 3
