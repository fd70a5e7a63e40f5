"""Exact codebook search over larger alphabets (32 quantiles, codebooks of
up to 16 points) on the GPU against the oracle, through the C ABI.

Brute force is out of reach here (over 10^8 subsets per block), so the
oracle solves with its pair-state DP route, which is pinned to brute force
on smaller alphabets in tests/test_oracle_dp.py.  Bars as in
tests/parity.py: pair statistics within 1e-4 relative, alphabets bit-exact,
the same multiplier, subsets identical except documented ties, codes
bit-exact except draws with |u - p| < 1e-6.
"""

import sys

import numpy as np
import pytest

from kv_cache_rate_amd import workloads as W
from oracle import blocks as oblocks
from oracle import codes as ocodes
from oracle import exact_dp, pipeline
from tests import parity

pytestmark = pytest.mark.gpu

WL = W.FEATURE_GROUP_EXACT_M32


def _say(msg):
    print(f"[gpu-dp-large] {msg}", flush=True)
    sys.stdout.flush()


def _kw(**over):
    kw = dict(tokens_per_block=WL.tokens_per_block, dims_per_block=WL.dims_per_block, s=WL.s,
              search="exact_dp", alphabet_m=WL.alphabet_m, B=WL.B, mode="bisect", iters=40,
              seed=WL.seed)
    kw.update(over)
    return kw


@pytest.mark.parametrize("B", [2.5, 1.5])
def test_slice_full_oracle(B):
    """One head x 1024 tokens of the feature-group tensor: 32 blocks, every
    output compared with the whole oracle pass."""
    x = np.ascontiguousarray(W.generate(WL)[0][:, :1, :1024, :])
    kw = _kw(B=B)
    _say(f"slice {x.shape} {kw}")
    g = parity.run_gpu([x], **kw)
    o = parity.run_oracle([x], **kw)
    assert o["route"] == "dp"
    rep = parity.full_compare(g, o, "exact_dp", kw["seed"], B, "bisect")
    _say(f"slice B={B}: {rep}")
    assert g["lam"] > 0.0 and np.all(g["m"] <= WL.s) and np.all(g["m"] >= 2)


@pytest.mark.parametrize("M", [24, 25])
def test_slice_table_boundary(M):
    """Alphabets of 24 points (the largest whose DP keeps its entropy terms
    in LDS tables) and 25 (the smallest that evaluates them per
    transition), on the 32-block slice against the whole oracle."""
    x = np.ascontiguousarray(W.generate(WL)[0][:, :1, :1024, :])
    kw = _kw(B=2.0, alphabet_m=M)
    g = parity.run_gpu([x], **kw)
    o = parity.run_oracle([x], **kw)
    assert o["route"] == "dp"
    rep = parity.full_compare(g, o, "exact_dp", kw["seed"], kw["B"], "bisect")
    _say(f"slice M={M}: {rep}")
    assert g["lam"] > 0.0


def test_ties_and_constant_blocks():
    """Values on a 0.1 grid (fewer than 32 distinct quantiles per block) and
    one constant block (a single level, no codes)."""
    rng = np.random.default_rng(21)
    x = np.round(rng.standard_normal((1, 2, 512, 32)), 1).astype(np.float32)
    x[0, 1, :256, :16] = 0.5
    kw = _kw(B=1.6, s=12)
    g = parity.run_gpu([x], **kw)
    o = parity.run_oracle([x], **kw)
    assert o["route"] == "dp"
    assert any(a.size < 32 for a in o["alphabets"])
    rep = parity.full_compare(g, o, "exact_dp", kw["seed"], kw["B"], "bisect")
    _say(f"ties: {rep}")
    const = 1 * 2 * 2 + 0  # head 1, chunk 0, group 0 in (outer, head, chunk, group) order
    assert g["m"][const] == 1 and int(g["off"][const + 1]) == int(g["off"][const])


def test_full_size_sampled():
    """All 2048 blocks on the GPU; on 64 sampled blocks the oracle's pair
    statistics, its DP minimiser at the GPU's multiplier and its codes."""
    t = W.generate(WL)
    kw = _kw()
    g = parity.run_gpu(t, **kw)
    R, n = g["m"].shape[0], WL.n
    assert g["rate_per_entry"] <= WL.B + 1e-12 and g["lam"] > 0.0
    rng = np.random.default_rng(22)
    sample = sorted(set([0, 1, R // 2, R - 1] + rng.integers(0, R, size=60).tolist()))
    blocks = np.stack([oblocks.block_of(t, WL.tokens_per_block, WL.dims_per_block, r) for r in sample])
    ev = pipeline.eval_pairs(blocks, WL.alphabet_m, pipeline.default_processes())
    o = {"n": n, "alphabets": [e[1] for e in ev], "pairs": [(e[2], e[3], e[4]) for e in ev]}
    o["subsets_chosen"] = [exact_dp.dp_minimise(*pr, n, float(n), g["lam"], WL.s)[1]
                           for pr in o["pairs"]]
    # pair statistics and alphabets
    M = WL.alphabet_m
    for k, r in enumerate(sample):
        assert np.array_equal(g["stats"][r].astype(np.float64), ev[k][0])
        Dp, ML, MR = o["pairs"][k]
        m = o["alphabets"][k].size
        for i in range(m):
            for j in range(i + 1, m):
                p = i * (2 * M - i - 1) // 2 + (j - i - 1)
                fl = 1e-9 * max(Dp.max(), 1e-300) / parity.D_RTOL
                assert abs(g["D"][r, p] - Dp[i, j]) <= parity.D_RTOL * max(abs(Dp[i, j]), fl)
                assert abs(g["H"][r, p, 0] - ML[i, j]) <= parity.D_RTOL * max(abs(ML[i, j]), 1e-9 / parity.D_RTOL)
                assert abs(g["H"][r, p, 1] - MR[i, j]) <= parity.D_RTOL * max(abs(MR[i, j]), 1e-9 / parity.D_RTOL)
    agree, ties, gap = parity.compare_choice_dp(g, o, g["lam"], float(n), blocks=sample)
    # codes of the sampled blocks: bit-exact away from |u - p| < 1e-6
    near_diff = 0
    for k, r in enumerate(sample):
        w = ocodes.code_width(int(g["m"][r]))
        seg = g["codes"][int(g["off"][r]):int(g["off"][r + 1])]
        cg = ocodes.unpack_block(seg, n, w)
        Q = g["codebook"][r, :int(g["m"][r])].astype(np.float64)
        co, nnear = ocodes.quantize_block(blocks[k], Q, WL.seed, r)
        diff = cg != co
        if diff.any():
            near = ocodes.near_mask(blocks[k], Q, WL.seed, r)
            assert np.all(near[diff]), f"block {r}: code differs away from |u-p|<1e-6"
            assert int(diff.sum()) <= nnear
            near_diff += int(diff.sum())
    _say(f"full size: lambda {g['lam']} rate {g['rate_per_entry']:.6f} sampled {len(sample)} "
         f"ties {ties} (max gap {gap:.2e}) near-draw code differences {near_diff}")
