"""Beam search over ordered codepoints (KVQ_BEAM) on the GPU against the
oracle's beam (oracle/exact_dp.py, beam_minimise), through the C ABI.

Bars as in tests/parity.py: alphabets bit-exact, pair statistics within
1e-4 relative, the same multiplier, the same subsets except documented
ties, codes bit-exact except draws with |u - p| < 1e-6.
"""

import sys

import numpy as np
import pytest

from kv_cache_rate_amd import workloads as W
from oracle import blocks as oblocks
from oracle import exact_dp, pipeline
from tests import parity

pytestmark = pytest.mark.gpu

FG = W.FEATURE_GROUP_EXACT_FP32


def _say(msg):
    print(f"[gpu-beam] {msg}", flush=True)
    sys.stdout.flush()


def _kw(**over):
    kw = dict(tokens_per_block=256, dims_per_block=16, s=16, search="beam", alphabet_m=32, B=2.5,
              mode="bisect", iters=40, seed=0, beam_width=4)
    kw.update(over)
    return kw


@pytest.mark.parametrize("width,B", [(1, 2.5), (4, 2.5), (8, 1.5)])
def test_slice_full_oracle(width, B):
    """One head x 1024 tokens of the feature-group tensor (32 blocks),
    32-quantile alphabet, |Q| <= 16: every output against the whole oracle
    pass."""
    x = np.ascontiguousarray(W.generate(FG)[0][:, :1, :1024, :])
    kw = _kw(beam_width=width, B=B)
    _say(f"slice {kw}")
    g = parity.run_gpu([x], **kw)
    o = parity.run_oracle([x], **kw)
    assert o["route"] == "beam"
    rep = parity.full_compare(g, o, "beam", kw["seed"], B, "bisect")
    _say(f"slice width={width} B={B}: {rep}")


def test_ties_and_constant_blocks():
    rng = np.random.default_rng(31)
    x = np.round(rng.standard_normal((1, 2, 512, 32)), 1).astype(np.float32)
    x[0, 0, 256:, 16:] = -1.25
    kw = _kw(B=1.7, s=12, beam_width=3)
    g = parity.run_gpu([x], **kw)
    o = parity.run_oracle([x], **kw)
    assert any(a.size < 32 for a in o["alphabets"])
    rep = parity.full_compare(g, o, "beam", kw["seed"], kw["B"], "bisect")
    _say(f"ties: {rep}")
    const = 3  # head 0, chunk 1, group 1
    assert g["m"][const] == 1 and int(g["off"][const + 1]) == int(g["off"][const])


def test_feature_group_full_size_sampled():
    """All 2048 feature-group blocks with the 12-quantile alphabet, |Q| <= 8
    and width 2; on 64 sampled blocks the oracle's beam at the GPU's
    multiplier gives the same subsets."""
    t = W.generate(FG)
    kw = _kw(s=8, alphabet_m=12, beam_width=2)
    g = parity.run_gpu(t, **kw)
    R, n = g["m"].shape[0], FG.n
    assert g["rate_per_entry"] <= kw["B"] + 1e-12 and g["lam"] > 0.0
    rng = np.random.default_rng(32)
    sample = sorted(set([0, 1, R // 2, R - 1] + rng.integers(0, R, size=60).tolist()))
    blocks = np.stack([oblocks.block_of(t, 256, 16, r) for r in sample])
    ev = pipeline.eval_pairs(blocks, 12, pipeline.default_processes())
    o = {"n": n, "alphabets": [e[1] for e in ev], "pairs": [(e[2], e[3], e[4]) for e in ev]}
    o["subsets_chosen"] = [exact_dp.beam_minimise(*pr, n, float(n), g["lam"], 8, 2)[1] for pr in o["pairs"]]
    for k, r in enumerate(sample):
        assert np.array_equal(g["stats"][r].astype(np.float64), ev[k][0])
    agree, ties, gap = parity.compare_choice_dp(g, o, g["lam"], float(n), blocks=sample)
    exact = sum(exact_dp.dp_minimise(*pr, n, float(n), g["lam"], 8)[1] == S
                for pr, S in zip(o["pairs"], o["subsets_chosen"]))
    _say(f"full size: lambda {g['lam']} rate {g['rate_per_entry']:.6f} ties {ties} "
         f"beam = exact DP on {exact}/{len(sample)} sampled blocks")
