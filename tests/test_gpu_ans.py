"""Entropy coding (kvq_ans_encode / kvq_ans_decode) against the oracle's rANS
coder (oracle/ans.py), through the C ABI.

The GPU admits a workload as usual; its fixed-width codes are coded on the
GPU and, independently, by the oracle from the same codes.  Bars:
* every coded block is byte-identical to the oracle's coding of the block,
  and the block offsets equal the running sum of the oracle's block sizes;
* the GPU decode returns exactly codebook[code] for every entry;
* the stream's length is within the oracle's per-block overhead bound of the
  ideal length under each block's model.
The oracle codes every block of the small workloads and a sample of blocks
of the one-layer long-context workload.
"""

import sys

import numpy as np
import pytest

from kv_cache_rate_amd import workloads as W
from oracle import ans as oans
from oracle import codes as ocodes

from . import parity

pytestmark = pytest.mark.gpu


def _say(msg):
    print(f"[gpu-ans] {msg}", flush=True)
    sys.stdout.flush()


def _admit_and_code(w, tensors):
    import torch
    from kv_cache_rate_amd import kvq
    dev = parity.to_cuda(tensors)
    search = kvq.KVQ_GRIDS if w.search == "grids" else kvq.KVQ_EXACT_DP
    plan = kvq.kvq_plan_blocks(dev, w.tokens_per_block, w.dims_per_block, w.s, search,
                               w.alphabet_m if search else 0)
    buf = kvq.allocate(plan, dequant=True)
    mode = kvq.KVQ_BISECT if w.mode == "bisect" else kvq.KVQ_SUBGRAD
    kvq.admit(plan, dev, buf, w.B, mode, w.iters, w.eta, 0.0, w.seed, dequant=True)
    ab = kvq.allocate_ans(plan)
    total = kvq.kvq_ans_encode(plan, buf["codes"], buf["m"], buf["off"], ab["scratch"], ab["stream"],
                               ab["block_off"], buf["workspace"])
    xh = torch.full((plan.n_blocks, plan.d_block), float("nan"), dtype=torch.float32, device="cuda")
    kvq.kvq_ans_decode(plan, ab["stream"], ab["block_off"], buf["codebook"], buf["m"], xh,
                       buf["workspace"])
    torch.cuda.synchronize()
    ws = buf["workspace"][:4].cpu().numpy().view(np.uint32)[0]
    out = {
        "plan": plan, "total": total, "status": int(ws),
        "codes": buf["codes"].cpu().numpy().view(np.uint32),
        "off": buf["off"].cpu().numpy().view(np.uint64),
        "m": buf["m"].cpu().numpy().astype(np.int64),
        "codebook": buf["codebook"].cpu().numpy(),
        "xhat_fixed": buf["xhat"].cpu().numpy(),
        "stream": ab["stream"][:max(total, 1)].cpu().numpy(),
        "block_off": ab["block_off"].cpu().numpy().view(np.uint64),
        "xhat": xh.cpu().numpy(),
    }
    return out


def _compare(g, sample=None):
    plan = g["plan"]
    R, n = plan.n_blocks, plan.d_block
    boff = g["block_off"]
    assert boff[0] == 0 and boff[R] == g["total"]
    assert np.all(np.diff(boff.astype(np.int64)) > 0)
    assert g["status"] & 4 == 0, "a decoded block did not end at the start state"
    # decode equals the fixed-width path's decode (exact codepoints)
    assert np.array_equal(g["xhat"], g["xhat_fixed"])
    rows = range(R) if sample is None else sample
    ideal = 0.0
    for r in rows:
        m = int(g["m"][r])
        w = ocodes.code_width(m)
        seg = g["codes"][int(g["off"][r]):int(g["off"][r + 1])]
        cr = ocodes.unpack_block(seg, n, w)
        ref = oans.encode_block(cr, m)
        got = g["stream"][int(boff[r]):int(boff[r + 1])]
        assert np.array_equal(got, ref), r
        assert np.array_equal(oans.decode_block(got, m, n), cr), r
        ideal += oans.model_bits(cr, m) + 16 * m
    if sample is None:
        extra = 8 * g["total"] - ideal
        assert 0 <= extra <= R * (32 * oans.LANES + 16)
    return 8.0 * g["total"] / (R * n)


def test_tiny_all_blocks():
    w = W.TINY_K_FP32
    g = _admit_and_code(w, W.generate(w))
    bpe = _compare(g)
    _say(f"tiny: {bpe:.3f} coded bits/entry")


def test_prefill_sampled():
    w = W.PREFILL_KV_FP16
    g = _admit_and_code(w, W.generate(w))
    R = g["plan"].n_blocks
    rng = np.random.default_rng(11)
    sample = sorted(set([0, 1, R // 2, R - 1] + rng.integers(0, R, size=28).tolist()))
    bpe = _compare(g, sample)
    fixed = 32.0 * float(g["off"][-1]) / (R * g["plan"].d_block)
    _say(f"prefill: {bpe:.3f} coded bits/entry vs {fixed:.3f} fixed-width")
    assert bpe < fixed


def test_feature_group_all_blocks_sampled():
    w = W.FEATURE_GROUP_EXACT_FP32
    g = _admit_and_code(w, W.generate(w))
    R = g["plan"].n_blocks
    _compare(g, list(range(0, R, 97)) + [R - 1])


def test_ragged_and_constant_blocks():
    """96-entry blocks (k = 7, 2^k - n = 32 added to the top symbol) with
    fp16 ties, and constant blocks (one level: no codes, table only)."""
    rng = np.random.default_rng(13)
    x = (np.round(rng.standard_normal((5, 3, 9, 32)) * 2) / 2).astype(np.float16)
    x[1, 2] = 0.75
    w = W.Workload(name="ragged_ans", index=0, tensors=(("K", x.shape),), dtype="f16",
                   tokens_per_block=3, dims_per_block=32, s=6, search="grids", B=1.5,
                   mode="bisect")
    g = _admit_and_code(w, [x])
    assert (g["m"] == 1).any()
    _compare(g)


def test_long_context_one_layer_sampled():
    w = W.reduced(W.LONG_CONTEXT_KV_FP16, 1)
    g = _admit_and_code(w, W.generate(w))
    R = g["plan"].n_blocks
    rng = np.random.default_rng(12)
    sample = sorted(set([0, R // 2, R - 1] + rng.integers(0, R, size=21).tolist()))
    bpe = _compare(g, sample)
    _say(f"long-context layer: {bpe:.3f} coded bits/entry")
