"""Decode attention over the quantized cache (kvq_decode_attention) against
the oracle (oracle/attention.py) on the GPU's own decoded cache.

The kernel reads only codes and codebooks and works in fp32; the oracle
decodes the same codes (kvq_dequantize's exact codepoints) and computes
softmax attention in fp64.  Bar: |o - o_ref| <= 2e-3 max|v| per output.
Derivation: a 128-term fp32 dot product carries a relative error below
128 * 2^-24 = 7.6e-6 of sum |q_i k_i|; with |scale q . k| below 64 here that
moves each score by < 5e-4, which changes every softmax weight by a factor
within exp(+-1e-3), so the output moves by < 2e-3 of the largest |v|.
"""

import sys

import numpy as np
import pytest

from kv_cache_rate_amd import workloads as W
from oracle import attention

from . import parity

pytestmark = pytest.mark.gpu


def _say(msg):
    print(f"[gpu-attn] {msg}", flush=True)
    sys.stdout.flush()


def _run(w, tensors, q_heads, seed=3):
    import torch
    from kv_cache_rate_amd import kvq
    dev = parity.to_cuda(tensors)
    plan = kvq.kvq_plan_blocks(dev, w.tokens_per_block, w.dims_per_block, w.s)
    buf = kvq.allocate(plan, dequant=True)
    kvq.admit(plan, dev, buf, w.B, kvq.KVQ_BISECT, w.iters, w.eta, 0.0, w.seed, dequant=True)
    outer, heads, T, D = tensors[0].shape
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((outer, q_heads, D)).astype(np.float32)
    qd = torch.from_numpy(q).cuda()
    out = torch.empty_like(qd)
    nb = kvq.kvq_decode_attention_workspace(plan, q_heads)
    work = torch.empty(nb, dtype=torch.uint8, device="cuda")
    scale = 1.0 / np.sqrt(D)
    kvq.kvq_decode_attention(plan, buf["codes"], buf["codebook"], buf["m"], buf["off"], qd, q_heads,
                             scale, out, work)
    torch.cuda.synchronize()
    xh = buf["xhat"].cpu().numpy().astype(np.float64)
    nbK = plan.tensor_blocks[0]
    K = xh[:nbK].reshape(outer, heads, T, D)
    V = xh[nbK:].reshape(outer, heads, T, D)
    ref = attention.decode_attention(K, V, q, scale)
    got = out.cpu().numpy().astype(np.float64)
    err = np.abs(got - ref).max()
    vmax = np.abs(V).max()
    _say(f"{w.name} q_heads={q_heads}: max |o - o_ref| = {err:.3g} (max|v| {vmax:.3g})")
    assert err <= 2e-3 * vmax
    return buf["m"].cpu().numpy()


@pytest.mark.parametrize("q_heads", [32, 64])
def test_prefill_cache(q_heads):
    """32 KV heads x 4096 tokens (K Gaussian with outlier channels, V
    Laplace); 1 and 2 query heads per KV head."""
    w = W.PREFILL_KV_FP16
    _run(w, W.generate(w), q_heads)


def test_long_context_layer_gqa():
    """One layer of the long-context cache: 8 KV heads x 32768 tokens, 32
    query heads (4 per KV head, the Llama-3-8B grouping)."""
    w = W.reduced(W.LONG_CONTEXT_KV_FP16, 1)
    _run(w, W.generate(w), 32)


def test_ragged_tail_split():
    """A token count that leaves a partial last split (3 x 16 + 5 chunks)."""
    rng = np.random.default_rng(21)
    x = rng.standard_normal((2, 2, 53 * 32, 128)).astype(np.float16)
    v = rng.laplace(size=(2, 2, 53 * 32, 128)).astype(np.float16)
    w = W.Workload(name="attn_ragged", index=0, tensors=(("K", x.shape), ("V", v.shape)),
                   dtype="f16", tokens_per_block=32, dims_per_block=128, s=16, search="grids",
                   B=2.0, mode="bisect")
    _run(w, [x, v], 8)


def test_narrow_and_constant_blocks():
    """Code widths 0 to 4 in one cache: constant chunks (one-point
    codebooks, no code words), chunks of two or three distinct values, and a
    low budget that pushes the rest to two or three points; K and V chunks
    of one token range get different widths."""
    rng = np.random.default_rng(22)
    shape = (2, 2, 37 * 32, 128)
    x = rng.standard_normal(shape).astype(np.float16)
    v = rng.laplace(size=shape).astype(np.float16)
    xc = x.reshape(2, 2, 37, 32, 128)
    vc = v.reshape(2, 2, 37, 32, 128)
    xc[0, 0, 3] = 0.5
    xc[1, 1, 36] = -2.0
    vc[0, 1, 0] = 1.25
    vc[1, 0, 20] = 0.0
    xc[0, 1, 7] = rng.choice(np.array([-1.0, 2.0], dtype=np.float16), size=(32, 128))
    vc[1, 1, 9] = rng.choice(np.array([-0.5, 0.25, 3.0], dtype=np.float16), size=(32, 128))
    w = W.Workload(name="attn_narrow", index=0, tensors=(("K", x.shape), ("V", v.shape)),
                   dtype="f16", tokens_per_block=32, dims_per_block=128, s=16, search="grids",
                   B=1.2, mode="bisect")
    m = _run(w, [x, v], 4)
    widths = set(int(np.ceil(np.log2(k))) for k in np.unique(m))
    _say(f"code widths {sorted(widths)}")
    assert widths == {0, 1, 2, 3, 4}
    _run(w, [x, v], 8)


@pytest.mark.parametrize("group", [3, 8])
def test_larger_and_odd_groups(group):
    """8 query heads per KV head (run as two passes of 4) and 3 (a pass of
    2 and one of 1): query head g reads KV head g // G."""
    rng = np.random.default_rng(23)
    x = rng.standard_normal((2, 2, 40 * 32, 128)).astype(np.float16)
    v = rng.laplace(size=(2, 2, 40 * 32, 128)).astype(np.float16)
    w = W.Workload(name=f"attn_g{group}", index=0, tensors=(("K", x.shape), ("V", v.shape)),
                   dtype="f16", tokens_per_block=32, dims_per_block=128, s=16, search="grids",
                   B=2.0, mode="bisect")
    _run(w, [x, v], 2 * group)
