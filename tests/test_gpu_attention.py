"""Decode attention over the quantized cache (kvq_decode_attention) against
the oracle (oracle/attention.py) on the GPU's own decoded cache.

The kernel reads only codes and codebooks and works in fp32; the oracle
decodes the same codes (kvq_dequantize's exact codepoints) and computes
softmax attention in fp64.  Every output is held to a bound worked out from
that case's own scores and values (``_fp32_bound``), not to a fixed fraction
of max|v|; the bound's premises are asserted on the same scores.

The bound follows the kernel's fp32 arithmetic (u = 2^-24; gamma_n =
n u / (1 - n u)).  Scores are kept in base-2 units, s_t = c q . k_t with
c = scale log2 e.
* Score of token t: the coefficient c q_i is rounded up to four times (scale
  and log2 e to fp32, their product, the product with q_i).  The 128-term
  dot product runs on the matrix cores: each 64-feature half is two chains
  of 32 one-term multiply-accumulate steps (each taken to round twice: the
  product, then the sum), the chains are added and then the halves, so
  |ds_t| <= gamma_70 S_t with S_t = c sum_i |q_i k_ti|.
* Weight of token t: 2^(s_t - m) for the running maximum m of the wave that
  holds the token (m may trail the wave's scores by up to 16), then
  rescaled by 2^(m_old - m_new) at every later move of that maximum (at
  most one per chunk, 8 chunks per wave), then at the wave and split
  merges.  The exponents telescope to s_t - M for the final maximum M,
  which is common to every token and cancels in the ratio, so only the
  score's own error and the subtractions' rounding remain: the latter adds
  up to at most u (|s_t - m_1| + (m_last - m_1)) <= u (2 (R + 2 dS) + 16)
  (R the range of the exact scores, dS the largest score error).  Every
  weight goes through at most 11 exp2 evaluations (20 are allowed for),
  each taken to be within 2 ulp (4 u) of 2^x.  Its relative error is then
  eps_t <= 2^(gamma_70 S_t + u (2 (R + 2 dS) + 16)) (1 + 4u)^20 - 1.
* Output: weights perturbed by (1 + eps_t) move o by at most
  sum_t w_t eps_t |v_t - o| / (1 - max eps).  A wave's weighted V sums are
  one multiply-accumulate chain over its 256 tokens (two roundings a step),
  with up to 8 rescalings, then the 4-wave merge and the split merge; its
  sum of weights is shorter.  So both sums have depth at most
  N = 512 + 8 + 4 + splits, adding gamma_N sum_t w_t |v_t| +
  (gamma_N + u) |o|, the last u for the division.
Second-order products stay below 1e-3 of the first-order terms (asserted),
so the sum is multiplied by 1.01.  The bound is a worst case; the observed
errors sit well inside it and the test logs the largest ratio.
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


U = 2.0 ** -24
LOG2E = 1.4426950408889634
SPLIT_CHUNKS = 32  # chunks (32-token blocks) per workgroup of the kernel (8 per wave)


def _gamma(n):
    assert n * U < 0.5
    return n * U / (1.0 - n * U)


def _fp32_bound(K, V, q, scale, ref):
    """Per-output bound on |o_kernel - o_ref| (module docstring), with its
    premises asserted on this case's scores.  ``K``, ``V``: decoded caches
    [outer, kv_heads, T, D] (fp64), ``q`` [outer, q_heads, D], ``ref`` the
    oracle's outputs."""
    O, Hk, T, D = K.shape
    Hq = q.shape[1]
    G = Hq // Hk
    chunks = T // 32
    splits = -(-chunks // SPLIT_CHUNKS)
    c = scale * LOG2E
    g70 = _gamma(70)
    gN = _gamma(512 + 8 + 4 + splits)
    bound = np.empty_like(ref)
    eps_max = 0.0
    for o in range(O):
        for g in range(Hq):
            h = g // G
            qv = q[o, g].astype(np.float64)
            s = c * (K[o, h] @ qv)                      # base-2 scores
            S = c * (np.abs(K[o, h]) @ np.abs(qv))
            R = float(s.max() - s.min())
            dS = g70 * float(S.max())
            # premises: no weight or rescaling factor leaves fp32's normal
            # range, so every exp2 result is a normal number
            assert np.all(np.isfinite(s)) and R + 2 * dS < 100.0, (o, g, R)
            eps = np.exp2(g70 * S + U * (2 * (R + 2 * dS) + 16)) * (1 + 4 * U) ** 20 - 1.0
            em = float(eps.max())
            eps_max = max(eps_max, em)
            assert em < 1e-3 and gN < 1e-3, (em, gN)
            p = np.exp((s - s.max()) / LOG2E)
            w = p / p.sum()
            Vh = V[o, h]
            r = ref[o, g]
            b1 = ((w * eps) @ np.abs(Vh - r)) / (1.0 - em)
            wv = w @ np.abs(Vh)
            bound[o, g] = 1.01 * (b1 + (gN + U) * (np.abs(r) + b1) + gN * (1 + 2 * em) * wv)
    return bound, eps_max


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
    err = np.abs(got - ref)
    bound, eps_max = _fp32_bound(K, V, q, scale, ref)
    ratio = float((err / bound).max())
    _say(f"{w.name} q_heads={q_heads}: max |o - o_ref| = {err.max():.3g}, largest error / bound "
         f"{ratio:.3g} (bound {bound.min():.3g} .. {bound.max():.3g}, max weight error {eps_max:.3g})")
    assert np.all(err <= bound), ratio
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


@pytest.mark.parametrize("group", [3, 5, 8])
def test_larger_and_odd_groups(group):
    """8 query heads per KV head (run as two passes of 4), 5 (a pass of 4
    and one of 1) and 3 (one pass with a row unused): query head g reads KV
    head g // G."""
    rng = np.random.default_rng(23)
    x = rng.standard_normal((2, 2, 40 * 32, 128)).astype(np.float16)
    v = rng.laplace(size=(2, 2, 40 * 32, 128)).astype(np.float16)
    w = W.Workload(name=f"attn_g{group}", index=0, tensors=(("K", x.shape), ("V", v.shape)),
                   dtype="f16", tokens_per_block=32, dims_per_block=128, s=16, search="grids",
                   B=2.0, mode="bisect")
    _run(w, [x, v], 2 * group)
