"""kvq_admit_noalloc (kvq_admit with the library's static device scratch in
place of a caller workspace) against kvq_admit, through the C ABI, on two
calls in a row with the second input smaller than the first: every output
must be identical bit for bit."""

import sys

import numpy as np
import pytest

from kv_cache_rate_amd import workloads as W

pytestmark = pytest.mark.gpu


def _say(msg):
    print(f"[no_alloc] {msg}", file=sys.stderr, flush=True)


def _inputs(torch, w, outer=None):
    host = W.generate(w)
    if outer is not None:
        host = [h[:outer] for h in host]
    return [torch.from_numpy(np.ascontiguousarray(h)).cuda() for h in host]


def _compare(torch, kvq, dev, w, mode, lam0, B):
    plan = kvq.kvq_plan_blocks(dev, w.tokens_per_block, w.dims_per_block, w.s)
    a = kvq.allocate(plan)
    b = kvq.allocate(plan)
    for buf in (a, b):  # different stale contents in the two sets of outputs
        for k in ("choice", "codebook", "off", "codes"):
            buf[k].fill_(0 if buf is a else -1)
    lam_a, rate_a = kvq.kvq_admit(plan, dev, a, B, mode, w.iters, w.eta, lam0, w.seed)
    lam_b, rate_b = kvq.kvq_admit_noalloc(plan, dev, b, B, mode, w.iters, w.eta, lam0, w.seed)
    torch.cuda.synchronize()
    assert lam_a == lam_b and rate_a == rate_b, (lam_a, lam_b, rate_a, rate_b)
    for k in ("D", "H", "stats", "choice", "codebook", "m", "off"):
        assert torch.equal(a[k], b[k]), k
    words = int(a["off"][-1].item())
    assert torch.equal(a["codes"][:words], b["codes"][:words])
    return plan.n_blocks, lam_b


def test_noalloc_matches_admit_on_two_calls_in_a_row():
    import torch
    from kv_cache_rate_amd import kvq
    # first call: prefill K and V (8192 blocks, a multi-tile offset scan),
    # bisection at a budget that binds
    w1 = W.PREFILL_KV_FP16
    _say(f"call 1: {w1.name}, bisect, B=1.5")
    R1, lam1 = _compare(torch, kvq, _inputs(torch, w1), w1, kvq.KVQ_BISECT, 0.0, 1.5)
    assert R1 == 8192 and lam1 > 0.0
    # second call, smaller: 16 of the decode batch's 64 sequences (128
    # blocks), one subgradient step from a warm multiplier
    w2 = W.DECODE_ADMIT_FP16
    _say(f"call 2: {w2.name}[:16], subgrad")
    R2, _ = _compare(torch, kvq, _inputs(torch, w2, outer=16), w2, kvq.KVQ_SUBGRAD, 0.52, w2.B)
    assert R2 == 128
    # and once more in the bisection mode on the small input
    _say(f"call 3: {w2.name}[:16], bisect")
    R3, _ = _compare(torch, kvq, _inputs(torch, w2, outer=16), w2, kvq.KVQ_BISECT, 0.0, 1.5)
    assert R3 == 128


def test_prepared_noalloc_matches_admit():
    """The binding's prepared form of kvq_admit_noalloc (arguments
    marshalled once) over three decode steps from one multiplier: the same
    multipliers, rates and codes as kvq_admit."""
    import torch
    from kv_cache_rate_amd import kvq
    w = W.DECODE_ADMIT_FP16
    dev = _inputs(torch, w, outer=16)
    plan = kvq.kvq_plan_blocks(dev, w.tokens_per_block, w.dims_per_block, w.s)
    a, b = kvq.allocate(plan), kvq.allocate(plan)
    call = kvq.prepare_admit(plan, dev, b, w.B, kvq.KVQ_SUBGRAD, w.iters, w.eta, w.seed, noalloc=True)
    la = lb = 0.52
    for step in range(3):
        la, ra = kvq.kvq_admit(plan, dev, a, w.B, kvq.KVQ_SUBGRAD, w.iters, w.eta, la, w.seed)
        lb, rb = call(lb)
        torch.cuda.synchronize()
        assert la == lb and ra == rb, (step, la, lb)
        words = int(a["off"][-1].item())
        assert torch.equal(a["codes"][:words], b["codes"][:words]), step
