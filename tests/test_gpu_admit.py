"""kvq_admit (eval, solve and quantize_pack in one call, one wait) against
the same three steps called one by one, on the same seeded inputs and
through the C ABI: every output must be identical bit for bit."""

import numpy as np
import pytest

from kv_cache_rate_amd import workloads as W

pytestmark = pytest.mark.gpu


def _run(kvq, torch, w, mode, lam0, fused):
    dev = [torch.from_numpy(np.ascontiguousarray(h)).cuda()
           for h in W.generate(w, which=1 if w.name.startswith("decode") else 0)]
    plan = kvq.kvq_plan_blocks(dev, w.tokens_per_block, w.dims_per_block, w.s)
    buf = kvq.allocate(plan)
    if fused:
        lam, rate = kvq.kvq_admit(plan, dev, buf, w.B, mode, w.iters, w.eta, lam0, w.seed)
    else:
        lam, rate = kvq.admit(plan, dev, buf, w.B, mode, w.iters, w.eta, lam0, w.seed)
    torch.cuda.synchronize()
    return lam, rate, buf


@pytest.mark.parametrize("name,mode,lam0", [("decode_admit_fp16", 1, 0.52), ("prefill_kv_fp16", 0, 0.0),
                                            ("tiny_k_fp32", 0, 0.0)])
def test_admit_matches_the_three_calls(name, mode, lam0):
    import torch
    from kv_cache_rate_amd import kvq
    w = W.BY_NAME[name]
    if name == "tiny_k_fp32":
        w = W.Workload(**{**w.__dict__, "B": 1.0})  # a binding budget
    lam_a, rate_a, a = _run(kvq, torch, w, mode, lam0, fused=False)
    lam_b, rate_b, b = _run(kvq, torch, w, mode, lam0, fused=True)
    assert lam_a == lam_b and rate_a == rate_b, (lam_a, lam_b, rate_a, rate_b)
    for k in ("D", "H", "stats", "choice", "codebook", "m", "off"):
        assert torch.equal(a[k], b[k]), k
    words = int(a["off"][-1].item())
    assert torch.equal(a["codes"][:words], b["codes"][:words])


def test_admit_reports_nonfinite_input():
    import torch
    from kv_cache_rate_amd import kvq
    x = np.random.default_rng(9).standard_normal((4, 8, 32, 128)).astype(np.float16)
    x[2, 3, 5, 7] = np.inf
    dev = [torch.from_numpy(x).cuda()]
    plan = kvq.kvq_plan_blocks(dev, 32, 128, 16)
    buf = kvq.allocate(plan)
    with pytest.raises(kvq.KvqError) as ei:
        kvq.kvq_admit(plan, dev, buf, 2.0, kvq.KVQ_SUBGRAD, 40, 1e-3, 0.3, 0)
    assert ei.value.status == kvq.KVQ_ENONFINITE


@pytest.mark.parametrize("outer,heads,tensors", [(1, 1, 1), (64, 8, 1), (32, 8, 2), (128, 8, 1), (5, 205, 1)])
def test_one_launch_admission_matches_the_three_calls(outer, heads, tensors):
    """Subgradient admission of fp16 head x 32-token blocks: up to 1024
    blocks take the one-launch kernel (score, choose at lambda, offsets by
    look-back, quantize, pack); 1025 blocks (5 x 205) take the three-step
    path.  Every output equals the three calls', bit for bit, from 1 block
    to 1024 and with K and V."""
    import torch
    from kv_cache_rate_amd import kvq
    rng = np.random.default_rng(1000 + outer * heads * tensors)
    xs = [(rng.standard_t(5.0, size=(outer, heads, 32, 128))).astype(np.float16) for _ in range(tensors)]
    dev = [torch.from_numpy(x).cuda() for x in xs]
    plan = kvq.kvq_plan_blocks(dev, 32, 128, 16)
    a = kvq.allocate(plan)
    b = kvq.allocate(plan)
    for k in ("choice", "codebook", "off", "codes"):
        b[k].fill_(-1)
    lam0 = 0.37
    lam_a, rate_a = kvq.admit(plan, dev, a, 2.0, kvq.KVQ_SUBGRAD, 40, 1e-3, lam0, 11)
    lam_b, rate_b = kvq.kvq_admit(plan, dev, b, 2.0, kvq.KVQ_SUBGRAD, 40, 1e-3, lam0, 11)
    torch.cuda.synchronize()
    assert lam_a == lam_b and rate_a == rate_b, (lam_a, lam_b, rate_a, rate_b)
    for k in ("D", "H", "stats", "choice", "codebook", "m", "off"):
        assert torch.equal(a[k], b[k]), k
    words = int(a["off"][-1].item())
    assert torch.equal(a["codes"][:words], b["codes"][:words])
    # and the next step from the returned multiplier agrees as well
    lam_a2, _ = kvq.admit(plan, dev, a, 2.0, kvq.KVQ_SUBGRAD, 40, 1e-3, lam_a, 12)
    lam_b2, _ = kvq.kvq_admit(plan, dev, b, 2.0, kvq.KVQ_SUBGRAD, 40, 1e-3, lam_b, 12)
    torch.cuda.synchronize()
    assert lam_a2 == lam_b2
    words = int(a["off"][-1].item())
    assert torch.equal(a["codes"][:words], b["codes"][:words])


def test_one_launch_admission_ties_and_constant_blocks():
    """The one-launch admission on blocks whose candidates tie (a constant
    block, an all-zero block, blocks of two and three distinct values: many
    candidates then share their codebook, D and H, and the lowest index must
    win) and whose codebooks merge equal points: every output equals the
    three calls', bit for bit."""
    import torch
    from kv_cache_rate_amd import kvq
    rng = np.random.default_rng(77)
    x = rng.standard_t(5.0, size=(2, 8, 32, 128)).astype(np.float16)
    x[0, 0] = np.float16(0.5)
    x[0, 1] = np.float16(0.0)
    x[0, 2] = rng.choice(np.array([-1.0, 1.0], dtype=np.float16), size=(32, 128))
    x[0, 3] = rng.choice(np.array([-2.0, 0.25, 3.0], dtype=np.float16), size=(32, 128))
    x[1, 5, :16] = np.float16(-0.75)  # half the block on one value
    dev = [torch.from_numpy(x).cuda()]
    plan = kvq.kvq_plan_blocks(dev, 32, 128, 16)
    a = kvq.allocate(plan)
    b = kvq.allocate(plan)
    for lam0 in (0.0, 0.37, 5.0):
        lam_a, rate_a = kvq.admit(plan, dev, a, 2.0, kvq.KVQ_SUBGRAD, 40, 1e-3, lam0, 5)
        lam_b, rate_b = kvq.kvq_admit(plan, dev, b, 2.0, kvq.KVQ_SUBGRAD, 40, 1e-3, lam0, 5)
        torch.cuda.synchronize()
        assert lam_a == lam_b and rate_a == rate_b, (lam0, lam_a, lam_b, rate_a, rate_b)
        for k in ("D", "H", "stats", "choice", "codebook", "m", "off"):
            assert torch.equal(a[k], b[k]), (lam0, k)
        words = int(a["off"][-1].item())
        assert torch.equal(a["codes"][:words], b["codes"][:words]), lam0
    assert int(a["m"][0].item()) == 1 and int(a["m"][1].item()) == 1


def test_one_launch_admission_ignores_stale_workspace_words():
    """Nothing clears the one-launch admission's published words between
    launches: each carries its launch's epoch.  A workspace filled with
    words that look published (all bits set), and one left by a launch whose
    input held an Inf (its status bit must not leak into the next launch),
    must both give the three calls' outputs bit for bit."""
    import torch
    from kv_cache_rate_amd import kvq
    rng = np.random.default_rng(31)
    x = rng.standard_t(5.0, size=(16, 8, 32, 128)).astype(np.float16)
    bad = x.copy()
    bad[3, 2, 1, 0] = np.inf
    dev, dev_bad = [torch.from_numpy(x).cuda()], [torch.from_numpy(bad).cuda()]
    plan = kvq.kvq_plan_blocks(dev, 32, 128, 16)
    a = kvq.allocate(plan)
    b = kvq.allocate(plan)
    lam_a, rate_a = kvq.admit(plan, dev, a, 2.0, kvq.KVQ_SUBGRAD, 40, 1e-3, 0.4, 3)
    for prep in ("ones", "nonfinite"):
        if prep == "ones":
            b["workspace"].fill_(255)
        else:
            with pytest.raises(kvq.KvqError) as ei:
                kvq.kvq_admit(plan, dev_bad, b, 2.0, kvq.KVQ_SUBGRAD, 40, 1e-3, 0.4, 3)
            assert ei.value.status == kvq.KVQ_ENONFINITE
        for k in ("choice", "codebook", "off", "codes"):
            b[k].fill_(-1)
        lam_b, rate_b = kvq.kvq_admit(plan, dev, b, 2.0, kvq.KVQ_SUBGRAD, 40, 1e-3, 0.4, 3)
        torch.cuda.synchronize()
        assert lam_a == lam_b and rate_a == rate_b, (prep, lam_a, lam_b, rate_a, rate_b)
        for k in ("D", "H", "stats", "choice", "codebook", "m", "off"):
            assert torch.equal(a[k], b[k]), (prep, k)
        words = int(a["off"][-1].item())
        assert torch.equal(a["codes"][:words], b["codes"][:words]), prep


def test_prepared_admit_matches_kvq_admit(noalloc=False):
    """prepare_admit (arguments marshalled once, the multiplier carried from
    step to step) gives kvq_admit's multipliers, rates and codes bit for bit
    over a short decode loop whose input changes every step."""
    import torch
    from kv_cache_rate_amd import kvq
    w = W.DECODE_ADMIT_FP16
    batches = [[torch.from_numpy(x).cuda() for x in W.generate(w, which=b)] for b in range(2)]
    cur = [torch.empty_like(t) for t in batches[0]]
    plan = kvq.kvq_plan_blocks(cur, w.tokens_per_block, w.dims_per_block, w.s)
    a, b = kvq.allocate(plan), kvq.allocate(plan)
    call = kvq.prepare_admit(plan, cur, b, w.B, kvq.KVQ_SUBGRAD, w.iters, w.eta, w.seed, noalloc=noalloc)
    la = lb = 0.52
    for step in range(4):
        for t, src in zip(cur, batches[step % 2]):
            t.copy_(src)
        la, ra = kvq.kvq_admit(plan, cur, a, w.B, kvq.KVQ_SUBGRAD, w.iters, w.eta, la, w.seed)
        lb, rb = call(lb)
        torch.cuda.synchronize()
        assert la == lb and ra == rb, (step, la, lb, ra, rb)
        for k in ("choice", "m", "off", "codebook"):
            assert torch.equal(a[k], b[k]), (step, k)
        assert torch.equal(a["codes"][:int(a["off"][-1])], b["codes"][:int(b["off"][-1])]), step
