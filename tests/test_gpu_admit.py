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
