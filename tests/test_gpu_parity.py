"""GPU parity: the HIP library (through its C ABI) against the oracle on the
same seeded inputs.  Bars are listed in tests/parity.py."""

import sys

import numpy as np
import pytest

from kv_cache_rate_amd import workloads as W
from oracle import blocks as oblocks
from oracle import ecasq
from tests import parity

pytestmark = pytest.mark.gpu


@pytest.fixture(params=["fast", "generic"])
def kernel_path(request, monkeypatch):
    """Run a case through the specialised kernels (fp16 sort-free eval,
    4096-entry quantize/decode) and through the generic ones."""
    if request.param == "generic":
        monkeypatch.setenv("KVQ_FORCE_GENERIC", "1")
    else:
        monkeypatch.delenv("KVQ_FORCE_GENERIC", raising=False)
    return request.param


def _say(msg):
    print(f"[gpu-parity] {msg}", flush=True)
    sys.stdout.flush()


def _kw(w, **over):
    kw = dict(tokens_per_block=w.tokens_per_block, dims_per_block=w.dims_per_block, s=w.s,
              search=w.search, alphabet_m=w.alphabet_m, B=w.B, mode=w.mode, iters=w.iters,
              eta=w.eta, seed=w.seed)
    kw.update(over)
    return kw


def _check(w, tensors, **over):
    kw = _kw(w, **over)
    _say(f"{w.name} {kw}")
    g = parity.run_gpu(tensors, **kw)
    o = parity.run_oracle(tensors, **kw)
    rep = parity.full_compare(g, o, kw["search"], kw["seed"], kw["B"], kw["mode"])
    _say(f"{w.name} report {rep}")
    return g, o, rep


@pytest.mark.parametrize("B", [3.0, 0.8, 1.0, 1.2])
def test_tiny_k_fp32(B, kernel_path):
    w = W.TINY_K_FP32
    g, o, rep = _check(w, W.generate(w), B=B)
    if B == 3.0:
        assert g["lam"] == 0.0  # log2 8 = 3 bits per entry never binds
    else:
        assert g["lam"] > 0.0


def test_prefill_kv_fp16(kernel_path):
    w = W.PREFILL_KV_FP16
    _check(w, W.generate(w))


def test_decode_admission_subgradient(kernel_path):
    """Previous batch: bisection gives lambda_prev; measured batch: choose at
    lambda_prev, one projected subgradient step (eta = 1e-3)."""
    w = W.DECODE_ADMIT_FP16
    prev = W.generate(w, which=0)
    g0, o0, _ = _check(w, prev, mode="bisect", seed=w.extra["prev_seed"])
    cur = W.generate(w, which=1)
    # each side continues from its own multiplier
    kw = _kw(w, mode="subgrad", seed=w.seed)
    _say(f"subgrad step from lambda_prev gpu={g0['lam']!r} oracle={o0['lam']!r}")
    g1 = parity.run_gpu(cur, **{**kw, "lam": g0["lam"]})
    o1 = parity.run_oracle(cur, **{**kw, "lam": o0["lam"]})
    rep = parity.full_compare(g1, o1, "grids", w.seed, w.B, "subgrad")
    _say(f"subgrad report {rep}")
    assert g1["rate_per_entry"] == pytest.approx(o1["rate_per_entry"], rel=1e-6)
    # lambda_next = lambda_prev + eta (Rbar - B): differences stay within the
    # inputs' differences
    tol = abs(g0["lam"] - o0["lam"]) + w.eta * 1e-6 * abs(o1["rate_per_entry"]) + 1e-15
    assert abs(g1["lam"] - o1["lam"]) <= tol


def test_feature_group_exact_dp():
    w = W.FEATURE_GROUP_EXACT_FP32
    g, o, rep = _check(w, W.generate(w))
    # the GPU's pair-state DP agrees with brute force on the first 64 blocks
    assert np.array_equal(g["choice"][:64].astype(np.int64), o["mask"][:64]) or rep["ties"] > 0


def test_tiny_k_fp32_scaled_to_1e33(kernel_path):
    """The tiny fp32 workload times 1e-33: codepoints ~1e-33 apart, so 2^24
    over an interval width overflows fp32 and the specialised quantizer must
    divide instead (codes bit-exact away from |u - p| < 1e-6)."""
    w = W.TINY_K_FP32
    x = [(a * np.float32(1e-33)).astype(np.float32) for a in W.generate(w)]
    assert np.all(np.isfinite(x[0])) and np.abs(x[0]).max() < 1e-31
    g, o, rep = _check(w, x, B=3.0)
    assert g["lam"] == 0.0


def test_long_context_one_layer_binding_budget(kernel_path):
    """One layer of the long-context workload at B = 1.5, where the budget
    binds: the whole bisection, the final choice and the codes against the
    whole oracle."""
    w = W.reduced(W.LONG_CONTEXT_KV_FP16, 1)
    g, o, rep = _check(w, W.generate(w), B=1.5)
    assert g["lam"] > 0.0


def test_long_context_one_layer(kernel_path):
    """The long-context workload reduced to one layer of K and V (16384
    blocks), same per-layer streams as the full tensors."""
    w = W.reduced(W.LONG_CONTEXT_KV_FP16, 1)
    _check(w, W.generate(w))


# ------------------------------------------------------------ edge cases ---

def _small(dtype, shape, rng, kind="normal"):
    if kind == "normal":
        x = rng.standard_normal(shape)
    elif kind == "ties":
        x = np.round(rng.standard_normal(shape) * 2) / 2
    elif kind == "const":
        x = np.full(shape, 0.75)
    return x.astype(dtype)


@pytest.mark.parametrize("dtype", [np.float16, np.float32])
def test_ragged_small_blocks(dtype):
    """Blocks of 3 tokens x 32 features (96 entries: not a power of two),
    R = 5 x 3 x 3 = 45 blocks (not a multiple of any workgroup tile)."""
    rng = np.random.default_rng(5)
    x = _small(dtype, (5, 3, 9, 32), rng)
    w = W.Workload(name="ragged", index=0, tensors=(("K", x.shape),), dtype="f16",
                   tokens_per_block=3, dims_per_block=32, s=6, search="grids", B=1.5,
                   mode="bisect")
    _check(w, [x])


@pytest.mark.parametrize("T,D,dtype,kind", [(5, 40, np.float32, "normal"), (10, 30, np.float16, "ties"),
                                              (8, 125, np.float32, "normal"), (12, 128, np.float16, "normal"),
                                              (31, 128, np.float32, "ties")])
def test_generic_sort_block_sizes(T, D, dtype, kind):
    """The generic kernels' register sort at every keys-per-thread count:
    blocks of 200, 300, 1000, 1536 and 3968 entries (padded to 256, 512,
    1024, 2048 and 4096 keys: 1, 2, 4, 8 and 16 per thread), with tied data
    in two of them, against the oracle."""
    rng = np.random.default_rng(7 + T * D)
    x = _small(dtype, (2, 3, 2 * T, 2 * D), rng, kind)
    w = W.Workload(name=f"sort{T}x{D}", index=0, tensors=(("K", x.shape),),
                   dtype="f16" if dtype == np.float16 else "f32",
                   tokens_per_block=T, dims_per_block=D, s=16, search="grids", B=1.7, mode="bisect")
    _check(w, [x])


@pytest.mark.parametrize("mode", ["bisect", "subgrad"])
@pytest.mark.parametrize("heads", [64, 65])
def test_final_pass_block_count_edges(heads, mode):
    """16 blocks per head of 2 x 16 entries: 1024 blocks (the most the
    few-block final pass takes: 16 workgroups of 64 and a 1024-thread scan)
    and 1040 (the many-block path), under bisection and a subgradient
    step."""
    rng = np.random.default_rng(53 + heads)
    x = _small(np.float32, (1, heads, 32, 16), rng)
    w = W.Workload(name=f"edge{heads}", index=0, tensors=(("K", x.shape),), dtype="f32",
                   tokens_per_block=2, dims_per_block=16, s=8, search="grids", B=1.8, mode=mode)
    g, o, rep = _check(w, [x], lam=0.21)
    assert g["m"].shape == (heads * 16,)


def test_ties_constant_and_negative_zero(kernel_path):
    """fp16 ties (fewer distinct levels than k), constant blocks (one level,
    zero-width codes) and -0 entries (equal to +0)."""
    rng = np.random.default_rng(6)
    x = _small(np.float16, (2, 2, 64, 128), rng, "ties")
    x[0, 0, :32] = np.float16(0.75)          # constant block
    x[1, 1, 32:, :64] = np.float16(-0.0)     # -0 entries
    x[1, 1, 32:, 64:] = np.float16(0.0)
    w = W.Workload(name="ties", index=0, tensors=(("K", x.shape),), dtype="f16",
                   tokens_per_block=32, dims_per_block=128, s=16, search="grids", B=1.0,
                   mode="bisect")
    g, o, rep = _check(w, [x])
    assert g["m"][0] == 1 and g["off"][1] == 0


def test_fp16_range_extremes(kernel_path):
    """The ends of the fp16 range: blocks of subnormals only (the lowest
    binade, where a value is its mantissa times 2^-24), subnormals mixed with
    small normals, magnitudes log-uniform over 2^-24 .. 65504 with both
    extremes present, values packed just below 65504, the three levels
    {-65504, 0, 65504}, and negative subnormals with -0; two Gaussian
    blocks as a control."""
    rng = np.random.default_rng(61)
    T, D = 32, 128
    sub = rng.integers(1, 1024, size=(T, D)) * 2.0 ** -24          # subnormal magnitudes
    sgn = rng.choice([-1.0, 1.0], size=(T, D))
    blocks = [
        sgn * sub,
        sgn * np.where(rng.random((T, D)) < 0.5, sub, np.exp2(rng.uniform(-14.0, -10.0, (T, D)))),
        sgn * np.exp2(rng.uniform(-24.0, np.log2(65504.0), (T, D))),
        rng.uniform(32768.0, 65504.0, (T, D)),
        rng.choice([-65504.0, 0.0, 65504.0], size=(T, D)),
        -sub * (rng.random((T, D)) < 0.7),
        rng.standard_normal((T, D)),
        rng.standard_normal((T, D)) * 3.0,
    ]
    blocks[2][0, :4] = [65504.0, -65504.0, 2.0 ** -24, -(2.0 ** -24)]
    blocks[2][1, :2] = [2.0 ** -14, -(2.0 ** -14)]                   # smallest normals
    x = np.stack(blocks)[None].astype(np.float16)                     # (1, 8, 32, 128)
    assert np.isfinite(x).all()
    assert (x.view(np.uint16)[0, 5] == 0x8000).any()                  # -0 present
    w = W.Workload(name="fp16_extremes", index=0, tensors=(("K", x.shape),), dtype="f16",
                   tokens_per_block=T, dims_per_block=D, s=16, search="grids", B=1.5,
                   mode="bisect")
    g, o, rep = _check(w, [x])
    assert g["m"].shape == (8,)
    assert g["m"][4] <= 3  # three distinct levels


@pytest.mark.parametrize("dtype,s,B,mode", [(np.float16, 16, 1.0, "bisect"), (np.float32, 8, 1.2, "bisect"),
                                             (np.float16, 16, 2.0, "subgrad")])
def test_single_block(dtype, s, B, mode):
    """One block (R = 1): the solve's single-workgroup path, the bisection
    on one block, and a subgradient step from a nonzero multiplier."""
    rng = np.random.default_rng(41)
    x = (rng.standard_normal((1, 1, 32, 128)) * 1.5).astype(dtype)
    w = W.Workload(name="single", index=0, tensors=(("K", x.shape),), dtype="f16" if dtype == np.float16 else "f32",
                   tokens_per_block=32, dims_per_block=128, s=s, search="grids", B=B, mode=mode)
    g, o, rep = _check(w, [x], lam=0.37)
    assert g["m"].shape == (1,)
    if mode == "bisect":
        assert g["lam"] > 0.0 and g["rate_per_entry"] <= B


def test_many_threshold_bins(kernel_path):
    """Log-uniform fp16 data (magnitudes over 2^-11 .. 2^11, random signs):
    the order statistics and the uniform thresholds of a block fall in
    about 127 distinct coarse bins, more than a large launch holds at
    once; this small launch holds all 144 and scores them in one round
    (the two-round case is the next test)."""
    rng = np.random.default_rng(43)
    mag = np.exp2(rng.uniform(-11.0, 11.0, size=(1, 4, 128, 128)))
    x = (mag * rng.choice([-1.0, 1.0], size=mag.shape)).astype(np.float16)
    w = W.Workload(name="many_bins", index=0, tensors=(("K", x.shape),), dtype="f16",
                   tokens_per_block=32, dims_per_block=128, s=16, search="grids", B=1.5,
                   mode="bisect")
    _check(w, [x])


def _fp16_keys(v):
    """Order-preserving 16-bit keys of fp16 values (-0 as +0)."""
    h = np.asarray(v, dtype=np.float16).view(np.uint16).astype(np.int64)
    h = np.where(h == 0x8000, 0, h)
    return np.where(h & 0x8000, 0xFFFF ^ h, h | 0x8000)


def _key_value(key):
    h = (key & 0x7FFF) if key & 0x8000 else (0xFFFF ^ key)
    return float(np.array([h], dtype=np.uint16).view(np.float16)[0])


def _claimed_bins(x, s):
    """Coarse bins (top 10 key bits) that the fp16 scoring kernel gives a
    slot: every bin holding an order statistic, and every bin holding data
    and the smallest fp16 key at or above a uniform threshold."""
    flat = np.asarray(x, dtype=np.float16).ravel()
    data_bins = set((_fp16_keys(flat) >> 6).tolist())
    xs = np.sort(flat.astype(np.float64))
    stats = xs[ecasq.quantile_ranks(xs.size, s)]
    claimed = set((_fp16_keys(stats) >> 6).tolist())
    for k in range(3, s + 1):
        for t in ecasq.uniform_points(xs[0], xs[-1], k)[1:-1]:
            key = int(_fp16_keys(np.float16(t)))
            if _key_value(key) < t:
                key += 1
            if (key >> 6) in data_bins:
                claimed.add(key >> 6)
    return claimed


def test_two_slot_rounds_in_large_launches():
    """16384 log-uniform fp16 blocks: a launch this large holds 112 slots
    per block, and these blocks claim more (checked here from the oracle's
    points), so the scoring kernel finishes them in two rounds.  The
    eval tables of sampled blocks are compared with the oracle's."""
    import torch
    from kv_cache_rate_amd import kvq
    rng = np.random.default_rng(47)
    shape = (2, 8, 32768, 128)
    x = np.exp2(rng.uniform(-11.0, 11.0, size=shape)).astype(np.float16)
    x *= rng.choice(np.array([-1.0, 1.0], dtype=np.float16), size=shape)
    t = [torch.from_numpy(x).cuda()]
    plan = kvq.kvq_plan_blocks(t, 32, 128, 16)
    R = plan.n_blocks
    assert R == 16384
    buf = kvq.allocate(plan)
    _say(f"two slot rounds: eval of {R} blocks")
    kvq.kvq_eval_candidates(plan, t, buf["D"], buf["H"], buf["stats"], buf["workspace"])
    torch.cuda.synchronize()
    D = buf["D"].cpu().numpy()
    H = buf["H"].cpu().numpy()
    stats = buf["stats"].cpu().numpy()
    sample = sorted(set([0, 1, R // 2, R - 1] + rng.integers(0, R, size=44).tolist()))
    over = 0
    for r in sample:
        xb = oblocks.block_of([x], 32, 128, r)
        if len(_claimed_bins(xb, 16)) > 112:
            over += 1
        Do, Ho, So, _ = ecasq.eval_block(xb.astype(np.float64), 16)
        floor = 1e-9 * max(Do.max(), 1e-300) / parity.D_RTOL
        eD = np.max(np.abs(D[:, r] - Do) / np.maximum(np.abs(Do), floor))
        eH = np.max(np.abs(H[:, r] - Ho) / np.maximum(np.abs(Ho), 1e-9 / parity.D_RTOL))
        assert eD <= parity.D_RTOL and eH <= parity.D_RTOL, (r, eD, eH)
        assert np.array_equal(stats[:, r].astype(np.float64), So), r
    _say(f"two slot rounds: {over} of {len(sample)} sampled blocks claim more than 112 bins")
    assert over >= len(sample) // 2


def test_strided_input():
    """A non-contiguous view (every other head of a larger tensor)."""
    import torch
    rng = np.random.default_rng(8)
    full = rng.standard_normal((1, 8, 64, 128)).astype(np.float16)
    dev = torch.from_numpy(full).cuda()[:, ::2]
    host = full[:, ::2]
    kw = dict(tokens_per_block=32, dims_per_block=128, s=16, search="grids", B=2.0,
              mode="bisect")
    _say(f"strided {kw}")
    g = parity.run_gpu([host], tensors_dev=[dev], **kw)
    o = parity.run_oracle([np.ascontiguousarray(host)], **kw)
    parity.full_compare(g, o, "grids", 0, 2.0)


def test_nonfinite_and_infeasible_are_reported():
    import torch
    from kv_cache_rate_amd import kvq
    rng = np.random.default_rng(9)
    x = rng.standard_normal((1, 2, 32, 128)).astype(np.float16)
    x[0, 1, 5, 7] = np.nan
    dev = [torch.from_numpy(x).cuda()]
    plan = kvq.kvq_plan_blocks(dev, 32, 128, 16)
    buf = kvq.allocate(plan)
    _say("nonfinite")
    with pytest.raises(kvq.KvqError) as e:
        kvq.admit(plan, dev, buf, 2.0)
    assert e.value.status == kvq.KVQ_ENONFINITE
    x[0, 1, 5, 7] = 1.0
    dev = [torch.from_numpy(x).cuda()]
    _say("infeasible")
    with pytest.raises(kvq.KvqError) as e:
        kvq.admit(plan, dev, buf, 0.0)  # no allocation has zero entropy here
    assert e.value.status == kvq.KVQ_EINFEASIBLE


def test_deterministic_repeat():
    """Two runs on the same inputs give bitwise equal outputs."""
    w = W.DECODE_ADMIT_FP16
    x = W.generate(w, which=1)
    kw = _kw(w, mode="bisect")
    _say("repeat")
    a = parity.run_gpu(x, **kw)
    b = parity.run_gpu(x, **kw)
    for k in ("D", "H", "stats", "codebook", "m", "off", "codes", "xhat"):
        assert np.array_equal(a[k], b[k]), k
    assert a["lam"] == b["lam"]


# ------------------------------------------------ weighted distortion ---

@pytest.mark.parametrize("name", ["tiny_k_fp32", "prefill_kv_fp16"])
def test_weighted_distortion(name):
    """Per-(tensor, head) log-normal distortion weights (a stand-in for
    attention sensitivity from a calibration batch) through
    kvq_solve_lambda_weighted; the bisection, choices and codes must match
    the oracle's weighted solve, and the weights must move the allocation."""
    from oracle import ecasq
    w = W.BY_NAME[name]
    B = 1.0 if name == "tiny_k_fp32" else 1.5  # budgets that bind (lambda > 0)
    x = W.generate(w)
    wt = W.sensitivity_weights(w)
    kw = _kw(w, B=B)
    g = parity.run_gpu(x, **kw, weights=wt)
    o = parity.run_oracle(x, **kw, weights=wt)
    rep = parity.full_compare(g, o, "grids", w.seed, B, "bisect", weights=wt)
    _say(f"{name} weighted report {rep}")
    assert o["lam"] > 0.0
    plain = ecasq.choose(o["D"], o["H"], float(o["n"]), o["lam"])
    assert np.any(plain != o["choice"])


# --------------------------------------------------- greedy post-pass ---

@pytest.mark.parametrize("name,B,iters", [("tiny_k_fp32", 1.0, 40), ("tiny_k_fp32", 1.2, 6),
                                          ("prefill_kv_fp16", 1.5, 10), ("decode_admit_fp16", 2.0, 40)])
def test_greedy_fill(name, B, iters):
    """KVQ_BISECT_GREEDY: bisection, then the remaining budget spent on the
    upgrades with the best distortion reduction per added bit.  Choices,
    codebooks, offsets and codes must equal the oracle's greedy (its slack
    is exact rational arithmetic, the GPU's fixed point at 2^-rate_shift
    bits; no decision here lies within that of a boundary)."""
    w = W.BY_NAME[name]
    x = W.generate(w)
    kw = _kw(w, B=B, mode="bisect_greedy", iters=iters)
    g = parity.run_gpu(x, **kw)
    o = parity.run_oracle(x, **kw)
    _say(f"{name} B={B} iters={iters}: lambda {g['lam']!r} swaps {len(o['swaps'])} "
         f"rate {g['rate_per_entry']:.6f} (bisection {o['rate_bits_bisect'] / (o['n'] * o['R']):.6f})")
    assert g["lam"] == o["lam"]
    assert np.array_equal(g["choice"].astype(np.int64), o["choice"])
    assert g["rate_per_entry"] == pytest.approx(o["rate_per_entry"], rel=1e-12)
    assert g["rate_per_entry"] <= B + 1e-12
    assert np.array_equal(g["off"], o["offsets"])
    agree = np.ones(o["R"], dtype=bool)
    assert parity.compare_codes(g, o, agree, w.seed) <= o["near"]


def _monotone_tables(R, seed, C=29):
    """Seeded score tables [R][C]: in every block H rises and D falls with
    the candidate index, D convex in H (distinct random steps, so no two
    objectives tie)."""
    rng = np.random.default_rng(seed)
    steps_h = rng.uniform(0.001, 0.05, size=(R, C - 1)) * rng.uniform(0.05, 1.0, size=(R, 1))
    H = np.concatenate([rng.uniform(0.2, 0.5, (R, 1)), steps_h], axis=1).cumsum(axis=1)
    slopes = np.sort(rng.uniform(0.5, 5.0, size=(R, C - 1)), axis=1)[:, ::-1]
    D = 100.0 - np.concatenate([np.zeros((R, 1)), (slopes * steps_h).cumsum(axis=1)], axis=1)
    return D, H


@pytest.mark.parametrize("R,iters,lo,hi", [(16, 40, 1, 128), (8, 4, 129, 256), (16, 4, 257, 512),
                                           (32, 4, 513, 1024), (40, 4, 1025, 16384)])
def test_greedy_fill_pool_sizes(R, iters, lo, hi):
    """The greedy post-pass on score tables given directly to
    kvq_solve_lambda, sized so that the upgrades fitting the slack left by
    the bisection (its pool) fall in each of the apply kernel's ranges: the
    register pool scanning 2, 4, 8 or 16 slots per lane, and the in-memory
    pool above 1024 entries.  Multiplier, choices and rate equal the
    oracle's bisection and greedy fill (page "Joint Tucker-rank and
    residual-bit KV allocator", Implementation notes)."""
    import torch
    from kv_cache_rate_amd import kvq
    D, H = _monotone_tables(R, seed=R)
    d = 4096.0
    B = float(np.mean(H[:, 14]))
    lam_o, ch_o, rate_o, Btot, _ = ecasq.solve_bisect(D, H, d, B, iters, None)
    rows = np.arange(R)
    rates = d * H
    slack = float(Btot) - float(rate_o)
    pool = int(((rates - rates[rows, ch_o][:, None] > 0) & (D[rows, ch_o][:, None] - D > 0) &
                (rates - rates[rows, ch_o][:, None] <= slack)).sum())
    assert lo <= pool <= hi, pool
    ch_g, rate_g, swaps = ecasq.greedy_fill(D, H, d, Btot, ch_o)
    # a plan of R fp16 head x 32 x 128 blocks (its data is never read here)
    x = torch.zeros((1, 1, 32 * R, 128), dtype=torch.float16, device="cuda")
    plan = kvq.kvq_plan_blocks([x], 32, 128, 16, kvq.KVQ_GRIDS, 0)
    assert plan.n_blocks == R and plan.n_cand == D.shape[1]
    buf = kvq.allocate(plan, dequant=False)
    buf["workspace"].zero_()  # no eval ran: its status word must start clear
    buf["D"].copy_(torch.from_numpy(np.ascontiguousarray(D.T)))
    buf["H"].copy_(torch.from_numpy(np.ascontiguousarray(H.T)))
    st = np.repeat(np.linspace(-1.0, 1.0, plan.n_stats, dtype=np.float32)[:, None], R, axis=1)
    buf["stats"].copy_(torch.from_numpy(st))
    lam, rate = kvq.kvq_solve_lambda(plan, buf["D"], buf["H"], buf["stats"], B, kvq.KVQ_BISECT_GREEDY, iters,
                                     1e-3, 0.0, buf["choice"], buf["codebook"], buf["m"], buf["off"],
                                     buf["workspace"])
    torch.cuda.synchronize()
    _say(f"greedy pool {pool} (R={R}, iters={iters}): swaps {len(swaps)} lambda {lam!r}")
    assert lam == lam_o
    assert np.array_equal(buf["choice"].cpu().numpy().astype(np.int64), ch_g)
    assert rate == pytest.approx(rate_g / (d * R), rel=1e-12)
    assert rate <= B + 1e-12
