"""Throughput of KV-cache admission with blockwise ECASQ on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                    [--no-cpu-baseline]

A step is one pass of the whole hot path over the workload's synthetic K/V
tensors (already resident in HBM): kvq_plan_blocks, kvq_eval_candidates,
kvq_solve_lambda (bisection to the bits-per-entry budget), kvq_quantize_pack
and kvq_dequantize.  The default workload is the long-context admission
shape: 32 layers x 8 KV heads x 32768 tokens x 128, fp16 K and V (4.3 GB),
head x 32-token blocks, s = 16, B = 2.0 bits per entry.

Prints ONE JSON line: the metric is KV GB/s quantized (input K/V bytes per
second of step time) with the roofline of the dominant kernel (algorithmic
bytes per launch over its HIP-event-timed duration against 8 TB/s) and the
CPU oracle timed on a bounded sample of the same workload.
"""

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


# Source files each timed call's kernels are built from (the recorded HBM
# traffic of a kernel is used only while these files are unchanged).
KERNEL_SOURCES = {
    "eval": ("kvq_eval16.hip", "kvq_internal.h", "kvq_grid_choice.h", "kvq_quant_block.h"),
    "solve": ("kvq_solve.hip", "kvq_internal.h", "kvq_grid_choice.h"),
    "quantize_pack": ("kvq_quant.hip", "kvq_internal.h", "kvq_quant_block.h"),
    "dequantize": ("kvq_quant.hip", "kvq_internal.h", "kvq_quant_block.h"),
}


def kernel_sources_sha(files=None):
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "kv_cache_rate_amd", "csrc")
    for f in sorted(files or os.listdir(csrc)):
        h.update(open(os.path.join(csrc, f), "rb").read())
    return h.hexdigest()[:16]


def algorithmic_bytes(plan, words_total, in_bytes_per_entry):
    """Bytes each call must move at minimum (inputs read once, outputs
    written once).  The score table is counted at 4 bytes per D and per H
    entry (8 bytes per candidate and block), the size the method needs; the
    library stores them in fp64 for exact agreement with the oracle, and
    that choice's extra bytes are reported separately
    (:func:`table_fp64_excess_bytes`), never as algorithmic traffic."""
    R, n = plan.n_blocks, plan.n_entries
    table = 8 * R * plan.n_cand
    meta = plan.codebook_bytes + plan.m_bytes + plan.offsets_bytes
    return {
        "eval": n * in_bytes_per_entry + table + plan.stats_bytes,
        "solve": table + plan.stats_bytes + meta + plan.choice_bytes,
        "quantize_pack": n * in_bytes_per_entry + meta + 4 * words_total,
        "dequantize": 4 * words_total + meta + 4 * n,
    }


def table_fp64_excess_bytes(plan):
    """Bytes the fp64 D and H tables write beyond 4-byte entries."""
    return plan.D_bytes + plan.H_bytes - 8 * plan.n_blocks * plan.n_cand


def load_profile(kernel, sha):
    """The rocprofv3 record of a kernel in profiles/traffic.json (HBM bytes
    and VALU instructions per launch), or None once the kernel's sources no
    longer hash to the recorded value."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    try:
        rec = json.load(open(path))
    except Exception:
        return None
    k = rec.get(kernel)
    if not k or k.get("source_sha") != sha:
        return None
    return k


# VALU issue peak: 256 CUs x 4 SIMDs, one wave64 VALU instruction per SIMD
# every 4 cycles (16 lanes per cycle), at 2.4 GHz; some pairs of simple
# instructions issue together in one quad-cycle (counted by the profile)
VALU_SIMDS = 256 * 4
VALU_CLOCK_HZ = 2.4e9
VALU_PEAK_WAVE_INSTR_PER_S = VALU_SIMDS * VALU_CLOCK_HZ / 4


def copy_bandwidth(torch, nbytes=1 << 30, reps=5):
    """Device-to-device copy rate on this GPU (read + write bytes per second),
    the practical ceiling the HBM-bound kernels are compared with."""
    src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    times = []
    for _ in range(reps):
        ev[0].record()
        dst.copy_(src)
        ev[1].record()
        torch.cuda.synchronize()
        times.append(ev[0].elapsed_time(ev[1]))
    del src, dst
    return 2.0 * nbytes / (float(np.median(times)) * 1e-3) / 1e9


def decode_latency(torch, kvq, W, steps=1000, warmup=20):
    """Small-launch regime: 512 blocks of one decode step (batch 64 x 8 KV
    heads x 32 new tokens x 128, fp16 Student-t).  The previous batch is
    admitted by bisection to give lambda_prev; each measured step admits the
    next batch with one projected subgradient step from the running lambda.
    Per-call times are HIP events; the step time is wall clock around
    eval -> solve (synchronising) -> quantize_pack -> synchronize.  The same
    steps are then timed through kvq_admit (one call, one wait per step),
    from the same starting multiplier."""
    w = W.DECODE_ADMIT_FP16
    prev = [torch.from_numpy(h).cuda() for h in W.generate(w, which=0)]
    cur = [torch.from_numpy(h).cuda() for h in W.generate(w, which=1)]
    plan = kvq.kvq_plan_blocks(cur, w.tokens_per_block, w.dims_per_block, w.s)
    buf = kvq.allocate(plan)
    st = torch.cuda.current_stream()
    lam, _ = kvq.admit(plan, prev, buf, w.B, kvq.KVQ_BISECT, w.iters, w.eta, 0.0,
                       w.extra["prev_seed"], st)
    lam0 = lam
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
    step_us, per = [], {"eval": [], "solve": [], "quantize_pack": []}
    for i in range(warmup + steps):
        t0 = time.perf_counter()
        ev[0].record(st)
        kvq.kvq_eval_candidates(plan, cur, buf["D"], buf["H"], buf["stats"], buf["workspace"], st)
        ev[1].record(st)
        lam, rate = kvq.kvq_solve_lambda(plan, buf["D"], buf["H"], buf["stats"], w.B, kvq.KVQ_SUBGRAD,
                                         w.iters, w.eta, lam, buf["choice"], buf["codebook"],
                                         buf["m"], buf["off"], buf["workspace"], st)
        ev[2].record(st)
        kvq.kvq_quantize_pack(plan, cur, buf["codebook"], buf["m"], buf["off"], w.seed,
                              buf["codes"], stream=st)
        ev[3].record(st)
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        if i >= warmup:
            step_us.append((t1 - t0) * 1e6)
            for j, k in enumerate(per):
                per[k].append(ev[j].elapsed_time(ev[j + 1]) * 1e3)
    # the same steps through kvq_admit: one C call and one wait per step
    lam_f = lam0
    fused_us = []
    for i in range(warmup + steps):
        t0 = time.perf_counter()
        lam_f, _ = kvq.kvq_admit(plan, cur, buf, w.B, kvq.KVQ_SUBGRAD, w.iters, w.eta, lam_f, w.seed, st)
        t1 = time.perf_counter()
        if i >= warmup:
            fused_us.append((t1 - t0) * 1e6)
    # and through a prepared kvq_admit (arguments marshalled once, as a
    # decode loop over fixed buffers would call it)
    admit = kvq.prepare_admit(plan, cur, buf, w.B, kvq.KVQ_SUBGRAD, w.iters, w.eta, w.seed, st)
    lam_p = lam0
    prep_us = []
    for i in range(warmup + steps):
        t0 = time.perf_counter()
        lam_p, _ = admit(lam_p)
        t1 = time.perf_counter()
        if i >= warmup:
            prep_us.append((t1 - t0) * 1e6)
    q = lambda v: {"p50": float(np.percentile(v, 50)), "p90": float(np.percentile(v, 90))}
    return {"workload": w.name, "steps": steps, "step_us": q(step_us),
            "calls_us": {k: q(v) for k, v in per.items()}, "lambda_final": lam,
            "kvq_admit_step_us": q(fused_us), "kvq_admit_lambda_final": lam_f,
            "kvq_admit_prepared_step_us": q(prep_us), "kvq_admit_prepared_lambda_final": lam_p}


def extensions(torch, kvq, W, w, plan, dev, buf, stream):
    """The rows beyond the admission step, measured on the same cache after
    the timed steps (not part of `value`): entropy-coded size and coding
    times, fused decode attention vs torch's fp16 attention on the
    uncompressed cache, and a decode stream's multiplier trace."""
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]

    def timed(fn, reps=20):
        fn()
        torch.cuda.synchronize()
        ts = []
        for _ in range(reps):
            ev[0].record(stream)
            fn()
            ev[1].record(stream)
            torch.cuda.synchronize()
            ts.append(ev[0].elapsed_time(ev[1]))
        return float(np.median(ts))

    out = {}
    # entropy coding of the symbol stream (rANS, per-block models)
    ab = kvq.allocate_ans(plan)
    total = [0]

    def enc():
        total[0] = kvq.kvq_ans_encode(plan, buf["codes"], buf["m"], buf["off"], ab["scratch"], ab["stream"],
                                      ab["block_off"], buf["workspace"], stream)
    t_enc = timed(enc)
    t_dec = timed(lambda: kvq.kvq_ans_decode(plan, ab["stream"], ab["block_off"], buf["codebook"], buf["m"],
                                             buf["xhat"], buf["workspace"], stream))
    out["entropy_coding"] = {"coded_bits_per_entry": 8.0 * total[0] / w.n_entries,
                             "fixed_width_bits_per_entry": 32.0 * float(buf["off"][-1].item()) / w.n_entries,
                             "encode_ms_incl_sync": t_enc, "decode_ms": t_dec}
    del ab
    # decode attention over the quantized cache, 4 query heads per KV head
    if plan.n_tensors == 2 and plan.tokens_per_block == 32 and plan.dims_per_block == 128:
        L, Hk, T, D = dev[0].shape
        Hq = 4 * Hk
        g = torch.Generator(device="cuda").manual_seed(5)
        q = torch.randn(L, Hq, D, device="cuda", dtype=torch.float32, generator=g)
        o = torch.empty_like(q)
        work = torch.empty(kvq.kvq_decode_attention_workspace(plan, Hq), dtype=torch.uint8, device="cuda")
        t_att = timed(lambda: kvq.kvq_decode_attention(plan, buf["codes"], buf["codebook"], buf["m"], buf["off"],
                                                       q, Hq, 1.0 / np.sqrt(D), o, work, stream))
        qh = q.to(dev[0].dtype).view(L, Hq, 1, D)
        t_sdpa = timed(lambda: torch.nn.functional.scaled_dot_product_attention(qh, dev[0], dev[1],
                                                                                enable_gqa=True))
        out["decode_attention"] = {"query_heads": Hq, "tokens": T, "layers": L, "fused_quantized_ms": t_att,
                                   "torch_sdpa_fp16_uncompressed_ms": t_sdpa,
                                   "codes_GB": 4.0 * float(buf["off"][-1].item()) / 1e9}
    # sensitivity-weighted distortion and the greedy fill against the plain
    # solve, on the same score table at a budget that binds (the step's own
    # budget leaves the multiplier at 0 here); last, since they rewrite the
    # step's choices
    if plan.search == kvq.KVQ_GRIDS:
        Bw = 1.5
        wd = torch.from_numpy(W.sensitivity_weights(w)).cuda()
        res = {}
        for name, weighted, mode in (("plain", False, kvq.KVQ_BISECT), ("weighted", True, kvq.KVQ_BISECT),
                                     ("plain_greedy_fill", False, kvq.KVQ_BISECT_GREEDY)):
            def solve():
                if weighted:
                    return kvq.kvq_solve_lambda_weighted(plan, buf["D"], buf["H"], wd, buf["stats"], Bw,
                                                         kvq.KVQ_BISECT, 40, 0.0, 0.0, buf["choice"],
                                                         buf["codebook"], buf["m"], buf["off"],
                                                         buf["workspace"], stream)
                return kvq.kvq_solve_lambda(plan, buf["D"], buf["H"], buf["stats"], Bw, mode, 40,
                                            0.0, 0.0, buf["choice"], buf["codebook"], buf["m"], buf["off"],
                                            buf["workspace"], stream)
            solve()
            ts = []
            for _ in range(5):
                torch.cuda.synchronize()
                t0 = time.perf_counter()
                lam, rate = solve()
                torch.cuda.synchronize()
                ts.append(1e3 * (time.perf_counter() - t0))
            res[name] = {"solve_ms_incl_sync": float(np.median(ts)), "lambda": lam, "rate_bits_per_entry": rate}
        out["binding_budget_solves"] = {"B_bits_per_entry": Bw,
                                        "weights": "log-normal(0, 0.5) per (tensor, layer, head)", **res}
    return out


def decode_stream(torch, kvq, W, steps=200, batches=16):
    """Decode stream: every step admits a fresh 512-block batch (Student-t
    decode workload, one batch per step from its own seed) with one
    subgradient step from the running multiplier; returns the multiplier
    and rate trace.  The first multiplier comes from bisection on batch 0."""
    w = W.DECODE_ADMIT_FP16
    data = []
    for b in range(batches):
        rng = np.random.default_rng(np.random.SeedSequence(3000 + b))
        (_, shp), = w.tensors
        data.append([torch.from_numpy(rng.standard_t(5.0, size=shp).astype(np.float16)).cuda()])
    plan = kvq.kvq_plan_blocks(data[0], w.tokens_per_block, w.dims_per_block, w.s)
    buf = kvq.allocate(plan)
    lam, _ = kvq.admit(plan, data[0], buf, w.B, kvq.KVQ_BISECT, w.iters, w.eta, 0.0, 0)
    lams, rates = [lam], []
    for t in range(steps):
        lam, rate = kvq.admit(plan, data[(t + 1) % batches], buf, w.B, kvq.KVQ_SUBGRAD, w.iters, w.eta, lam,
                              t + 1)
        lams.append(lam)
        rates.append(rate)
    return {"steps": steps, "eta": w.eta, "B": w.B, "lambda_first": lams[:6], "lambda_last": lams[-1],
            "rate_mean_last_100": float(np.mean(rates[-100:])),
            "rate_min_max_last_100": [float(np.min(rates[-100:])), float(np.max(rates[-100:]))]}


def exact_search(torch, kvq, W, reps=5):
    """Searches over a quantile alphabet on the feature-group tensor: the
    exact DP (12 quantiles with |Q| <= 8, 32 quantiles with |Q| <= 16) and
    the beam over ordered codepoints (widths 2 and 4 on the same two).
    Medians of eval (HIP events) and of the solve call (host clock: it
    synchronises), with the multiplier and modelled rate."""
    out = {}
    t = [torch.from_numpy(np.ascontiguousarray(a)).cuda() for a in W.generate(W.FEATURE_GROUP_EXACT_FP32)]
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    cases = [("exact_dp", W.FEATURE_GROUP_EXACT_FP32, 0), ("exact_dp", W.FEATURE_GROUP_EXACT_M32, 0),
             ("beam", W.FEATURE_GROUP_EXACT_FP32, 2), ("beam", W.FEATURE_GROUP_EXACT_M32, 4)]
    for search, w, width in cases:
        sm = kvq.KVQ_EXACT_DP if search == "exact_dp" else kvq.KVQ_BEAM
        plan = kvq.kvq_plan_blocks(t, w.tokens_per_block, w.dims_per_block, w.s, sm, w.alphabet_m, width)
        buf = kvq.allocate(plan)
        te, ts = [], []
        for _ in range(reps + 1):
            ev[0].record()
            kvq.kvq_eval_candidates(plan, t, buf["D"], buf["H"], buf["stats"], buf["workspace"])
            ev[1].record()
            torch.cuda.synchronize()
            te.append(ev[0].elapsed_time(ev[1]))
            t0 = time.perf_counter()
            lam, rate = kvq.kvq_solve_lambda(plan, buf["D"], buf["H"], buf["stats"], w.B, kvq.KVQ_BISECT,
                                             w.iters, w.eta, 0.0, buf["choice"], buf["codebook"], buf["m"],
                                             buf["off"], buf["workspace"])
            ts.append(1e3 * (time.perf_counter() - t0))
        key = f"{search}_m{w.alphabet_m}_s{w.s}" + (f"_w{width}" if width else "")
        out[key] = {"alphabet": w.alphabet_m, "max_levels": w.s, "beam_width": width or None,
                    "blocks": plan.n_blocks, "pairs_per_block": plan.n_cand,
                    "eval_ms": float(np.median(te[1:])), "solve_ms": float(np.median(ts[1:])),
                    "lambda": lam, "rate_bits_per_entry": rate}
        del buf
    return out


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def oracle_stages(w, b, procs):
    """The oracle, as it stands, on blocks ``b`` ([R, n] fp64) of workload
    ``w``, stage by stage: scoring (``procs`` worker processes), the
    multiplier, quantize + pack and decode (one core each).  Returns the
    per-stage wall times in seconds."""
    from oracle import codes as ocodes
    from oracle import ecasq, pipeline
    t = {}
    if w.search != "grids":
        t0 = time.perf_counter()
        out = pipeline.run(b, search=w.search, s=w.s, alphabet_m=w.alphabet_m, B=w.B, mode="bisect",
                           iters=w.iters, seed=w.seed, processes=procs)
        t["all_stages"] = time.perf_counter() - t0
        return t
    R, n = b.shape
    t0 = time.perf_counter()
    D, H, S, books = pipeline.eval_grids(b, w.s, procs)
    t1 = time.perf_counter()
    if w.mode == "bisect":
        lam, choice, rate, Btot, probes = ecasq.solve_bisect(D, H, float(n), w.B, w.iters)
    else:
        choice, rbar, lam = ecasq.subgrad_step(D, H, float(n), w.B, 0.5, w.eta)
    t2 = time.perf_counter()
    chosen = [books[r][choice[r]] for r in range(R)]
    cs = [ocodes.quantize_block(b[r], chosen[r], w.seed, r)[0] for r in range(R)]
    ocodes.pack(cs, [ocodes.code_width(Q.size) for Q in chosen])
    t3 = time.perf_counter()
    for r in range(R):
        ocodes.dequantize_block(cs[r], chosen[r])
    t4 = time.perf_counter()
    t.update(eval=t1 - t0, solve=t2 - t1, quantize_pack=t3 - t2, dequantize=t4 - t3)
    return t


def cpu_baseline(w, tensors, target_s=10.0):
    """The oracle, as it stands, on the first blocks of the workload: eval
    (all host cores), bisection, quantize+pack and decode (one core), with
    the time of each stage."""
    from oracle import blocks as oblocks
    from oracle import pipeline
    procs = pipeline.default_processes()
    per_tensor = tensors[0].shape[1] * (tensors[0].shape[2] // w.tokens_per_block) * \
        (tensors[0].shape[3] // w.dims_per_block)
    layer_blocks = per_tensor  # blocks of one outer index of tensor 0

    def sample(nb):
        sub = [tensors[0][:1]]
        b = oblocks.partition(sub, w.tokens_per_block, w.dims_per_block)
        return b[:nb]

    pilot_n = min(layer_blocks, 16 * procs)
    t_pilot = sum(oracle_stages(w, sample(pilot_n), procs).values())
    nb = int(min(layer_blocks, max(pilot_n, pilot_n * target_s / max(t_pilot, 1e-3))))
    b = sample(nb)
    stages = oracle_stages(w, b, procs)
    t = sum(stages.values())
    in_bytes = b.size * (2 if w.dtype == "f16" else 4)
    return {"value": in_bytes / t / 1e9, "unit": "GB/s", "cores": procs, "kind": "oracle",
            "sample": f"first {nb} blocks ({b.size} entries) of layer 0 of K: eval on {procs} "
                      f"processes, then bisection (B={w.B}), quantize+pack and decode on one core; "
                      f"{t:.2f} s wall",
            "stage_s": stages, "stage_cores": {"eval": procs, "solve": 1, "quantize_pack": 1, "dequantize": 1},
            "elements_per_s": b.size / t, "cpu_model": cpu_model(), "numpy": np.__version__}


def per_workload(torch, kvq, W, reps=20):
    """Every other configuration: eval + quantize_pack (HIP events, median of
    ``reps`` after 3 warm-up calls) as KV GB/s and elements/s, the solve,
    and the oracle on one core over a bounded sample of the same blocks."""
    from oracle import blocks as oblocks
    out = {}
    for w in (W.TINY_K_FP32, W.PREFILL_KV_FP16, W.DECODE_ADMIT_FP16, W.FEATURE_GROUP_EXACT_FP32):
        host = W.generate(w)
        dev = [torch.from_numpy(np.ascontiguousarray(h)).cuda() for h in host]
        search = {"grids": kvq.KVQ_GRIDS, "exact_dp": kvq.KVQ_EXACT_DP}[w.search]
        plan = kvq.kvq_plan_blocks(dev, w.tokens_per_block, w.dims_per_block, w.s, search,
                                   w.alphabet_m if search else 0)
        buf = kvq.allocate(plan)
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
        tq, ts = [], []
        mode = kvq.KVQ_BISECT if w.mode == "bisect" else kvq.KVQ_SUBGRAD
        lam0 = 0.0 if mode == kvq.KVQ_BISECT else 0.5
        for i in range(reps + 3):
            ev[0].record()
            kvq.kvq_eval_candidates(plan, dev, buf["D"], buf["H"], buf["stats"], buf["workspace"])
            ev[1].record()
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            kvq.kvq_solve_lambda(plan, buf["D"], buf["H"], buf["stats"], w.B, mode, w.iters, w.eta, lam0,
                                 buf["choice"], buf["codebook"], buf["m"], buf["off"], buf["workspace"])
            t1 = time.perf_counter()
            ev[1].record()
            kvq.kvq_quantize_pack(plan, dev, buf["codebook"], buf["m"], buf["off"], w.seed, buf["codes"])
            ev[2].record()
            torch.cuda.synchronize()
            if i >= 3:
                tq.append(ev[1].elapsed_time(ev[2]))
                ts.append(1e3 * (t1 - t0))
        # eval alone, timed separately (the solve's host wait sits between)
        te = []
        for i in range(reps + 3):
            ev[0].record()
            kvq.kvq_eval_candidates(plan, dev, buf["D"], buf["H"], buf["stats"], buf["workspace"])
            ev[1].record()
            torch.cuda.synchronize()
            if i >= 3:
                te.append(ev[0].elapsed_time(ev[1]))
        ms = float(np.median(te)) + float(np.median(tq))
        words = int(buf["off"][-1].item())
        alg = algorithmic_bytes(plan, words, 2 if w.dtype == "f16" else 4)
        b = oblocks.partition(host[:1], w.tokens_per_block, w.dims_per_block)
        nb = min(b.shape[0], 64 if w.search == "grids" else 16)
        stages = oracle_stages(w, b[:nb], 1)
        tc = sum(stages.values())
        out[w.name] = {"blocks": plan.n_blocks, "entries": plan.n_entries,
                       "eval_ms": float(np.median(te)), "quantize_pack_ms": float(np.median(tq)),
                       "solve_ms_incl_sync": float(np.median(ts)),
                       "kv_GBps": w.input_bytes / (ms * 1e-3) / 1e9,
                       "elements_per_s": plan.n_entries / (ms * 1e-3),
                       "frac_of_hbm": (alg["eval"] + alg["quantize_pack"]) / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                       "oracle_1core": {"blocks": nb, "stage_s": stages,
                                        "elements_per_s": nb * plan.d_block / tc,
                                        "kv_GBps": nb * plan.d_block * (2 if w.dtype == "f16" else 4) / tc / 1e9}}
        del buf, dev
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default="long_context_kv_fp16")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the copy-bandwidth and decode-latency measurements")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="BYTES",
                    help="only run a device-to-device copy of BYTES (reference for HBM "
                         "byte counters) and exit")
    ap.add_argument("--read-probe", type=int, default=0, metavar="BYTES",
                    help="only run a sum over BYTES of device memory (a read-only kernel of "
                         "known size, to cross-check the HBM read counter's scale) and exit")
    a = ap.parse_args()
    if a.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path; "
              "run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch
    from kv_cache_rate_amd import kvq
    from kv_cache_rate_amd import workloads as W

    if a.copy_probe:
        src = torch.ones(a.copy_probe // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes": src.numel() * 4, "copies": 3}), flush=True)
        return
    if a.read_probe:
        src = torch.ones(a.read_probe // 4, dtype=torch.float32, device="cuda")
        tot = 0.0
        for _ in range(3):
            tot += float(src.sum().item())
        print(json.dumps({"read_probe_bytes": src.numel() * 4, "sums": 3, "total": tot}), flush=True)
        return

    w = W.BY_NAME[a.workload]
    log(f"generating {w.name}: {w.n_entries} entries, {w.input_bytes / 1e9:.2f} GB")
    t0 = time.time()
    host = W.generate(w)
    log(f"generated in {time.time() - t0:.1f} s; copying to HBM")
    dev = [torch.from_numpy(h).cuda() for h in host]
    torch.cuda.synchronize()
    search = kvq.KVQ_GRIDS if w.search == "grids" else kvq.KVQ_EXACT_DP
    mode = kvq.KVQ_BISECT if w.mode == "bisect" else kvq.KVQ_SUBGRAD
    plan = kvq.kvq_plan_blocks(dev, w.tokens_per_block, w.dims_per_block, w.s, search,
                               w.alphabet_m if search else 0)
    buf = kvq.allocate(plan, dequant=True)
    stream = torch.cuda.current_stream()
    names = ["eval", "solve", "quantize_pack", "dequantize"]

    def step(events=None):
        p = kvq.kvq_plan_blocks(dev, w.tokens_per_block, w.dims_per_block, w.s, search,
                                w.alphabet_m if search else 0)
        if events is not None:
            events[0].record(stream)
        kvq.kvq_eval_candidates(p, dev, buf["D"], buf["H"], buf["stats"], buf["workspace"], stream)
        if events is not None:
            events[1].record(stream)
        lam, rate = kvq.kvq_solve_lambda(p, buf["D"], buf["H"], buf["stats"], w.B, mode, w.iters,
                                         w.eta, 0.0, buf["choice"], buf["codebook"], buf["m"],
                                         buf["off"], buf["workspace"], stream)
        if events is not None:
            events[2].record(stream)
        kvq.kvq_quantize_pack(p, dev, buf["codebook"], buf["m"], buf["off"], w.seed, buf["codes"],
                              stream=stream)
        if events is not None:
            events[3].record(stream)
        kvq.kvq_dequantize(p, buf["codes"], buf["codebook"], buf["m"], buf["off"], buf["xhat"], stream)
        if events is not None:
            events[4].record(stream)
        return lam, rate

    for i in range(a.warmup):
        lam, rate = step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(a.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(a.steps):
        lam, rate = step(evs[i])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / max(1, a.steps)
    # per-call times: median over the timed steps
    per = {k: float(np.median([evs[i][j].elapsed_time(evs[i][j + 1]) for i in range(a.steps)]))
           for j, k in enumerate(names)}
    words_total = int(buf["off"][-1].item())
    alg = algorithmic_bytes(plan, words_total, 2 if w.dtype == "f16" else 4)
    dom = max(per, key=per.get)
    achieved = alg[dom] / (per[dom] * 1e-3) / 1e9
    sha = kernel_sources_sha()
    prof = load_profile(dom, kernel_sources_sha(KERNEL_SOURCES[dom]))
    traffic = prof.get("bytes_per_launch") if prof else None
    value = w.input_bytes / (ms_per_step * 1e-3) / 1e9
    admit_ms = per["eval"] + per["quantize_pack"]
    extras = {}
    if not a.no_extras:
        log("measuring copy bandwidth and decode-step latency")
        extras["copy_GBps"] = copy_bandwidth(torch)
        extras["decode_admission_latency"] = decode_latency(torch, kvq, W)
        log("measuring entropy coding, decode attention and a decode stream")
        extras["extensions"] = extensions(torch, kvq, W, w, plan, dev, buf, stream)
        extras["extensions"]["decode_stream"] = decode_stream(torch, kvq, W)
        extras["extensions"]["exact_search"] = exact_search(torch, kvq, W)
        log("measuring the other workloads")
        extras["per_workload"] = per_workload(torch, kvq, W)
    rec = {
        "metric": "KV GB/s quantized (fp16 in) and % of HBM roofline at 32-token blocks",
        "value": value, "unit": "GB/s", "n_gpus": 1, "steps": a.steps, "warmup": a.warmup,
        "ms_per_step": ms_per_step, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f16" if w.dtype == "f16" else "f32",
        "data": "synthetic (seeded numpy; N(0,1) x per-layer U[0.5,4] scale, 1% +-10 sigma)",
        "config": {"workload": w.name, "tensors": [list(s) for _, s in w.tensors],
                   "block": f"head x {w.tokens_per_block} tokens x {w.dims_per_block}",
                   "s": w.s, "B_bits_per_entry": w.B, "lambda_search": f"{w.mode} {w.iters}",
                   "n_blocks": w.n_blocks, "entries": w.n_entries,
                   "step": "plan+eval+solve+quantize_pack+dequantize"},
        "roofline": {"bound": "hbm", "kernel": dom, "achieved": achieved, "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS, "traffic": traffic,
                     "algorithmic_bytes": alg[dom],
                     "table_fp64_excess_bytes": table_fp64_excess_bytes(plan) if dom in ("eval", "solve")
                     else 0},
        "kernels_ms": per,
        "valu_issue": None,
        "eval_plus_quantize": {"ms": admit_ms,
                               "kv_GBps": w.input_bytes / (admit_ms * 1e-3) / 1e9,
                               "elements_per_s": w.n_entries / (admit_ms * 1e-3),
                               "frac_of_hbm": (alg["eval"] + alg["quantize_pack"]) /
                                              (admit_ms * 1e-3) / 1e9 / HBM_PEAK_GBS},
        "lambda": lam, "rate_bits_per_entry": rate,
        "packed_bits_per_entry": 32.0 * words_total / w.n_entries,
        "source_sha": sha,
        "kernel_source_sha": {k: kernel_sources_sha(v) for k, v in KERNEL_SOURCES.items()},
    }
    if prof and prof.get("valu_wave_instructions_per_launch"):
        ins = prof["valu_wave_instructions_per_launch"]
        rate = ins / (per[dom] * 1e-3)
        # the dominant kernel's second roof: VALU issue (profiled instruction
        # count per launch over this run's kernel time)
        rec["valu_issue"] = {"kernel": dom, "wave_instructions_per_launch": ins,
                             "achieved_per_s": rate, "peak_per_s": VALU_PEAK_WAVE_INSTR_PER_S,
                             "frac": rate / VALU_PEAK_WAVE_INSTR_PER_S}
        dual = prof.get("valu_dual_issue_quads_per_launch")
        if dual is not None:
            # quad-cycles the SIMDs' VALUs are busy (a dual-issued pair takes
            # one) over this run's kernel time
            rec["valu_issue"]["dual_issue_quads_per_launch"] = dual
            rec["valu_issue"]["busy_frac"] = 4.0 * (ins - dual) / (
                VALU_SIMDS * VALU_CLOCK_HZ * per[dom] * 1e-3)
    if extras:
        rec["copy_GBps"] = extras["copy_GBps"]
        rec["eval_plus_quantize"]["frac_of_copy"] = (alg["eval"] + alg["quantize_pack"]) / \
            (admit_ms * 1e-3) / 1e9 / extras["copy_GBps"]
        rec["roofline"]["frac_of_copy"] = achieved / extras["copy_GBps"]
        rec["decode_admission_latency"] = extras["decode_admission_latency"]
        rec["extensions"] = extras["extensions"]
        rec["per_workload"] = extras["per_workload"]
    if not a.no_cpu_baseline:
        log("timing the CPU oracle on a bounded sample")
        rec["cpu_baseline"] = cpu_baseline(w, host)
    else:
        rec["cpu_baseline"] = None
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
