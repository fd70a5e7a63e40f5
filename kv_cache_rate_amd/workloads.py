"""Seeded synthetic KV workloads.

This module holds the workload descriptions (tensor shapes, dtype, block
shape, codebook limit, budget, multiplier mode, Philox seed) and the seeded
generators of their input tensors.  It contains none of the quantizer's
arithmetic: both the HIP library's callers and the CPU reference consume the
arrays it returns.

The page "Rate-adaptive KV-cache quantizer" evaluates on a 1-3B decoder over
WikiText / LongBench at 4K-16K contexts; neither the model nor the datasets
are available, so these synthetic tensors stand in for them, with the shapes
and distributions listed per workload (the D-Quant abstract notes that
rotated, normalised KV values are roughly normal, which motivates Gaussian
bulks with heavy-tailed or outlier-channel variants).

Every generator draws from ``numpy.random.default_rng`` seeded by a
``SeedSequence`` whose entropy is ``1000 + i`` for workload i; large tensors
are produced per (tensor, layer) chunk from spawned child sequences, so any
chunk can be regenerated alone.
"""

from dataclasses import dataclass, field
from concurrent.futures import ThreadPoolExecutor
import os

import numpy as np


@dataclass(frozen=True)
class Workload:
    name: str
    index: int                    # 1-based position in the workload list
    tensors: tuple                # ((name, (outer, heads, tokens, dim)), ...)
    dtype: str                    # "f16" | "f32"
    tokens_per_block: int
    dims_per_block: int
    s: int                        # codebook size limit |Q| <= s
    search: str                   # "grids" | "exact_dp"
    B: float                      # budget, bits per entry
    mode: str                     # "bisect" | "subgrad"
    iters: int = 40
    eta: float = 1e-3
    seed: int = 0                 # Philox seed of the measured batch
    alphabet_m: int = 12
    note: str = ""
    extra: dict = field(default_factory=dict)

    @property
    def n(self):
        return self.tokens_per_block * self.dims_per_block

    @property
    def np_dtype(self):
        return np.float16 if self.dtype == "f16" else np.float32

    @property
    def n_blocks(self):
        tot = 0
        for _, (o, h, t, d) in self.tensors:
            tot += o * h * (t // self.tokens_per_block) * (d // self.dims_per_block)
        return tot

    @property
    def n_entries(self):
        return self.n_blocks * self.n

    @property
    def input_bytes(self):
        return self.n_entries * (2 if self.dtype == "f16" else 4)


TINY_K_FP32 = Workload(
    name="tiny_k_fp32", index=1,
    tensors=(("K", (1, 8, 256, 128)),), dtype="f32",
    tokens_per_block=32, dims_per_block=128, s=8, search="grids",
    B=3.0, mode="bisect", seed=0,
    note="1 layer K only, N(0,1) x per-(head,channel) LogNormal(0,0.5) scale",
    extra={"test_budgets": (0.8, 1.0, 1.2)})

PREFILL_KV_FP16 = Workload(
    name="prefill_kv_fp16", index=2,
    tensors=(("K", (1, 32, 4096, 128)), ("V", (1, 32, 4096, 128))), dtype="f16",
    tokens_per_block=32, dims_per_block=128, s=16, search="grids",
    B=2.5, mode="bisect", seed=0,
    note="K N(0,1) with 4 outlier channels per head x20; V Laplace(0,1)")

DECODE_ADMIT_FP16 = Workload(
    name="decode_admit_fp16", index=3,
    tensors=(("K", (64, 8, 32, 128)),), dtype="f16",
    tokens_per_block=32, dims_per_block=128, s=16, search="grids",
    B=2.0, mode="subgrad", eta=1e-3, seed=1,
    note="64 sequences x 8 KV heads x 32 new tokens, Student-t(5); multiplier "
         "warm-started by bisection on a previous batch (Philox seed 0)",
    extra={"prev_seed": 0})

LONG_CONTEXT_KV_FP16 = Workload(
    name="long_context_kv_fp16", index=4,
    tensors=(("K", (32, 8, 32768, 128)), ("V", (32, 8, 32768, 128))), dtype="f16",
    tokens_per_block=32, dims_per_block=128, s=16, search="grids",
    B=2.0, mode="bisect", seed=0,
    note="32 layers x 8 KV heads x 32768 tokens x 128 (Llama-3-8B-like GQA); "
         "N(0,1) x per-layer U[0.5,4] scale, 1% entries replaced by +-10 sigma")

FEATURE_GROUP_EXACT_FP32 = Workload(
    name="feature_group_exact_fp32", index=5,
    tensors=(("X", (1, 8, 8192, 128)),), dtype="f32",
    tokens_per_block=256, dims_per_block=16, s=8, search="exact_dp",
    B=2.5, mode="bisect", seed=0, alphabet_m=12,
    note="Hadamard-rotated N(0, diag sigma^2), log10 sigma^2 ~ U[-2,2]; blocks "
         "head x 16-dim feature group x 256 tokens; exact search over a "
         "12-quantile alphabet")

WORKLOADS = (TINY_K_FP32, PREFILL_KV_FP16, DECODE_ADMIT_FP16,
             LONG_CONTEXT_KV_FP16, FEATURE_GROUP_EXACT_FP32)

# The feature-group workload (same tensor) with the exact search widened to
# a 32-quantile alphabet and codebooks of up to 16 points.
FEATURE_GROUP_EXACT_M32 = Workload(
    name="feature_group_exact_m32_fp32", index=5,
    tensors=(("X", (1, 8, 8192, 128)),), dtype="f32",
    tokens_per_block=256, dims_per_block=16, s=16, search="exact_dp",
    B=2.5, mode="bisect", seed=0, alphabet_m=32,
    note="feature-group tensor; exact search over a 32-quantile alphabet, |Q| <= 16")

BY_NAME = {w.name: w for w in WORKLOADS + (FEATURE_GROUP_EXACT_M32,)}


def _threads():
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _tiny_k(w):
    rng = np.random.default_rng(np.random.SeedSequence(1000 + w.index))
    (_, shp), = w.tensors
    o, h, t, d = shp
    scale = rng.lognormal(mean=0.0, sigma=0.5, size=(h, d))
    z = rng.standard_normal(size=shp)
    return [(z * scale[None, :, None, :]).astype(np.float32)]


def _prefill_kv(w):
    kseq, vseq = np.random.SeedSequence(1000 + w.index).spawn(2)
    (_, kshp), (_, vshp) = w.tensors
    rk = np.random.default_rng(kseq)
    o, h, t, d = kshp
    K = rk.standard_normal(size=kshp, dtype=np.float32)
    for hh in range(h):
        ch = rk.choice(d, size=4, replace=False)
        K[:, hh, :, ch] *= 20.0
    rv = np.random.default_rng(vseq)
    V = rv.laplace(loc=0.0, scale=1.0, size=vshp).astype(np.float32)
    return [K.astype(np.float16), V.astype(np.float16)]


def _decode_batch(w, which):
    seqs = np.random.SeedSequence(1000 + w.index).spawn(2)
    rng = np.random.default_rng(seqs[which])
    (_, shp), = w.tensors
    return [rng.standard_t(df=5, size=shp).astype(np.float16)]


def long_context_sigma(w):
    """Per-layer scale sigma_l ~ U[0.5, 4], shared by K and V."""
    seq = np.random.SeedSequence(1000 + w.index).spawn(1)[0]
    layers = LONG_CONTEXT_KV_FP16.tensors[0][1][0]
    return np.random.default_rng(seq).uniform(0.5, 4.0, size=layers)


def long_context_chunk(w, tensor, layer, out=None):
    """One [heads, tokens, dim] layer of K (tensor 0) or V (tensor 1)."""
    _, (L, h, t, d) = w.tensors[tensor]
    sigma = long_context_sigma(w)[layer]
    root = np.random.SeedSequence(1000 + w.index)
    seq = np.random.SeedSequence(root.entropy, spawn_key=(1 + tensor, layer))
    rng = np.random.default_rng(seq)
    nel = h * t * d
    z = rng.standard_normal(nel, dtype=np.float32)
    u = rng.random(nel, dtype=np.float32)
    z *= np.float32(sigma)
    big = np.float32(10.0 * sigma)
    z[u < np.float32(0.005)] = big
    z[(u >= np.float32(0.005)) & (u < np.float32(0.01))] = -big
    res = z.astype(np.float16).reshape(h, t, d)
    if out is not None:
        out[...] = res
        return out
    return res


def _long_context(w, layers=None):
    _, (L, h, t, d) = w.tensors[0]
    layers = range(L) if layers is None else layers
    layers = list(layers)
    outs = [np.empty((len(layers), h, t, d), dtype=np.float16) for _ in w.tensors]

    def job(arg):
        ti, li = arg
        long_context_chunk(w, ti, layers[li], out=outs[ti][li])

    jobs = [(ti, li) for ti in range(len(w.tensors)) for li in range(len(layers))]
    with ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(job, jobs))
    return outs


def _feature_group(w):
    from scipy.linalg import hadamard
    rng = np.random.default_rng(np.random.SeedSequence(1000 + w.index))
    (_, shp), = w.tensors
    o, h, t, d = shp
    log_var = rng.uniform(-2.0, 2.0, size=(h, d))
    sigma = np.sqrt(10.0 ** log_var)
    z = rng.standard_normal(size=shp) * sigma[None, :, None, :]
    Hm = hadamard(d).astype(np.float64) / np.sqrt(d)
    x = z @ Hm.T
    return [x.astype(np.float32)]


def generate(w, which=1, layers=None):
    """Input tensors (numpy, host) of workload ``w``.

    ``which`` selects the batch for the decode workload (0 = previous batch
    that warms the multiplier, 1 = measured batch).  ``layers`` restricts the
    long-context workload to a subset of layers (each layer is generated from
    its own child stream, so a subset equals the same slices of the whole).
    """
    gen = {1: lambda: _tiny_k(w), 2: lambda: _prefill_kv(w),
           3: lambda: _decode_batch(w, which), 4: lambda: _long_context(w, layers),
           5: lambda: _feature_group(w)}
    return gen[w.index]()


def reduced(w, layers):
    """The long-context workload restricted to its first ``layers`` layers
    (same per-layer streams; used for parity runs the CPU reference can
    finish)."""
    ts = tuple((nm, (layers,) + shp[1:]) for nm, shp in w.tensors)
    return Workload(**{**w.__dict__, "tensors": ts, "name": w.name + f"_{layers}l"})


def sensitivity_weights(w, sigma=0.5):
    """Per-block distortion weights standing in for attention sensitivity
    measured on a calibration batch (no model or calibration data exists
    here): one log-normal(0, sigma) weight per (tensor, outer index, head),
    shared by that head's token chunks and feature groups, seeded from the
    workload.  Returned in block order (tensor, outer, head, chunk, group)
    as fp64."""
    rng = np.random.default_rng(np.random.SeedSequence(2000 + w.index))
    out = []
    for _, (o, h, t, d) in w.tensors:
        per_head = rng.lognormal(0.0, sigma, size=(o, h))
        reps = (t // w.tokens_per_block) * (d // w.dims_per_block)
        out.append(np.repeat(per_head.reshape(-1), reps))
    return np.concatenate(out).astype(np.float64)
