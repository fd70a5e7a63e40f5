"""kv_cache_rate_amd — rate-adaptive KV-cache quantizer (blockwise ECASQ) on
AMD Instinct MI355X (gfx950).

The compute path is the C-ABI library ``libkvq.so`` (hand-written HIP
kernels); :mod:`kv_cache_rate_amd.kvq` is its thin ctypes binding, with the
same entry-point names, and uses PyTorch only for device memory and streams.
:mod:`kv_cache_rate_amd.workloads` holds the seeded synthetic inputs.

Importing the package does not load the library; the binding loads it on
first use and raises if it is missing (there is no CPU fallback).
"""

__all__ = ["kvq", "workloads"]
