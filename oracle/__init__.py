"""Plain fp64 CPU oracle for blockwise entropy-constrained unbiased scalar
quantization (ECASQ) at KV-cache admission.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports, calls or
links anything in this package: only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with
the HIP library and imports nothing from ``kv_cache_rate_amd``.

Every function follows a passage of the page "Rate-adaptive KV-cache
quantizer" (synthcore idea 2502) and is written as the plain definition: each
element is visited directly, numpy's sort / searchsorted / bincount / argmin
serve as library steps, and there is no blocking, fusion or reordering beyond
what the definition states.  Where the page leaves a step open the reading
taken is stated in the function's docstring.

Modules
-------
blocks     block partition of [outer, heads, tokens, dim] tensors
ecasq      candidate codebooks, closed-form scoring, dual solve
exact_dp   quantile alphabet, pair statistics, brute force and pair-state DP
philox     Philox4x32-10 counter-based generator
codes      stochastic interpolation, fixed-width packing, decode
ans        rANS entropy coding of each block's symbol stream
attention  decode attention over the decoded cache
pipeline   the whole admission pass for one configuration

Parity status: every function is pinned by ``tests/test_oracle_*.py``
(closed forms, invariants, brute force, an independent Philox
implementation); none is "parity unpinned".
"""

from . import blocks, ecasq, exact_dp, philox, codes, ans, attention, pipeline  # noqa: F401
