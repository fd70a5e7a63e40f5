"""Decode attention over the quantized cache (oracle; test infrastructure
only).

Page "Rate-adaptive KV-cache quantizer", Implementation notes: the cache is
decoded before attention.  For one new query per query head the attention
output is the plain definition
    o = sum_t softmax_t(scale * q . k_t) v_t
over every cached token t, with k_t and v_t the decoded codepoints of the
quantized K and V (Key formulas (3): each stored entry is one codepoint of
its block).  Grouped query heads: query head g reads KV head g // G with
G = query heads / KV heads.  Everything is fp64.
"""

import numpy as np


def decode_attention(K, V, q, scale):
    """``K``, ``V``: decoded caches [outer, kv_heads, T, D]; ``q``:
    [outer, q_heads, D].  Returns o [outer, q_heads, D] (fp64)."""
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    q = np.asarray(q, dtype=np.float64)
    O, Hk, T, D = K.shape
    Hq = q.shape[1]
    G = Hq // Hk
    out = np.zeros((O, Hq, D))
    for o in range(O):
        for g in range(Hq):
            h = g // G
            s = scale * (K[o, h] @ q[o, g])
            p = np.exp(s - s.max())
            out[o, g] = (p @ V[o, h]) / p.sum()
    return out
