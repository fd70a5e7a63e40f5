"""Block partition of KV tensors (oracle; test infrastructure only).

Page "Rate-adaptive KV-cache quantizer", Implementation notes: the cache is
cut into blocks of one attention head by 32 tokens, or one head by one
feature group.  The page does not fix the order of blocks or of entries
inside a block; the reading used here (and by the library) is:

* blocks are numbered tensor-major (K before V), then outer index (layer or
  sequence), head, token chunk, feature group, all row-major;
* inside a block the entries are row-major, token first then feature.

This order fixes the Philox counters and the packed-code offsets.
"""

import numpy as np


def partition(tensors, tokens_per_block, dims_per_block):
    """Return the blocks of ``tensors`` as a float64 array ``[R, n]``.

    ``tensors`` is a list of arrays shaped ``[outer, heads, tokens, dim]``
    (fp16, fp32 or fp64).  ``n = tokens_per_block * dims_per_block``.
    Negative zero is mapped to +0 (the sign of a zero carries no value and
    would otherwise split equal codepoints); a non-finite entry raises
    ``ValueError`` because neither the interpolation probabilities nor the
    distortion are defined for it.
    """
    out = []
    for t in tensors:
        t = np.asarray(t)
        if t.ndim != 4:
            raise ValueError("tensor must be [outer, heads, tokens, dim]")
        o, h, tok, dim = t.shape
        if tok % tokens_per_block or dim % dims_per_block:
            raise ValueError("tensor shape is not a multiple of the block shape")
        x = t.astype(np.float64)
        x = x.reshape(o, h, tok // tokens_per_block, tokens_per_block,
                      dim // dims_per_block, dims_per_block)
        x = x.transpose(0, 1, 2, 4, 3, 5)
        out.append(x.reshape(-1, tokens_per_block * dims_per_block))
    blocks = np.concatenate(out, axis=0) if out else np.zeros((0, tokens_per_block * dims_per_block))
    if not np.all(np.isfinite(blocks)):
        raise ValueError("non-finite entry in KV input")
    blocks = blocks + 0.0  # -0.0 + 0.0 == +0.0 under round-to-nearest
    return blocks


def block_of(tensors, tokens_per_block, dims_per_block, r):
    """Return block ``r`` alone (same order and canonicalisation as
    :func:`partition`) without materialising the others."""
    for t in tensors:
        o, h, tok, dim = t.shape
        nb = o * h * (tok // tokens_per_block) * (dim // dims_per_block)
        if r < nb:
            ng = dim // dims_per_block
            nc = tok // tokens_per_block
            g = r % ng
            c = (r // ng) % nc
            hh = (r // (ng * nc)) % h
            oo = r // (ng * nc * h)
            x = np.asarray(t[oo, hh, c * tokens_per_block:(c + 1) * tokens_per_block,
                             g * dims_per_block:(g + 1) * dims_per_block]).astype(np.float64)
            x = x.reshape(-1)
            if not np.all(np.isfinite(x)):
                raise ValueError("non-finite entry in KV input")
            return x + 0.0
        r -= nb
    raise IndexError("block index out of range")


def n_blocks(tensors, tokens_per_block, dims_per_block):
    return sum(t.shape[0] * t.shape[1] * (t.shape[2] // tokens_per_block)
               * (t.shape[3] // dims_per_block) for t in tensors)
