"""Stochastic interpolation, fixed-width packing and decode (oracle; test
infrastructure only).

Page "Rate-adaptive KV-cache quantizer", Key formulas (3): an entry x in
[q_i, q_{i+1}] becomes q_{i+1} with probability p = (x-q_i)/(q_{i+1}-q_i) and
q_i otherwise.  Implementation notes: the stored form is the codebook, the
symbol stream and the block lengths; decoding happens before attention.

Readings taken here:
* the draw for entry t of block r is the Philox uniform u of
  :mod:`oracle.philox`; the code is i+1 when u < p, else i; p is computed in
  fp64 from the fp32 codepoints.
* codes are stored at a fixed width w_r = ceil(log2 m_r) bits (0 for a
  one-level block) in a little-endian bit stream: code t of block r sits at
  stream bits [t w_r, t w_r + w_r), stream bit b being bit (b mod 32) of
  32-bit word off_r + b // 32; block r starts at word
  off_r = sum_{r' < r} ceil(d_{r'} w_{r'} / 32); unused tail bits are 0.
  The offsets array (R + 1 entries) carries the block lengths.
"""

import numpy as np

from .ecasq import interval_index
from .philox import block_uniforms

NEAR = 1e-6


def code_width(m):
    """Bits per code for an m-level codebook."""
    m = int(m)
    return 0 if m <= 1 else (m - 1).bit_length()


def _draws(x, Q, seed, r):
    """Interval index i, interpolation probability p (fp64, from the fp32
    codepoints) and Philox uniform u of every entry of block r."""
    x = np.asarray(x, dtype=np.float64)
    Q = np.asarray(Q, dtype=np.float64)
    i = interval_index(Q, x)
    p = (x - Q[i]) / (Q[i + 1] - Q[i])
    u = block_uniforms(seed, r, x.size)
    return i, p, u


def quantize_block(x, Q, seed, r):
    """Codes of one block.  Returns ``(codes uint32[n], near)`` where
    ``near`` counts draws with |u - p| < 1e-6 (where an fp32 computation of
    p may legitimately decide the other way)."""
    n = np.asarray(x).size
    if np.asarray(Q).size == 1:
        return np.zeros(n, dtype=np.uint32), 0
    i, p, u = _draws(x, Q, seed, r)
    codes = (i + (u < p)).astype(np.uint32)
    near = int(np.count_nonzero(np.abs(u - p) < NEAR))
    return codes, near


def near_mask(x, Q, seed, r):
    """Boolean mask of the entries whose draw is within 1e-6 of p (the
    entries :func:`quantize_block` counts as near)."""
    if np.asarray(Q).size == 1:
        return np.zeros(np.asarray(x).size, dtype=bool)
    _, p, u = _draws(x, Q, seed, r)
    return np.abs(u - p) < NEAR


def block_words(n, w):
    return (n * w + 31) // 32


def offsets(n, widths):
    """Word offsets (R + 1 entries) of blocks of length n with the given widths."""
    widths = np.asarray(widths, dtype=np.int64)
    sizes = (n * widths + 31) // 32
    off = np.zeros(widths.size + 1, dtype=np.uint64)
    off[1:] = np.cumsum(sizes).astype(np.uint64)
    return off


def pack_block(codes, w):
    """Pack one block's codes into ceil(n w / 32) words."""
    codes = np.asarray(codes, dtype=np.uint64)
    n = codes.size
    nw = block_words(n, w)
    words = np.zeros(nw, dtype=np.uint64)
    if w == 0:
        return words.astype(np.uint32)
    for k in range(w):
        bit = (codes >> np.uint64(k)) & np.uint64(1)
        pos = np.arange(n, dtype=np.int64) * w + k
        np.bitwise_or.at(words, pos >> 5, bit << (pos & 31).astype(np.uint64))
    return words.astype(np.uint32)


def unpack_block(words, n, w):
    """Inverse of :func:`pack_block`."""
    if w == 0:
        return np.zeros(n, dtype=np.uint32)
    words = np.asarray(words, dtype=np.uint64)
    codes = np.zeros(n, dtype=np.uint64)
    for k in range(w):
        pos = np.arange(n, dtype=np.int64) * w + k
        bit = (words[pos >> 5] >> (pos & 31).astype(np.uint64)) & np.uint64(1)
        codes |= bit << np.uint64(k)
    return codes.astype(np.uint32)


def pack(codes_per_block, widths):
    """Concatenate packed blocks.  Returns ``(words uint32, off uint64[R+1])``."""
    n = codes_per_block[0].size if len(codes_per_block) else 0
    off = offsets(n, widths)
    words = np.zeros(int(off[-1]), dtype=np.uint32)
    for r, (c, w) in enumerate(zip(codes_per_block, widths)):
        words[int(off[r]):int(off[r + 1])] = pack_block(c, int(w))
    return words, off


def dequantize_block(codes, Q):
    """Decoded entries Q[code] as fp32 (the stored codepoints)."""
    Q = np.asarray(Q, dtype=np.float64)
    return Q[np.asarray(codes, dtype=np.int64)].astype(np.float32)
