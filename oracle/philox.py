"""Philox4x32-10 counter-based generator (oracle; test infrastructure only).

Definition: J. K. Salmon, M. A. Moraes, R. O. Dror, D. E. Shaw, "Parallel
random numbers: as easy as 1, 2, 3", SC'11.  A round maps the counter
(c0, c1, c2, c3) with key (k0, k1) to

    (hi(M1*c2) ^ c1 ^ k0,  lo(M1*c2),  hi(M0*c0) ^ c3 ^ k1,  lo(M0*c0))

with M0 = 0xD2511F53, M1 = 0xCD9E8D57; between rounds the key is bumped by
the Weyl constants (0x9E3779B9, 0xBB67AE85); ten rounds in all.

Stochastic-rounding reading (the pages name no generator; the draw for an
entry is indexed by (seed, block, entry)):
    key     = (seed mod 2**32, seed >> 32)
    counter = (t >> 2, r mod 2**32, r >> 32, 0)   for entry t of block r
    word    = output word t & 3
    u       = (word >> 8) * 2**-24               (24-bit uniform on [0, 1))
"""

import numpy as np

M0 = 0xD2511F53
M1 = 0xCD9E8D57
W0 = 0x9E3779B9
W1 = 0xBB67AE85
_MASK = np.uint64(0xFFFFFFFF)


def philox4x32_10(ctr, key):
    """Apply Philox4x32-10 to counters ``ctr`` ([N, 4] uint32) under
    ``key`` ([2] or [N, 2] uint32).  Returns [N, 4] uint32."""
    c = np.asarray(ctr, dtype=np.uint64).reshape(-1, 4).copy()
    k = np.asarray(key, dtype=np.uint64)
    k0 = np.broadcast_to(k[..., 0], (c.shape[0],)).copy()
    k1 = np.broadcast_to(k[..., 1], (c.shape[0],)).copy()
    m0 = np.uint64(M0)
    m1 = np.uint64(M1)
    for rnd in range(10):
        p0 = m0 * c[:, 0]          # < 2**64: exact in uint64
        p1 = m1 * c[:, 2]
        n0 = ((p1 >> np.uint64(32)) ^ c[:, 1] ^ k0) & _MASK
        n1 = p1 & _MASK
        n2 = ((p0 >> np.uint64(32)) ^ c[:, 3] ^ k1) & _MASK
        n3 = p0 & _MASK
        c = np.stack([n0, n1, n2, n3], axis=1)
        if rnd < 9:
            k0 = (k0 + np.uint64(W0)) & _MASK
            k1 = (k1 + np.uint64(W1)) & _MASK
    return c.astype(np.uint32)


def block_words(seed, r, n):
    """The n 32-bit draws of block ``r`` (entry t uses word t & 3 of counter
    (t >> 2, r_lo, r_hi, 0))."""
    seed = int(seed)
    r = int(r)
    groups = (n + 3) // 4
    ctr = np.zeros((groups, 4), dtype=np.uint64)
    ctr[:, 0] = np.arange(groups, dtype=np.uint64)
    ctr[:, 1] = r & 0xFFFFFFFF
    ctr[:, 2] = r >> 32
    key = np.array([seed & 0xFFFFFFFF, seed >> 32], dtype=np.uint64)
    return philox4x32_10(ctr, key).reshape(-1)[:n]


def block_uniforms(seed, r, n):
    """24-bit uniforms u_t = (word_t >> 8) * 2**-24 for block ``r``."""
    w = block_words(seed, r, n)
    return (w >> np.uint32(8)).astype(np.float64) * 2.0 ** -24
