"""Entropy coding of a block's symbol stream with interleaved rANS (oracle;
test infrastructure only).

Page "Rate-adaptive KV-cache quantizer", Implementation notes: the stored
form is the codebook, the symbol stream and the block lengths, with
arithmetic coding of the stream.  The budget on the page constrains the
modelled rate sum_r d_r H_r; coding the symbols with a model of their
frequencies turns that rate into stored bytes.  rANS (range asymmetric
numeral systems, J. Duda, "Asymmetric numeral systems", arXiv:0902.0271 and
arXiv:1311.2540) is the arithmetic-coding family member used here because
its state updates are exact integer arithmetic that parallel lanes can run
in lock step.

Readings taken here (the page names no coder, precision or layout):
* model: the block's own symbol counts.  With n entries, k = ceil(log2 n)
  and M = 2^k, the frequency of symbol j is its count c_j, except that the
  most frequent symbol (lowest index among equals) also receives M - n; the
  frequencies therefore sum to M and every present symbol has f_j >= 1.
  C_j = sum_{i<j} f_i.
* coder: 32-bit states x in [2^16, 2^32), 16-bit output words.  Encoding
  symbol s from state x: if x >= f_s 2^(32-k), emit the word x mod 2^16 and
  set x <- floor(x / 2^16); then x <- floor(x / f_s) 2^k + (x mod f_s) + C_s.
  Decoding: slot = x mod M, s is the symbol with C_s <= slot < C_s + f_s,
  x <- f_s floor(x / 2^k) + slot - C_s, and if x < 2^16 then
  x <- x 2^16 + (next word).
* interleaving: L = 8 states; state i codes entries t = i + 8 j (j = 0, 1,
  ...).  All states start at 2^16.  The encoder runs j from the last step
  down to 0; the decoder runs j upwards.  Words emitted at step j (one per
  state at most, in state order) form group j.
* block layout (little-endian 16-bit words): f_0 .. f_{m-1}; then the final
  states, state i as (x_i >> 16, x_i & 0xffff) for i = 0..7; then groups
  j = 0, 1, ... in order; then one zero word if needed so the block is a
  whole number of 32-bit words.  Block lengths (bytes) are stored as
  exclusive-scan offsets, as for the fixed-width stream.
"""

import numpy as np

LANES = 8
STATE_LOW = 1 << 16


def precision_bits(n):
    """k = ceil(log2 n): the model's frequencies sum to 2^k >= n."""
    n = int(n)
    return max(1, (n - 1).bit_length())


def frequencies(codes, m):
    """Model of a block: integer frequencies f (sum 2^k) and k."""
    codes = np.asarray(codes, dtype=np.int64)
    n = codes.size
    k = precision_bits(n)
    f = np.bincount(codes, minlength=m).astype(np.int64)[:m]
    if n:
        f[int(np.argmax(f))] += (1 << k) - n  # argmax: lowest index among equals
    return f, k


def encode_block(codes, m):
    """Encoded bytes (uint8 array, length a multiple of 4) of one block's
    codes (values in [0, m))."""
    codes = [int(c) for c in np.asarray(codes).tolist()]
    n = len(codes)
    f, k = frequencies(codes, m)
    C = np.concatenate([[0], np.cumsum(f)[:-1]]).astype(np.int64)
    x = [STATE_LOW] * LANES
    steps = (n + LANES - 1) // LANES
    groups = [None] * steps
    for j in range(steps - 1, -1, -1):
        words = []
        for i in range(LANES):
            t = i + LANES * j
            if t >= n:
                continue
            s = codes[t]
            fs, cs = int(f[s]), int(C[s])
            if x[i] >= fs << (32 - k):
                words.append(x[i] & 0xFFFF)
                x[i] >>= 16
            x[i] = ((x[i] // fs) << k) + (x[i] % fs) + cs
        groups[j] = words
    out = [int(v) for v in f]
    for i in range(LANES):
        out += [x[i] >> 16, x[i] & 0xFFFF]
    for j in range(steps):
        out += groups[j]
    if len(out) % 2:
        out.append(0)
    return np.asarray(out, dtype="<u2").view(np.uint8)


def decode_block(data, m, n):
    """Codes (int64[n]) of one encoded block; also checks that every state
    returns to its start."""
    w = np.asarray(data, dtype=np.uint8).view("<u2").astype(np.int64).tolist()
    f = w[:m]
    k = precision_bits(n)
    M = 1 << k
    C = [0] * m
    for j in range(1, m):
        C[j] = C[j - 1] + f[j - 1]
    if sum(f) != M:
        raise ValueError("frequency table does not sum to 2^k")
    pos = m
    x = []
    for i in range(LANES):
        x.append((w[pos] << 16) | w[pos + 1])
        pos += 2
    out = np.zeros(n, dtype=np.int64)
    steps = (n + LANES - 1) // LANES
    for j in range(steps):
        for i in range(LANES):
            t = i + LANES * j
            if t >= n:
                continue
            slot = x[i] & (M - 1)
            s = 0
            while not (C[s] <= slot < C[s] + f[s]):
                s += 1
            out[t] = s
            x[i] = f[s] * (x[i] >> k) + slot - C[s]
            if x[i] < STATE_LOW:
                x[i] = (x[i] << 16) | w[pos]
                pos += 1
    if any(v != STATE_LOW for v in x):
        raise ValueError("rANS states did not return to their start")
    return out


def model_bits(codes, m):
    """sum_t log2(M / f_{s_t}): the ideal code length of the block's symbols
    under its model (bits)."""
    f, k = frequencies(codes, m)
    codes = np.asarray(codes, dtype=np.int64)
    return float(np.sum(k - np.log2(f[codes].astype(np.float64))))
