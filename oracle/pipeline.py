"""The whole admission pass for one configuration (oracle; test
infrastructure only).

Page "Rate-adaptive KV-cache quantizer", Implementation notes: at admission
each block builds its candidate alphabet, scores every candidate codebook by
D_r and H_r, the blocks choose argmin D_r + lambda d_r H_r under one global
lambda, and the chosen codebooks quantize the block by unbiased
interpolation; the codebook, symbol stream and block lengths are stored.
This module chains the steps of :mod:`ecasq`, :mod:`exact_dp` and
:mod:`codes` in that order and nothing else.
"""

import math
import os
from multiprocessing import get_context

import numpy as np

from . import codes as _codes
from . import ecasq, exact_dp


def _eval_grids_chunk(args):
    blocks, s = args
    C = ecasq.n_candidates(s)
    R = blocks.shape[0]
    n = blocks.shape[1]
    D = np.empty((R, C))
    H = np.empty((R, C))
    S = np.empty((R, len(ecasq.quantile_ranks(n, s))))
    books = []
    for r in range(R):
        D[r], H[r], S[r], cands = ecasq.eval_block(blocks[r], s)
        books.append(cands)
    return D, H, S, books


def _eval_exact_chunk(args):
    blocks, m_alpha, smax = args
    R, n = blocks.shape
    out = []
    for r in range(R):
        x = blocks[r]
        xs = np.sort(x)
        raw = xs[exact_dp.alphabet_ranks(n, m_alpha)]
        A = np.unique(raw)
        Dp, ML, MR = exact_dp.pair_stats(x, A)
        Dt, Ht, S_list = exact_dp.brute_force_tables(Dp, ML, MR, n, smax)
        out.append((raw, A, Dp, ML, MR, Dt, Ht, S_list))
    return out


def _eval_pairs_chunk(args):
    blocks, m_alpha = args
    R, n = blocks.shape
    out = []
    for r in range(R):
        x = blocks[r]
        raw = np.sort(x)[exact_dp.alphabet_ranks(n, m_alpha)]
        A = np.unique(raw)
        out.append((raw, A) + exact_dp.pair_stats(x, A))
    return out


# Exact search: brute force over the subsets while there are at most this
# many per block, the pair-state DP beyond (both give the same minimiser).
EXACT_BRUTE_MAX = 20000


def n_subsets(m, smax):
    """Endpoint-containing subsets of m points with 2..smax points."""
    if m <= 2:
        return 1
    return sum(math.comb(m - 2, k) for k in range(0, min(smax, m) - 1))


def _map(fn, chunks, processes):
    if processes and processes > 1 and len(chunks) > 1:
        with get_context("fork").Pool(processes) as pool:
            return pool.map(fn, chunks)
    return [fn(c) for c in chunks]


def _split(blocks, parts):
    parts = max(1, min(parts, blocks.shape[0]))
    return np.array_split(blocks, parts)


def eval_grids(blocks, s, processes=None):
    """D, H ([R, C]), order statistics and candidate codebooks of every block."""
    processes = processes or 1
    chunks = _split(blocks, processes * 4)
    res = _map(_eval_grids_chunk, [(c, s) for c in chunks], processes)
    D = np.concatenate([r[0] for r in res])
    H = np.concatenate([r[1] for r in res])
    S = np.concatenate([r[2] for r in res])
    books = [b for r in res for b in r[3]]
    return D, H, S, books


def eval_exact(blocks, m_alpha, smax, processes=None):
    """Alphabet, pair statistics and brute-force subset tables of every block."""
    processes = processes or 1
    chunks = _split(blocks, processes * 4)
    res = _map(_eval_exact_chunk, [(c, m_alpha, smax) for c in chunks], processes)
    return [b for r in res for b in r]


def eval_pairs(blocks, m_alpha, processes=None):
    """Alphabet and pair statistics of every block (no subset tables)."""
    processes = processes or 1
    chunks = _split(blocks, processes * 4)
    res = _map(_eval_pairs_chunk, [(c, m_alpha) for c in chunks], processes)
    return [b for r in res for b in r]


def run(blocks, *, search="grids", s=16, alphabet_m=12, B=2.0, mode="bisect",
        iters=40, lam_prev=0.0, eta=1e-3, seed=0, quantize=True, processes=None, weights=None,
        beam_width=None):
    """Admission of ``blocks`` ([R, n] fp64).  Returns a dict of every
    intermediate and final result (see the keys below).  ``weights`` ([R])
    weights each block's distortion in the dual choice (grid search only).
    ``search``: "grids", "exact_dp" (brute force or the DP, same minimiser)
    or "beam" (beam search of ``beam_width`` over the same alphabet)."""
    if weights is not None and search != "grids":
        raise ValueError("distortion weights apply to the grid search")
    if search == "beam" and not (beam_width and beam_width >= 1):
        raise ValueError("the beam search needs beam_width >= 1")
    R, n = blocks.shape
    d = float(n)
    out = {"n": n, "R": R}
    if search == "grids":
        D, H, stats, books = eval_grids(blocks, s, processes)
        out.update(D=D, H=H, stats=stats, books=books)
        Dt, Ht = D, H
    elif search == "beam" or (search == "exact_dp" and n_subsets(alphabet_m, s) > EXACT_BRUTE_MAX):
        ev = eval_pairs(blocks, alphabet_m, processes)
        out.update(alphabet_raw=np.stack([e[0] for e in ev]), alphabets=[e[1] for e in ev],
                   pairs=[(e[2], e[3], e[4]) for e in ev], route="dp" if search == "exact_dp" else "beam")
        Dt = Ht = None
    elif search == "exact_dp":
        ev = eval_exact(blocks, alphabet_m, s, processes)
        Cmax = max(len(e[7]) for e in ev)
        Dt = np.full((R, Cmax), np.inf)
        Ht = np.zeros((R, Cmax))
        for r, e in enumerate(ev):
            k = len(e[7])
            Dt[r, :k] = e[5]
            Ht[r, :k] = e[6]
        out.update(alphabet_raw=np.stack([e[0] for e in ev]),
                   pairs=[(e[2], e[3], e[4]) for e in ev],
                   alphabets=[e[1] for e in ev], subsets=[e[7] for e in ev],
                   D=Dt, H=Ht)
    else:
        raise ValueError(search)

    if out.get("route") in ("dp", "beam"):
        if mode != "bisect":
            raise ValueError("the DP and beam routes run the bisection")
        lam, subs, rate, Btot, probes = exact_dp.solve_bisect_dp(
            out["pairs"], n, B, s, iters, processes,
            beam_width if out["route"] == "beam" else None)
        out.update(lam=lam, subsets_chosen=subs, rate_bits=rate, B_total=Btot, probes=probes,
                   rate_per_entry=rate / (d * R))
    elif mode in ("bisect", "bisect_greedy"):
        lam, choice, rate, Btot, probes = ecasq.solve_bisect(Dt, Ht, d, B, iters, weights)
        out.update(lam=lam, choice=choice, rate_bits=rate, B_total=Btot, probes=probes,
                   rate_per_entry=rate / (d * R))
        if mode == "bisect_greedy":
            if search != "grids":
                raise ValueError("the greedy post-pass applies to the grid search")
            choice, rate, swaps = ecasq.greedy_fill(Dt, Ht, d, Btot, choice, weights)
            out.update(choice=choice, rate_bits=rate, rate_per_entry=rate / (d * R), swaps=swaps,
                       choice_bisect=out["choice"], rate_bits_bisect=out["rate_bits"])
    elif mode == "subgrad":
        choice, rbar, lam_next = ecasq.subgrad_step(Dt, Ht, d, B, lam_prev, eta, weights)
        out.update(lam=lam_next, lam_used=lam_prev, choice=choice, rate_per_entry=rbar,
                   rate_bits=rbar * d * R)
    else:
        raise ValueError(mode)

    # Chosen codebooks.
    book = np.zeros((R, s), dtype=np.float32)
    m = np.zeros(R, dtype=np.int64)
    chosen = []
    for r in range(R):
        if search == "grids":
            Q = books[r][choice[r]]
        elif out.get("route") in ("dp", "beam"):
            Q = out["alphabets"][r][list(out["subsets_chosen"][r])]
        else:
            A = out["alphabets"][r]
            Q = A[list(out["subsets"][r][choice[r]])]
        chosen.append(Q)
        m[r] = Q.size
        book[r, :Q.size] = Q.astype(np.float32)
    widths = np.array([_codes.code_width(k) for k in m], dtype=np.int64)
    out.update(codebook=book, m=m, width=widths, chosen=chosen,
               offsets=_codes.offsets(n, widths))
    if search in ("exact_dp", "beam"):
        masks = np.zeros(R, dtype=np.int64)
        for r in range(R):
            S = (out["subsets_chosen"][r] if out.get("route") in ("dp", "beam")
                 else out["subsets"][r][choice[r]])
            for idx in S:
                masks[r] |= 1 << idx
        out["mask"] = masks

    if quantize:
        all_codes = []
        near = 0
        for r in range(R):
            c, k = _codes.quantize_block(blocks[r], chosen[r], seed, r)
            all_codes.append(c)
            near += k
        words, off = _codes.pack(all_codes, widths)
        out.update(codes=all_codes, words=words, near=near)
        out["packed_bits_per_entry"] = 32.0 * words.size / (n * R)
    return out


def default_processes():
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1

