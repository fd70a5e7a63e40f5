"""Helpers for the GPU parity tests: run the HIP library through its C ABI
on seeded inputs, run the oracle on the same host arrays, and compare.

Bars (written out here and in the tests):
* D and H: within 1e-4 relative of the oracle (plus an absolute floor of
  1e-9 of the block's largest distortion, for candidates whose distortion is
  0 up to round-off); the maximum relative error is reported.
* order statistics, codepoints, levels, offsets: bit-exact.
* chosen codebook: identical by value, except documented ties where the
  oracle's objectives of the two choices differ by < 1e-5 relative.
* lambda: identical (both sides replay the same bisection); rate <= budget.
* packed codes: bit-exact, except draws with |u - p| < 1e-6 (counted).
* decoded entries: exactly the stored codepoints.
"""

import numpy as np

from oracle import blocks as oblocks
from oracle import codes as ocodes
from oracle import exact_dp
from oracle import pipeline

D_RTOL = 1e-4
TIE_RTOL = 1e-5


def to_cuda(arrays):
    import torch
    return [torch.from_numpy(np.ascontiguousarray(a)).cuda() for a in arrays]


def run_gpu(tensors, *, tokens_per_block, dims_per_block, s, search, alphabet_m=12, B, mode,
            iters=40, eta=1e-3, lam=0.0, seed=0, dequant=True, tensors_dev=None, weights=None,
            beam_width=0):
    """Run plan -> eval -> solve -> quantize -> dequantize through the C ABI
    and return every output as numpy (``weights``: per-block distortion
    weights, solved with kvq_solve_lambda_weighted)."""
    import torch
    from kv_cache_rate_amd import kvq
    dev = tensors_dev if tensors_dev is not None else to_cuda(tensors)
    sm = {"grids": kvq.KVQ_GRIDS, "exact_dp": kvq.KVQ_EXACT_DP, "beam": kvq.KVQ_BEAM}[search]
    plan = kvq.kvq_plan_blocks(dev, tokens_per_block, dims_per_block, s, sm,
                               alphabet_m if sm else 0, beam_width if search == "beam" else 0)
    buf = kvq.allocate(plan, dequant=dequant)
    md = {"bisect": kvq.KVQ_BISECT, "subgrad": kvq.KVQ_SUBGRAD,
          "bisect_greedy": kvq.KVQ_BISECT_GREEDY}[mode]
    if weights is None:
        lam_out, rate = kvq.admit(plan, dev, buf, B, md, iters, eta, lam, seed, dequant=dequant)
    else:
        wd = torch.from_numpy(np.ascontiguousarray(weights, dtype=np.float64)).cuda()
        kvq.kvq_eval_candidates(plan, dev, buf["D"], buf["H"], buf["stats"], buf["workspace"])
        lam_out, rate = kvq.kvq_solve_lambda_weighted(plan, buf["D"], buf["H"], wd, buf["stats"], B, md,
                                                      iters, eta, lam, buf["choice"], buf["codebook"],
                                                      buf["m"], buf["off"], buf["workspace"])
        kvq.kvq_quantize_pack(plan, dev, buf["codebook"], buf["m"], buf["off"], seed, buf["codes"])
        if dequant:
            kvq.kvq_dequantize(plan, buf["codes"], buf["codebook"], buf["m"], buf["off"], buf["xhat"])
    torch.cuda.synchronize()
    out = {k: v.cpu().numpy() for k, v in buf.items() if k != "workspace"}
    if sm == kvq.KVQ_GRIDS:  # candidate-major on the device; block-major here
        out["D"] = np.ascontiguousarray(out["D"].T)
        out["H"] = np.ascontiguousarray(out["H"].T)
        out["stats"] = np.ascontiguousarray(out["stats"].T)
    out["off"] = out["off"].view(np.uint64)
    out["codes"] = out["codes"].view(np.uint32)
    out["lam"] = lam_out
    out["rate_per_entry"] = rate
    out["plan"] = plan
    return out


def run_oracle(tensors, *, tokens_per_block, dims_per_block, s, search, alphabet_m=12, B, mode,
               iters=40, eta=1e-3, lam=0.0, seed=0, processes=None, weights=None, beam_width=0):
    b = oblocks.partition(tensors, tokens_per_block, dims_per_block)
    out = pipeline.run(b, search=search, s=s, alphabet_m=alphabet_m, B=B, mode=mode, iters=iters,
                       lam_prev=lam, eta=eta, seed=seed,
                       processes=processes or pipeline.default_processes(), weights=weights,
                       beam_width=beam_width or None)
    out["blocks"] = b
    return out


def rel_err(a, b, floor):
    return np.abs(a - b) / np.maximum(np.abs(b), floor)


def compare_tables(g, o, search):
    """D/H (or pair statistics) within D_RTOL; returns the max relative errors."""
    rep = {}
    if search == "grids":
        Dg, Hg, Do, Ho = g["D"], g["H"], o["D"], o["H"]
        floorD = 1e-9 * np.maximum(Do.max(axis=1, keepdims=True), 1e-300) / D_RTOL
        eD = rel_err(Dg, Do, floorD)
        eH = rel_err(Hg, Ho, 1e-9 / D_RTOL)
        rep["max_rel_D"] = float(eD.max())
        rep["max_rel_H"] = float(eH.max())
        assert eD.max() <= D_RTOL, rep
        assert eH.max() <= D_RTOL, rep
        assert np.array_equal(g["stats"].astype(np.float64), o["stats"]), "order statistics differ"
    else:
        R = g["D"].shape[0]
        M = g["stats"].shape[1]  # alphabet size of the pair triangle
        eD = 0.0
        eM = 0.0
        for r in range(R):
            Dp, ML, MR = o["pairs"][r]
            m = o["alphabets"][r].size
            for i in range(m):
                for j in range(i + 1, m):
                    p = i * (2 * M - i - 1) // 2 + (j - i - 1)
                    fl = 1e-9 * max(Dp.max(), 1e-300) / D_RTOL
                    eD = max(eD, abs(g["D"][r, p] - Dp[i, j]) / max(abs(Dp[i, j]), fl))
                    eM = max(eM, abs(g["H"][r, p, 0] - ML[i, j]) / max(abs(ML[i, j]), 1e-9 / D_RTOL))
                    eM = max(eM, abs(g["H"][r, p, 1] - MR[i, j]) / max(abs(MR[i, j]), 1e-9 / D_RTOL))
        rep["max_rel_pairD"] = float(eD)
        rep["max_rel_pairM"] = float(eM)
        assert eD <= D_RTOL and eM <= D_RTOL, rep
        assert np.array_equal(g["stats"].astype(np.float64), o["alphabet_raw"]), "alphabet differs"
    return rep


def compare_choice(g, o, lam, d, weights=None):
    """Codebooks identical by value except documented ties.  Returns
    (mask of blocks whose codebooks agree, tie count, max tie gap)."""
    R = g["m"].shape[0]
    agree = np.zeros(R, dtype=bool)
    ties = 0
    max_gap = 0.0
    if o.get("route") in ("dp", "beam"):
        return compare_choice_dp(g, o, lam, d)
    Dw = o["D"] if weights is None else np.asarray(weights, dtype=np.float64)[:, None] * o["D"]
    obj = Dw + (lam * d) * o["H"]
    for r in range(R):
        mg = int(g["m"][r])
        Qg = g["codebook"][r, :mg].astype(np.float64)
        Qo = o["chosen"][r]
        if mg == Qo.size and np.array_equal(Qg, Qo):
            agree[r] = True
            continue
        oc = o["choice"][r]
        if "subsets" in o:
            mask = int(g["choice"][r]) & 0xFFFFFFFF
            S = tuple(i for i in range(32) if mask >> i & 1)
            cand = o["subsets"][r].index(S)
            Qc = o["alphabets"][r][list(S)]
        else:
            cand = int(g["choice"][r])
            Qc = o["books"][r][cand]
        assert np.array_equal(Qc, Qg), f"block {r}: GPU codebook is not candidate {cand}"
        gap = (obj[r, cand] - obj[r, oc]) / max(abs(obj[r, oc]), 1e-300)
        assert gap < TIE_RTOL, f"block {r}: objective gap {gap} is not a tie"
        ties += 1
        max_gap = max(max_gap, gap)
    return agree, ties, max_gap


def subset_of_mask(mask):
    mask = int(mask) & 0xFFFFFFFF
    return tuple(i for i in range(32) if mask >> i & 1)


def compare_choice_dp(g, o, lam, d, blocks=None):
    """Exact search solved by the oracle's DP route: the GPU's subset (its
    bitmask) equals the oracle's, except documented ties whose objectives
    D + lam d H (scored from the oracle's pair statistics) differ by <
    TIE_RTOL relative.  ``blocks`` restricts the check to those block
    indices (the oracle's lists then hold those blocks in that order)."""
    rows = range(g["m"].shape[0]) if blocks is None else blocks
    agree = np.zeros(g["m"].shape[0], dtype=bool)
    ties = 0
    max_gap = 0.0
    n = int(o["n"])
    for k, r in enumerate(rows):
        kk = r if blocks is None else k
        Sg = subset_of_mask(g["choice"][r])
        So = tuple(o["subsets_chosen"][kk])
        A = o["alphabets"][kk]
        mg = int(g["m"][r])
        assert mg == len(Sg) and np.array_equal(g["codebook"][r, :mg].astype(np.float64), A[list(Sg)]), \
            f"block {r}: codebook is not the masked alphabet points"
        if Sg == So:
            agree[r] = True
            continue
        Dp, ML, MR = o["pairs"][kk]
        Dg_, Hg_ = exact_dp.subset_score(Dp, ML, MR, n, Sg)
        Do_, Ho_ = exact_dp.subset_score(Dp, ML, MR, n, So)
        og, oo = Dg_ + (lam * d) * Hg_, Do_ + (lam * d) * Ho_
        gap = (og - oo) / max(abs(oo), 1e-300)
        assert gap < TIE_RTOL, f"block {r}: objective gap {gap} is not a tie"
        ties += 1
        max_gap = max(max_gap, gap)
    return agree, ties, max_gap


def compare_codes(g, o, agree, seed):
    """Codes bit-exact for blocks with equal codebooks, except near draws."""
    n = o["n"]
    R = o["R"]
    mismatched = 0
    off_g = g["off"]
    for r in range(R):
        w = int(ocodes.code_width(int(g["m"][r])))
        seg = g["codes"][int(off_g[r]):int(off_g[r + 1])]
        cg = ocodes.unpack_block(seg, n, w)
        # decoded entries are exactly the stored codepoints
        if "xhat" in g:
            Qg = g["codebook"][r]
            assert np.array_equal(g["xhat"][r], Qg[cg.astype(np.int64)]), f"block {r}: decode"
        if not agree[r]:
            continue
        co = o["codes"][r]
        diff = cg != co
        if diff.any():
            near = ocodes.near_mask(o["blocks"][r], o["chosen"][r], seed, r)
            assert np.all(near[diff]), f"block {r}: code differs away from |u-p|<1e-6"
            mismatched += int(diff.sum())
    return mismatched


LAM_RTOL = 1e-6


def full_compare(g, o, search, seed, B=None, mode="bisect", lam_used_gpu=None, weights=None):
    """Compare a GPU run with an oracle run on the same inputs.

    The two bisections replay the same probes; they can part only where a
    probe's modelled rate lies within the tables' round-off of the budget.
    Then both multipliers must be feasible and within LAM_RTOL, and every
    block whose codebook differs must be a documented tie at the oracle's
    multiplier (checked by compare_choice)."""
    rep = compare_tables(g, o, search)
    d = float(o["n"])
    rep["lam_path_divergence"] = 0
    if mode == "bisect":
        assert g["rate_per_entry"] <= B + 1e-12
        assert o["rate_per_entry"] <= B + 1e-12
        if g["lam"] != o["lam"]:
            assert abs(g["lam"] - o["lam"]) <= LAM_RTOL * max(abs(o["lam"]), 1e-300), \
                (g["lam"], o["lam"])
            rep["lam_path_divergence"] = 1
    rep["lam"] = g["lam"]
    lam_used = o["lam"] if mode == "bisect" else o["lam_used"]
    agree, ties, gap = compare_choice(g, o, lam_used, d, weights)
    rep["ties"] = ties
    rep["max_tie_gap"] = gap
    assert np.array_equal(g["m"], o["m"]) or ties > 0
    if ties == 0 and rep["lam_path_divergence"] == 0:
        assert np.array_equal(g["off"], o["offsets"]), "offsets differ"
    rep["code_mismatch_near"] = compare_codes(g, o, agree, seed)
    rep["oracle_near"] = o["near"]
    # every differing code is one of the oracle's near draws
    assert rep["code_mismatch_near"] <= o["near"], rep
    return rep
