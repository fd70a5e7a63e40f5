"""Thin ctypes binding of libkvq (include/kvq.h).

The functions keep the C names (``kvq_plan_blocks``, ``kvq_eval_candidates``,
``kvq_solve_lambda``, ``kvq_quantize_pack``, ``kvq_dequantize``) and only
marshal arguments: every step of the computation runs in the HIP kernels of
``libkvq.so``.  PyTorch provides device memory and the current stream.  The
library is loaded on first use; if it is missing the call raises (there is
no CPU fallback).
"""

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
# KVQ_LIB names another build of the same library (the host-sanitizer build
# of the CPU validation tests); by default the in-tree libkvq.so.
LIB_PATH = os.environ.get("KVQ_LIB") or os.path.join(PKG, "libkvq.so")

KVQ_OK = 0
KVQ_EINVAL = -1
KVQ_EINFEASIBLE = -2
KVQ_ENONFINITE = -3
KVQ_ENOSPC = -4
KVQ_EHIP = -5

KVQ_F16 = 1
KVQ_F32 = 2
KVQ_GRIDS = 0
KVQ_EXACT_DP = 1
KVQ_BEAM = 2
KVQ_BISECT = 0
KVQ_SUBGRAD = 1
KVQ_BISECT_GREEDY = 2

EXPORTED = ("kvq_status_string", "kvq_last_error", "kvq_plan_blocks", "kvq_eval_candidates",
            "kvq_solve_lambda", "kvq_solve_lambda_weighted", "kvq_quantize_pack", "kvq_admit",
            "kvq_admit_noalloc",
            "kvq_dequantize",
            "kvq_ans_sizes",
            "kvq_ans_encode", "kvq_ans_decode", "kvq_decode_attention_workspace",
            "kvq_decode_attention")


class KvqTensor(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p), ("dtype", ctypes.c_int32), ("pad_", ctypes.c_int32),
                ("shape", ctypes.c_int64 * 4), ("stride", ctypes.c_int64 * 4)]


class KvqBlockSpec(ctypes.Structure):
    _fields_ = [("tokens_per_block", ctypes.c_int32), ("dims_per_block", ctypes.c_int32),
                ("s", ctypes.c_int32), ("search", ctypes.c_int32), ("alphabet_m", ctypes.c_int32),
                ("beam_width", ctypes.c_int32)]


class KvqPlan(ctypes.Structure):
    _fields_ = [("n_blocks", ctypes.c_int64), ("n_entries", ctypes.c_int64),
                ("d_block", ctypes.c_int32), ("n_cand", ctypes.c_int32),
                ("n_stats", ctypes.c_int32), ("s", ctypes.c_int32), ("search", ctypes.c_int32),
                ("alphabet_m", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("n_tensors", ctypes.c_int32), ("tokens_per_block", ctypes.c_int32),
                ("dims_per_block", ctypes.c_int32),
                ("tensor_blocks", ctypes.c_int64 * 2), ("shape", (ctypes.c_int64 * 4) * 2),
                ("D_bytes", ctypes.c_size_t), ("H_bytes", ctypes.c_size_t),
                ("stats_bytes", ctypes.c_size_t), ("choice_bytes", ctypes.c_size_t),
                ("codebook_bytes", ctypes.c_size_t), ("m_bytes", ctypes.c_size_t),
                ("offsets_bytes", ctypes.c_size_t), ("workspace_bytes", ctypes.c_size_t),
                ("max_code_words", ctypes.c_uint64), ("rate_shift", ctypes.c_int32),
                ("beam_width", ctypes.c_int32)]


class KvqError(RuntimeError):
    def __init__(self, status, detail):
        super().__init__(f"{status_string(status)} ({detail})")
        self.status = status
        self.detail = detail


_LIB = None


def lib():
    """Load libkvq.so (raises if it has not been built)."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m kv_cache_rate_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, i64, u64, f64 = (ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64,
                                  ctypes.c_uint64, ctypes.c_double)
        L.kvq_status_string.restype = ctypes.c_char_p
        L.kvq_status_string.argtypes = [i32]
        L.kvq_last_error.restype = ctypes.c_char_p
        L.kvq_last_error.argtypes = []
        L.kvq_plan_blocks.restype = i32
        L.kvq_plan_blocks.argtypes = [ctypes.POINTER(KvqTensor), i32, ctypes.POINTER(KvqBlockSpec),
                                      ctypes.POINTER(KvqPlan)]
        L.kvq_eval_candidates.restype = i32
        L.kvq_eval_candidates.argtypes = [ctypes.POINTER(KvqPlan), ctypes.POINTER(KvqTensor), i32,
                                          vp, vp, vp, vp, vp]
        L.kvq_solve_lambda.restype = i32
        L.kvq_solve_lambda.argtypes = [ctypes.POINTER(KvqPlan), vp, vp, vp, f64, i32, i32, f64,
                                       ctypes.POINTER(f64), ctypes.POINTER(f64), vp, vp, vp, vp,
                                       vp, vp]
        L.kvq_solve_lambda_weighted.restype = i32
        L.kvq_solve_lambda_weighted.argtypes = [ctypes.POINTER(KvqPlan), vp, vp, vp, vp, f64, i32, i32,
                                                f64, ctypes.POINTER(f64), ctypes.POINTER(f64), vp, vp,
                                                vp, vp, vp, vp]
        L.kvq_quantize_pack.restype = i32
        L.kvq_quantize_pack.argtypes = [ctypes.POINTER(KvqPlan), ctypes.POINTER(KvqTensor), i32,
                                        vp, vp, vp, u64, vp, u64, vp]
        L.kvq_admit.restype = i32
        L.kvq_admit.argtypes = [ctypes.POINTER(KvqPlan), ctypes.POINTER(KvqTensor), i32, vp, vp, vp, f64,
                                i32, i32, f64, ctypes.POINTER(f64), ctypes.POINTER(f64), vp, vp, vp, vp,
                                u64, vp, u64, vp, vp]
        L.kvq_admit_noalloc.restype = i32
        L.kvq_admit_noalloc.argtypes = [ctypes.POINTER(KvqPlan), ctypes.POINTER(KvqTensor), i32, vp, vp, vp,
                                        f64, i32, i32, f64, ctypes.POINTER(f64), ctypes.POINTER(f64), vp, vp,
                                        vp, vp, u64, vp, u64, vp]
        L.kvq_dequantize.restype = i32
        L.kvq_dequantize.argtypes = [ctypes.POINTER(KvqPlan), vp, vp, vp, vp, vp, vp]
        L.kvq_ans_sizes.restype = i32
        L.kvq_ans_sizes.argtypes = [ctypes.POINTER(KvqPlan), ctypes.POINTER(u64), ctypes.POINTER(u64)]
        L.kvq_ans_encode.restype = i32
        L.kvq_ans_encode.argtypes = [ctypes.POINTER(KvqPlan), vp, vp, vp, vp, u64, vp, u64, vp, vp,
                                     ctypes.POINTER(u64), vp]
        L.kvq_decode_attention_workspace.restype = i32
        L.kvq_decode_attention_workspace.argtypes = [ctypes.POINTER(KvqPlan), i32, ctypes.POINTER(u64)]
        L.kvq_decode_attention.restype = i32
        L.kvq_decode_attention.argtypes = [ctypes.POINTER(KvqPlan), vp, vp, vp, vp, vp, i32,
                                           ctypes.c_float, vp, vp, u64, vp]
        L.kvq_ans_decode.restype = i32
        L.kvq_ans_decode.argtypes = [ctypes.POINTER(KvqPlan), vp, vp, vp, vp, vp, vp, vp]
        _LIB = L
    return _LIB


def status_string(st):
    return lib().kvq_status_string(st).decode()


def last_error():
    return lib().kvq_last_error().decode()


def _check(st):
    if st != KVQ_OK:
        raise KvqError(st, last_error())


_DTYPE_CODES = {}  # dtype object -> KVQ_F16 / KVQ_F32, filled on first sight


def _dtype_code(t):
    dt = getattr(t, "dtype", None)
    code = _DTYPE_CODES.get(dt)
    if code is None:
        name = str(dt)
        if name.endswith("float16"):
            code = KVQ_F16
        elif name.endswith("float32"):
            code = KVQ_F32
        else:
            raise ValueError(f"unsupported KV dtype {name}")
        _DTYPE_CODES[dt] = code
    return code


_I64x4 = ctypes.c_int64 * 4


def as_kvq_tensor(t):
    """Describe a 4-D torch tensor (or numpy array, for planning only)."""
    if t.ndim != 4:
        raise ValueError("KV tensors are [outer, heads, tokens, dim]")
    if hasattr(t, "data_ptr"):
        data = t.data_ptr()
        strides = t.stride()
    else:  # numpy: planning reads shapes and strides only
        data = t.ctypes.data
        strides = tuple(s // t.itemsize for s in t.strides)
    return KvqTensor(data, _dtype_code(t), 0, _I64x4(*t.shape), _I64x4(*strides))


def _tensor_array(tensors):
    return (KvqTensor * len(tensors))(*[as_kvq_tensor(t) for t in tensors])


def _ptr(x):
    if x is None:
        return None
    return x.data_ptr() if hasattr(x, "data_ptr") else int(x)


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    return getattr(stream, "cuda_stream", stream)


def kvq_plan_blocks(tensors, tokens_per_block, dims_per_block, s, search=KVQ_GRIDS, alphabet_m=0,
                    beam_width=0):
    spec = KvqBlockSpec(tokens_per_block, dims_per_block, s, search, alphabet_m, beam_width)
    plan = KvqPlan()
    arr = _tensor_array(tensors)
    _check(lib().kvq_plan_blocks(arr, len(tensors), ctypes.byref(spec), ctypes.byref(plan)))
    return plan


def kvq_eval_candidates(plan, tensors, D, H, stats, workspace, stream=None):
    arr = _tensor_array(tensors)
    _check(lib().kvq_eval_candidates(ctypes.byref(plan), arr, len(tensors), _ptr(D), _ptr(H),
                                     _ptr(stats), _ptr(workspace), _stream(stream)))


def kvq_solve_lambda(plan, D, H, stats, B, mode, iters, eta, lam, choice, codebook, m, word_off,
                     workspace, stream=None):
    """Returns ``(lambda, rate_bits_per_entry)``."""
    lam_io = ctypes.c_double(lam)
    rate = ctypes.c_double(0.0)
    _check(lib().kvq_solve_lambda(ctypes.byref(plan), _ptr(D), _ptr(H), _ptr(stats), float(B), mode,
                                  iters, float(eta), ctypes.byref(lam_io), ctypes.byref(rate),
                                  _ptr(choice), _ptr(codebook), _ptr(m), _ptr(word_off),
                                  _ptr(workspace), _stream(stream)))
    return lam_io.value, rate.value


def kvq_solve_lambda_weighted(plan, D, H, weight, stats, B, mode, iters, eta, lam, choice, codebook,
                              m, word_off, workspace, stream=None):
    """Returns ``(lambda, rate_bits_per_entry)``; ``weight`` is a device
    fp64 [R] array (or None)."""
    lam_io = ctypes.c_double(lam)
    rate = ctypes.c_double(0.0)
    _check(lib().kvq_solve_lambda_weighted(ctypes.byref(plan), _ptr(D), _ptr(H), _ptr(weight), _ptr(stats),
                                           float(B), mode, iters, float(eta), ctypes.byref(lam_io),
                                           ctypes.byref(rate), _ptr(choice), _ptr(codebook), _ptr(m),
                                           _ptr(word_off), _ptr(workspace), _stream(stream)))
    return lam_io.value, rate.value


def kvq_quantize_pack(plan, tensors, codebook, m, word_off, seed, codes, capacity_words=None,
                      stream=None):
    arr = _tensor_array(tensors)
    cap = capacity_words if capacity_words is not None else codes.numel()
    _check(lib().kvq_quantize_pack(ctypes.byref(plan), arr, len(tensors), _ptr(codebook), _ptr(m),
                                   _ptr(word_off), int(seed), _ptr(codes), int(cap),
                                   _stream(stream)))


def kvq_dequantize(plan, codes, codebook, m, word_off, xhat, stream=None):
    _check(lib().kvq_dequantize(ctypes.byref(plan), _ptr(codes), _ptr(codebook), _ptr(m),
                                _ptr(word_off), _ptr(xhat), _stream(stream)))


def kvq_ans_sizes(plan):
    """Returns ``(scratch_bytes, stream_bytes)``."""
    a, b = ctypes.c_uint64(0), ctypes.c_uint64(0)
    _check(lib().kvq_ans_sizes(ctypes.byref(plan), ctypes.byref(a), ctypes.byref(b)))
    return a.value, b.value


def kvq_ans_encode(plan, codes, m, word_off, scratch, stream, block_off, workspace, stream_obj=None):
    """Returns the coded stream's length in bytes."""
    total = ctypes.c_uint64(0)
    _check(lib().kvq_ans_encode(ctypes.byref(plan), _ptr(codes), _ptr(m), _ptr(word_off), _ptr(scratch),
                                int(scratch.numel() * scratch.element_size()), _ptr(stream),
                                int(stream.numel() * stream.element_size()), _ptr(block_off),
                                _ptr(workspace), ctypes.byref(total), _stream(stream_obj)))
    return total.value


def kvq_ans_decode(plan, stream, block_off, codebook, m, xhat, workspace, stream_obj=None):
    _check(lib().kvq_ans_decode(ctypes.byref(plan), _ptr(stream), _ptr(block_off), _ptr(codebook),
                                _ptr(m), _ptr(xhat), _ptr(workspace), _stream(stream_obj)))


def kvq_decode_attention_workspace(plan, q_heads):
    b = ctypes.c_uint64(0)
    _check(lib().kvq_decode_attention_workspace(ctypes.byref(plan), int(q_heads), ctypes.byref(b)))
    return b.value


def kvq_decode_attention(plan, codes, codebook, m, word_off, q, q_heads, scale, out, work, stream=None):
    _check(lib().kvq_decode_attention(ctypes.byref(plan), _ptr(codes), _ptr(codebook), _ptr(m),
                                      _ptr(word_off), _ptr(q), int(q_heads), float(scale), _ptr(out),
                                      _ptr(work), int(work.numel() * work.element_size()),
                                      _stream(stream)))


def allocate_ans(plan, device="cuda"):
    """Device buffers for kvq_ans_encode / kvq_ans_decode."""
    import torch
    sb, tb = kvq_ans_sizes(plan)
    return {"scratch": torch.empty(max(4, sb), dtype=torch.uint8, device=device),
            "stream": torch.empty(max(4, tb), dtype=torch.uint8, device=device),
            "block_off": torch.empty(plan.n_blocks + 1, dtype=torch.int64, device=device)}


# ---------------------------------------------------------------------------
# Buffer allocation and chaining (marshalling only; no arithmetic).

def allocate(plan, device="cuda", dequant=False):
    """Device buffers of the sizes ``plan`` asks for, as torch tensors
    (GRIDS tables are candidate-major: D, H are [C, R], stats [n_stats, R]).

    64-bit offsets are held in an int64 tensor and codes in an int32 tensor
    (same bits as the uint64 / uint32 the library writes)."""
    import torch
    R = plan.n_blocks
    if plan.search == KVQ_GRIDS:  # candidate-major tables
        D = torch.empty((plan.n_cand, R), dtype=torch.float64, device=device)
        H = torch.empty((plan.n_cand, R), dtype=torch.float64, device=device)
        stats = torch.empty((plan.n_stats, R), dtype=torch.float32, device=device)
    else:
        D = torch.empty((R, plan.n_cand), dtype=torch.float64, device=device)
        H = torch.empty((R, plan.n_cand, 2), dtype=torch.float64, device=device)
        stats = torch.empty((R, plan.n_stats), dtype=torch.float32, device=device)
    buf = {
        "D": D, "H": H, "stats": stats,
        "choice": torch.empty(R, dtype=torch.int32, device=device),
        "codebook": torch.empty((R, plan.s), dtype=torch.float32, device=device),
        "m": torch.empty(R, dtype=torch.uint8, device=device),
        "off": torch.empty(R + 1, dtype=torch.int64, device=device),
        "workspace": torch.empty(plan.workspace_bytes, dtype=torch.uint8, device=device),
        "codes": torch.empty(max(1, plan.max_code_words), dtype=torch.int32, device=device),
    }
    if dequant:
        buf["xhat"] = torch.empty((R, plan.d_block), dtype=torch.float32, device=device)
    return buf


def kvq_admit(plan, tensors, buf, B, mode=KVQ_BISECT, iters=40, eta=1e-3, lam=0.0, seed=0, stream=None):
    """kvq_eval_candidates, kvq_solve_lambda and kvq_quantize_pack in one C
    call with one wait at the end, on the buffers of ``buf`` (as allocate()
    returns them).  Returns ``(lambda, rate_bits_per_entry)``."""
    arr = _tensor_array(tensors)
    lam_io = ctypes.c_double(lam)
    rate = ctypes.c_double(0.0)
    codes = buf["codes"]
    _check(lib().kvq_admit(ctypes.byref(plan), arr, len(tensors), _ptr(buf["D"]), _ptr(buf["H"]),
                           _ptr(buf["stats"]), float(B), mode, iters, float(eta), ctypes.byref(lam_io),
                           ctypes.byref(rate), _ptr(buf["choice"]), _ptr(buf["codebook"]), _ptr(buf["m"]),
                           _ptr(buf["off"]), int(seed), _ptr(codes), int(codes.numel()),
                           _ptr(buf["workspace"]), _stream(stream)))
    return lam_io.value, rate.value


def prepare_admit(plan, tensors, buf, B, mode=KVQ_SUBGRAD, iters=40, eta=1e-3, seed=0, stream=None,
                  noalloc=False):
    """kvq_admit (or, with ``noalloc``, kvq_admit_noalloc) for a loop over one
    set of buffers, such as a decode loop: the arguments are marshalled once
    and each call only sets the incoming multiplier.  The tensors' contents
    may change between calls; their storage and shapes, the buffers and the
    stream may not.  Returns a function ``lam -> (lambda,
    rate_bits_per_entry)`` with kvq_admit's results."""
    L = lib()
    fn = L.kvq_admit_noalloc if noalloc else L.kvq_admit
    vp = ctypes.c_void_p
    arr = _tensor_array(tensors)
    lam_io = ctypes.c_double(0.0)
    rate = ctypes.c_double(0.0)
    codes = buf["codes"]
    args = [ctypes.byref(plan), arr, ctypes.c_int32(len(tensors)), vp(_ptr(buf["D"])), vp(_ptr(buf["H"])),
            vp(_ptr(buf["stats"])), ctypes.c_double(B), ctypes.c_int32(mode), ctypes.c_int32(iters),
            ctypes.c_double(eta), ctypes.byref(lam_io), ctypes.byref(rate), vp(_ptr(buf["choice"])),
            vp(_ptr(buf["codebook"])), vp(_ptr(buf["m"])), vp(_ptr(buf["off"])), ctypes.c_uint64(int(seed)),
            vp(_ptr(codes)), ctypes.c_uint64(int(codes.numel()))]
    if not noalloc:
        args.append(vp(_ptr(buf["workspace"])))
    args.append(vp(_stream(stream)))
    keep = (plan, tensors, buf, arr)

    def call(lam):
        lam_io.value = lam
        st = fn(*args)
        if st:
            raise KvqError(st, last_error())
        return lam_io.value, rate.value
    call.keep = keep  # the marshalled pointers stay valid while the call lives
    return call


def kvq_admit_noalloc(plan, tensors, buf, B, mode=KVQ_BISECT, iters=40, eta=1e-3, lam=0.0, seed=0,
                      stream=None):
    """kvq_admit with the library's static device scratch in place of a
    workspace (no allocation in the call).  Returns ``(lambda,
    rate_bits_per_entry)``."""
    arr = _tensor_array(tensors)
    lam_io = ctypes.c_double(lam)
    rate = ctypes.c_double(0.0)
    codes = buf["codes"]
    _check(lib().kvq_admit_noalloc(ctypes.byref(plan), arr, len(tensors), _ptr(buf["D"]), _ptr(buf["H"]),
                                   _ptr(buf["stats"]), float(B), mode, iters, float(eta), ctypes.byref(lam_io),
                                   ctypes.byref(rate), _ptr(buf["choice"]), _ptr(buf["codebook"]),
                                   _ptr(buf["m"]), _ptr(buf["off"]), int(seed), _ptr(codes),
                                   int(codes.numel()), _stream(stream)))
    return lam_io.value, rate.value


def admit(plan, tensors, buf, B, mode=KVQ_BISECT, iters=40, eta=1e-3, lam=0.0, seed=0,
          stream=None, dequant=False):
    """Chain eval -> solve -> quantize_pack (-> dequantize) on ``buf``.
    Returns ``(lambda, rate_bits_per_entry)``."""
    kvq_eval_candidates(plan, tensors, buf["D"], buf["H"], buf["stats"], buf["workspace"], stream)
    lam, rate = kvq_solve_lambda(plan, buf["D"], buf["H"], buf["stats"], B, mode, iters, eta, lam,
                                 buf["choice"], buf["codebook"], buf["m"], buf["off"],
                                 buf["workspace"], stream)
    kvq_quantize_pack(plan, tensors, buf["codebook"], buf["m"], buf["off"], seed, buf["codes"],
                      stream=stream)
    if dequant:
        kvq_dequantize(plan, buf["codes"], buf["codebook"], buf["m"], buf["off"], buf["xhat"], stream)
    return lam, rate
