"""The C-ABI library loads, exports every declared symbol, and validates
arguments on the host (CPU only: no call here touches a GPU)."""

import ctypes
import os
import re
import subprocess

import numpy as np
import pytest

from kv_cache_rate_amd import kvq
from kv_cache_rate_amd import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kvq.h")


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*(kvq_[a-z_]+)\s*\(", text, re.M)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(kvq.LIB_PATH):
        pytest.fail("libkvq.so is not built (run python -m kv_cache_rate_amd.build)")
    return kvq.lib()


def test_exports_every_declared_symbol(L):
    names = declared_functions()
    assert set(names) == set(kvq.EXPORTED)
    out = subprocess.run(["nm", "-D", "--defined-only", kvq.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
    for n in names:
        assert n in exported, n
        assert hasattr(L, n)


def test_status_strings(L):
    for st in (0, -1, -2, -3, -4, -5):
        assert kvq.status_string(st).startswith("KVQ_")
    assert "unknown" in kvq.status_string(7)


def _np(shape, dtype=np.float16):
    return np.zeros(shape, dtype=dtype)


@pytest.mark.parametrize("w", W.WORKLOADS, ids=[w.name for w in W.WORKLOADS])
def test_plan_sizes(L, w):
    ts = [np.lib.stride_tricks.as_strided(np.zeros(1, w.np_dtype), shape=shp,
                                          strides=(0, 0, 0, 0)) for _, shp in w.tensors]
    # as_strided with zero strides would give zero element strides; give real ones
    ts = []
    for _, shp in w.tensors:
        o, h, t, d = shp
        base = np.zeros(1, dtype=w.np_dtype)
        ts.append(np.lib.stride_tricks.as_strided(
            base, shape=shp, strides=tuple(s * base.itemsize for s in (h * t * d, t * d, d, 1))))
    search = kvq.KVQ_GRIDS if w.search == "grids" else kvq.KVQ_EXACT_DP
    p = kvq.kvq_plan_blocks(ts, w.tokens_per_block, w.dims_per_block, w.s, search,
                            w.alphabet_m if search else 0)
    assert p.n_blocks == w.n_blocks
    assert p.n_entries == w.n_entries
    assert p.d_block == 4096
    if search == kvq.KVQ_GRIDS:
        assert p.n_cand == 1 + 2 * (w.s - 2)
        assert p.n_stats == (73 if w.s == 16 else 19)
        assert p.D_bytes == w.n_blocks * p.n_cand * 8
    else:
        assert p.n_cand == 66 and p.n_stats == 12
        assert p.D_bytes == w.n_blocks * 66 * 8 and p.H_bytes == 2 * p.D_bytes
    assert p.max_code_words == w.n_blocks * (4096 * (w.s - 1).bit_length() // 32)
    assert p.codebook_bytes == w.n_blocks * w.s * 4
    assert p.offsets_bytes == (w.n_blocks + 1) * 8
    # the exact rate sums cannot overflow 64 bits
    assert w.n_entries * 4 * 2.0 ** p.rate_shift < 2.0 ** 63


def test_plan_rejects_bad_arguments(L):
    t = np.zeros((1, 2, 64, 128), dtype=np.float16)
    with pytest.raises(kvq.KvqError) as e:
        kvq.kvq_plan_blocks([t], 30, 128, 16)  # 64 tokens not a multiple of 30
    assert e.value.status == kvq.KVQ_EINVAL
    with pytest.raises(kvq.KvqError) as e:
        kvq.kvq_plan_blocks([t], 32, 128, 17)  # s > 16
    assert e.value.status == kvq.KVQ_EINVAL and "s=17" in e.value.detail
    with pytest.raises(kvq.KvqError):
        kvq.kvq_plan_blocks([t], 64, 128, 16)  # 8192 entries per block
    with pytest.raises(kvq.KvqError):
        kvq.kvq_plan_blocks([t, t.astype(np.float32)], 32, 128, 16)  # dtype mismatch
    with pytest.raises(kvq.KvqError):
        kvq.kvq_plan_blocks([t], 32, 128, 8, kvq.KVQ_EXACT_DP, 33)  # alphabet > 32
    with pytest.raises(kvq.KvqError):
        kvq.kvq_plan_blocks([t], 32, 128, 8, kvq.KVQ_EXACT_DP, 1)  # alphabet < 2
    with pytest.raises(ValueError):
        kvq.kvq_plan_blocks([t.astype(np.float64)], 32, 128, 16)
    with pytest.raises(kvq.KvqError) as e:
        kvq.kvq_plan_blocks([np.zeros((1, 2, 0, 128), dtype=np.float16)], 32, 128, 16)  # no tokens
    assert e.value.status == kvq.KVQ_EINVAL and "empty" in e.value.detail
    with pytest.raises(kvq.KvqError) as e:
        kvq.kvq_plan_blocks([], 32, 128, 16)  # no tensor
    assert e.value.status == kvq.KVQ_EINVAL


def test_plan_larger_alphabet(L):
    """A 32-point alphabet has 496 pairs; the tables scale with it."""
    t = np.zeros((1, 8, 8192, 128), dtype=np.float32)
    p = kvq.kvq_plan_blocks([t], 256, 16, 16, kvq.KVQ_EXACT_DP, 32)
    assert p.n_cand == 32 * 31 // 2 == 496 and p.n_stats == 32
    assert p.D_bytes == 2048 * 496 * 8 and p.H_bytes == 2 * p.D_bytes
    assert p.stats_bytes == 2048 * 32 * 4
    assert p.max_code_words == 2048 * (4096 * 4 // 32)


def test_plan_beam(L):
    """KVQ_BEAM plans like KVQ_EXACT_DP (same alphabet tables) and carries
    its width; widths outside 1..8 and missing alphabets are rejected."""
    t = np.zeros((1, 8, 8192, 128), dtype=np.float32)
    p = kvq.kvq_plan_blocks([t], 256, 16, 16, kvq.KVQ_BEAM, 32, 4)
    assert p.search == kvq.KVQ_BEAM and p.beam_width == 4
    assert p.n_cand == 496 and p.n_stats == 32 and p.H_bytes == 2 * p.D_bytes
    q = kvq.kvq_plan_blocks([t], 256, 16, 16, kvq.KVQ_EXACT_DP, 32)
    assert q.beam_width == 0 and q.D_bytes == p.D_bytes
    for width in (0, 9):
        with pytest.raises(kvq.KvqError) as e:
            kvq.kvq_plan_blocks([t], 256, 16, 16, kvq.KVQ_BEAM, 32, width)
        assert e.value.status == kvq.KVQ_EINVAL and "beam_width" in e.value.detail
    with pytest.raises(kvq.KvqError):
        kvq.kvq_plan_blocks([t], 256, 16, 16, kvq.KVQ_BEAM, 0, 2)  # no alphabet
    with pytest.raises(kvq.KvqError):
        kvq.kvq_plan_blocks([t], 256, 16, 16, 3, 12)  # unknown search


def test_calls_validate_before_launch(L):
    """Null pointers, mismatched tensors and short code buffers are refused on
    the host; nothing is launched so no GPU is needed."""
    t = np.zeros((1, 2, 64, 128), dtype=np.float16)
    p = kvq.kvq_plan_blocks([t], 32, 128, 16)
    lam = ctypes.c_double(0.0)
    rate = ctypes.c_double(0.0)
    Lb = kvq.lib()
    arr = kvq._tensor_array([t])
    assert Lb.kvq_eval_candidates(ctypes.byref(p), arr, 1, None, None, None, None, None) == kvq.KVQ_EINVAL
    assert "null" in kvq.last_error()
    other = np.zeros((1, 2, 96, 128), dtype=np.float16)
    arr2 = kvq._tensor_array([other])
    assert Lb.kvq_eval_candidates(ctypes.byref(p), arr2, 1, 8, 8, 8, 8, None) == kvq.KVQ_EINVAL
    assert "shape" in kvq.last_error()
    assert Lb.kvq_solve_lambda(ctypes.byref(p), 8, 8, 8, -1.0, 0, 40, 0.0, ctypes.byref(lam),
                               ctypes.byref(rate), 8, 8, 8, 8, 8, None) == kvq.KVQ_EINVAL
    assert Lb.kvq_solve_lambda(ctypes.byref(p), 8, 8, 8, 2.0, 5, 40, 0.0, ctypes.byref(lam),
                               ctypes.byref(rate), 8, 8, 8, 8, 8, None) == kvq.KVQ_EINVAL
    assert Lb.kvq_quantize_pack(ctypes.byref(p), arr, 1, 8, 8, 8, 0, 8, p.max_code_words - 1,
                                None) == kvq.KVQ_ENOSPC
    assert Lb.kvq_dequantize(ctypes.byref(p), 8, None, 8, 8, 8, None) == kvq.KVQ_EINVAL


def test_admit_validates_before_launch(L):
    """kvq_admit checks the arguments of all three steps before it launches
    anything: null tables, a greedy or unknown mode, a negative budget and a
    short code buffer are refused on the host (the pointers are not
    dereferenced, so no GPU is needed)."""
    t = np.zeros((1, 2, 64, 128), dtype=np.float16)
    p = kvq.kvq_plan_blocks([t], 32, 128, 16)
    lam = ctypes.c_double(0.0)
    rate = ctypes.c_double(0.0)
    Lb = kvq.lib()
    arr = kvq._tensor_array([t])

    def call(D=8, B=2.0, mode=kvq.KVQ_BISECT, cap=None):
        return Lb.kvq_admit(ctypes.byref(p), arr, 1, D, 8, 8, B, mode, 40, 1e-3, ctypes.byref(lam),
                            ctypes.byref(rate), 8, 8, 8, 8, 0, 8,
                            p.max_code_words if cap is None else cap, 8, None)
    assert call(D=None) == kvq.KVQ_EINVAL
    assert call(mode=kvq.KVQ_BISECT_GREEDY) == kvq.KVQ_EINVAL
    assert "kvq_admit" in kvq.last_error()
    assert call(mode=7) == kvq.KVQ_EINVAL
    assert call(B=-1.0) == kvq.KVQ_EINVAL
    assert call(cap=p.max_code_words - 1) == kvq.KVQ_ENOSPC


def test_admit_noalloc_validates_before_launch(L):
    """kvq_admit_noalloc refuses on the host, before it touches its static
    scratch or any GPU: bad arguments as kvq_admit does, and a plan whose
    solve scratch exceeds the static 44 KB (more than 3,668,992 blocks)."""
    Lb = kvq.lib()
    lam = ctypes.c_double(0.0)
    rate = ctypes.c_double(0.0)

    def call(p, arr, D=8, B=2.0, mode=kvq.KVQ_BISECT, cap=None):
        return Lb.kvq_admit_noalloc(ctypes.byref(p), arr, 1, D, 8, 8, B, mode, 40, 1e-3, ctypes.byref(lam),
                                    ctypes.byref(rate), 8, 8, 8, 8, 0, 8,
                                    p.max_code_words if cap is None else cap, None)
    t = np.zeros((1, 2, 64, 128), dtype=np.float16)
    p = kvq.kvq_plan_blocks([t], 32, 128, 16)
    arr = kvq._tensor_array([t])
    assert call(p, arr, D=None) == kvq.KVQ_EINVAL
    assert call(p, arr, mode=kvq.KVQ_BISECT_GREEDY) == kvq.KVQ_EINVAL
    assert "kvq_admit_noalloc" in kvq.last_error()
    assert call(p, arr, mode=7) == kvq.KVQ_EINVAL
    assert call(p, arr, B=-1.0) == kvq.KVQ_EINVAL
    assert call(p, arr, cap=p.max_code_words - 1) == kvq.KVQ_ENOSPC
    # the largest plan the scratch holds is accepted past this check (it then
    # fails only on the missing pointers); one block more is refused
    base = np.zeros(1, dtype=np.float16)
    for blocks, want in ((3668993, kvq.KVQ_ENOSPC), (3668992, kvq.KVQ_EINVAL)):
        big = np.lib.stride_tricks.as_strided(base, shape=(1, 1, 32 * blocks, 128), strides=(2, 2, 256, 2))
        pb = kvq.kvq_plan_blocks([big], 32, 128, 16)
        assert pb.n_blocks == blocks
        got = call(pb, kvq._tensor_array([big]), D=8 if want == kvq.KVQ_ENOSPC else None)
        assert got == want, (blocks, got, kvq.last_error())
        if want == kvq.KVQ_ENOSPC:
            assert "3668992" in kvq.last_error()


def test_entropy_coding_sizes_and_validation(L):
    """kvq_ans_sizes: 4 bytes per fixed-width word plus a per-block margin
    (table, final states, and the coder's slack); encode and decode refuse
    null pointers and short buffers on the host."""
    t = np.zeros((2, 4, 64, 128), dtype=np.float16)
    p = kvq.kvq_plan_blocks([t], 32, 128, 16)
    sb, tb = kvq.kvq_ans_sizes(p)
    margin = 128 + 4 * ((4096 + 63) // 64)
    assert sb == tb == 4 * p.max_code_words + p.n_blocks * margin
    Lb = kvq.lib()
    total = ctypes.c_uint64(0)
    assert Lb.kvq_ans_encode(ctypes.byref(p), 8, 8, 8, 8, sb, 8, tb, 8, None, ctypes.byref(total),
                             None) == kvq.KVQ_EINVAL
    assert Lb.kvq_ans_encode(ctypes.byref(p), 8, 8, 8, 8, sb - 1, 8, tb, 8, 8, ctypes.byref(total),
                             None) == kvq.KVQ_ENOSPC
    assert "kvq_ans_sizes" in kvq.last_error()
    assert Lb.kvq_ans_encode(ctypes.byref(p), 8, 8, 8, 8, sb, 8, tb, 8, 8, None, None) == kvq.KVQ_EINVAL
    assert Lb.kvq_ans_decode(ctypes.byref(p), None, 8, 8, 8, 8, 8, None) == kvq.KVQ_EINVAL
    assert Lb.kvq_ans_decode(ctypes.byref(p), 10, 8, 8, 8, 8, 8, None) == kvq.KVQ_EINVAL  # unaligned


def test_decode_attention_validation(L):
    """Shapes the attention kernel does not take are refused on the host."""
    k = np.zeros((1, 8, 256, 128), dtype=np.float16)
    p = kvq.kvq_plan_blocks([k, k], 32, 128, 16)
    assert kvq.kvq_decode_attention_workspace(p, 32) == 1 * 8 * 4 * 1 * (128 + 2) * 4
    Lb = kvq.lib()
    b = ctypes.c_uint64(0)
    # any whole number of query heads per KV head (here 3 and 8)
    assert kvq.kvq_decode_attention_workspace(p, 24) == 1 * 8 * 3 * 1 * (128 + 2) * 4
    assert kvq.kvq_decode_attention_workspace(p, 64) == 1 * 8 * 8 * 1 * (128 + 2) * 4
    assert Lb.kvq_decode_attention_workspace(ctypes.byref(p), 20, ctypes.byref(b)) == kvq.KVQ_EINVAL
    assert Lb.kvq_decode_attention_workspace(ctypes.byref(p), 0, ctypes.byref(b)) == kvq.KVQ_EINVAL
    p1 = kvq.kvq_plan_blocks([k], 32, 128, 16)
    assert Lb.kvq_decode_attention_workspace(ctypes.byref(p1), 8, ctypes.byref(b)) == kvq.KVQ_EINVAL
    p2 = kvq.kvq_plan_blocks([k, k], 16, 128, 16)
    assert Lb.kvq_decode_attention_workspace(ctypes.byref(p2), 8, ctypes.byref(b)) == kvq.KVQ_EINVAL
    assert Lb.kvq_decode_attention(ctypes.byref(p), 8, 8, 8, 8, 8, 32, ctypes.c_float(0.1), 8, 8,
                                   10, None) == kvq.KVQ_ENOSPC



def test_missing_library_fails_loudly(tmp_path):
    """Without the HIP library every call raises: there is no CPU fallback."""
    import sys
    code = ("from kv_cache_rate_amd import kvq\n"
            "try:\n"
            "    kvq.lib()\n"
            "except RuntimeError as e:\n"
            "    print('raised:', e)\n"
            "else:\n"
            "    print('loaded')\n")
    env = dict(os.environ, KVQ_LIB=str(tmp_path / "libkvq_absent.so"))
    res = subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=env, capture_output=True, text=True,
                         timeout=120)
    assert res.returncode == 0, res.stderr
    assert res.stdout.startswith("raised:") and "is missing" in res.stdout, res.stdout
