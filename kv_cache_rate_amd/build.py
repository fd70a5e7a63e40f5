"""Build libkvq.so (HIP for gfx950) in-tree.

    python -m kv_cache_rate_amd.build [--jobs N]

Every source under ``csrc/`` is compiled with hipcc for gfx950 and linked into
``kv_cache_rate_amd/libkvq.so``.  Packed-fp32 instructions are disabled
(``-Xclang -target-feature -Xclang -packed-fp32-ops``).
"""

import argparse
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libkvq.so")
ARCH = "gfx950"

SOURCES = ["kvq_host.cpp", "kvq_eval.hip", "kvq_eval16.hip", "kvq_solve.hip", "kvq_quant.hip",
           "kvq_ans.hip", "kvq_attn.hip"]

COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-Wno-unused-command-line-argument", "-I", INCLUDE, "-I", CSRC]


def hipcc():
    exe = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(exe):
        raise RuntimeError("hipcc not found; the HIP library cannot be built")
    return exe


def compile_one(src):
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc()] + COMMON + ["-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{res.stderr}")
    return obj, res.stderr


def build(jobs=None, verbose=False):
    """Compile every source and link ``libkvq.so``; returns its path."""
    os.makedirs(BUILD, exist_ok=True)
    jobs = jobs or min(len(SOURCES), os.cpu_count() or 1)
    with ThreadPoolExecutor(jobs) as ex:
        results = list(ex.map(compile_one, SOURCES))
    if verbose:
        for _, err in results:
            if err.strip():
                print(err, file=sys.stderr)
    tmp = LIB + ".tmp"
    cmd = [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp] + [o for o, _ in results]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stderr}")
    os.replace(tmp, LIB)
    return LIB


SANITIZED_LIB = os.path.join(BUILD, "asan", "libkvq_asan.so")


def build_host_sanitized():
    """Build of the library with AddressSanitizer and
    UndefinedBehaviorSanitizer on the host code only (argument validation,
    planning, launch sequencing; device code is built as usual, without
    them).  For the CPU validation tests; returns its path."""
    out = os.path.dirname(SANITIZED_LIB)
    os.makedirs(out, exist_ok=True)
    objs = []
    for src in SOURCES:
        obj = os.path.join(out, os.path.splitext(src)[0] + ".o")
        cmd = [hipcc(), "-O1", "-g", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
               "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
               "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-fno-sanitize-recover=undefined",
               "-Wno-unused-command-line-argument", "-I", INCLUDE, "-I", CSRC,
               "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
        objs.append((obj, cmd))

    def run(job):
        obj, cmd = job
        res = subprocess.run(cmd, capture_output=True, text=True)
        if res.returncode != 0:
            raise RuntimeError(f"sanitized build failed on {obj}:\n{res.stderr}")
        return obj
    with ThreadPoolExecutor(min(len(objs), os.cpu_count() or 1)) as ex:
        objs = list(ex.map(run, objs))
    cmd = [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", "-shared-libsan",
           "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-o", SANITIZED_LIB] + objs
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"sanitized link failed:\n{res.stderr}")
    return SANITIZED_LIB


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=None)
    ap.add_argument("-v", "--verbose", action="store_true")
    a = ap.parse_args()
    print(build(a.jobs, a.verbose))


if __name__ == "__main__":
    main()
