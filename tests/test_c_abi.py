"""The boundary from plain C: a C11 program that includes only
include/kvq.h, links libkvq.so and plans the long-context cache (host-only
calls, so no GPU is needed) compiles without warnings and gets the
workload's plan (524288 blocks, 29 candidates, 73 order statistics); a bad
block spec returns KVQ_EINVAL with its status string."""

import os
import shutil
import subprocess

import pytest

from kv_cache_rate_amd import kvq

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

PROGRAM = r"""
#include <stdio.h>
#include <string.h>
#include "kvq.h"

int main(void) {
    kvq_tensor t[2];
    memset(t, 0, sizeof t);
    for (int i = 0; i < 2; ++i) {  /* K and V, [32, 8, 32768, 128] fp16, contiguous */
        const int64_t shape[4] = {32, 8, 32768, 128};
        t[i].data = (const void*)(uintptr_t)(0x100000u * (unsigned)(i + 1));  /* never dereferenced */
        t[i].dtype = KVQ_F16;
        memcpy(t[i].shape, shape, sizeof shape);
        t[i].stride[3] = 1;
        t[i].stride[2] = 128;
        t[i].stride[1] = 128LL * 32768;
        t[i].stride[0] = 128LL * 32768 * 8;
    }
    kvq_block_spec spec = {32, 128, 16, KVQ_GRIDS, 0, 0};
    kvq_plan p;
    kvq_status st = kvq_plan_blocks(t, 2, &spec, &p);
    printf("%d %lld %lld %d %d %llu %llu\n", (int)st, (long long)p.n_blocks, (long long)p.n_entries,
           p.n_cand, p.n_stats, (unsigned long long)p.max_code_words, (unsigned long long)p.workspace_bytes);
    spec.s = 1;
    st = kvq_plan_blocks(t, 2, &spec, &p);
    printf("%d %s\n", (int)st, kvq_status_string(st));
    return 0;
}
"""


def test_plain_c_program_plans_the_long_context_cache(tmp_path):
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("no C compiler")
    if not os.path.exists(kvq.LIB_PATH):
        pytest.fail("libkvq.so is not built (run python -m kv_cache_rate_amd.build)")
    src = tmp_path / "plan.c"
    src.write_text(PROGRAM)
    exe = tmp_path / "plan"
    libdir = os.path.dirname(kvq.LIB_PATH)
    cmd = [gcc, "-std=c11", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROOT, "include"), "-I", "/opt/rocm/include", str(src),
           "-L", libdir, "-lkvq", f"-Wl,-rpath,{libdir}", "-o", str(exe)]
    res = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
    assert res.returncode == 0, res.stderr
    out = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert out.returncode == 0, out.stderr
    lines = out.stdout.split("\n")
    st, R, n, C, S, words, ws = (int(v) for v in lines[0].split())
    assert (st, R, n, C, S) == (0, 524288, 2 ** 31, 29, 73)
    assert words == 2 ** 31 * 4 // 32 and ws > 0
    assert lines[1].split()[0] == str(kvq.KVQ_EINVAL)
    assert "KVQ_EINVAL" in lines[1]
