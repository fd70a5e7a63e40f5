"""Pins of the oracle's Philox4x32-10 (CPU only).

The oracle is checked against rocRAND's Philox4x32-10 engine, an
independently written implementation shipped as a C++ source header in the
ROCm image, compiled for the host here with g++.  The engine's public API
maps (seed, subsequence, offset) to key = seed, counter = (offset/4 as 64
bits, subsequence as 64 bits), which covers the counter layout used for
stochastic rounding: (t >> 2, r_lo, r_hi, 0).
"""

import os
import shutil
import subprocess
import tempfile

import numpy as np
import pytest

from oracle import philox

ROCRAND = "/opt/rocm/include/rocrand/rocrand_philox4x32_10.h"

PROG = r"""
#include <cstdio>
#include <cstdlib>
#include <rocrand/rocrand_philox4x32_10.h>
int main(int argc, char** argv) {
  // each line of stdin: seed group r  -> prints the 4 words of counter (group, r_lo, r_hi, 0)
  unsigned long long seed, group, r;
  while (scanf("%llu %llu %llu", &seed, &group, &r) == 3) {
    // counter (x, y) = group | r_lo << 32 is reached by discarding 4 * X
    // draws, in steps that keep 4 * step below 2^64
    unsigned long long X = ((r & 0xffffffffULL) << 32) | group;
    rocrand_device::philox4x32_10_engine e(seed, r >> 32, 0);
    while (X) {
      unsigned long long step = X < (1ULL << 61) ? X : (1ULL << 61);
      e.discard(4ULL * step);
      X -= step;
    }
    unsigned a = e(), b = e(), c = e(), d = e();
    printf("%u %u %u %u\n", a, b, c, d);
  }
  return 0;
}
"""


@pytest.fixture(scope="module")
def rocrand_prog():
    if not os.path.exists(ROCRAND) or shutil.which("g++") is None:
        pytest.skip("rocRAND source header or g++ not available")
    d = tempfile.mkdtemp()
    src = os.path.join(d, "p.cpp")
    exe = os.path.join(d, "p")
    open(src, "w").write(PROG)
    subprocess.check_call(["g++", "-O1", "-x", "c++", "-D__HIP_PLATFORM_AMD__",
                           "-I/opt/rocm/include", src, "-o", exe])
    return exe


def test_matches_rocrand(rocrand_prog, rng):
    cases = [(0, 0, 0), (0, 1, 0), (0, 0, 1), (2**64 - 1, 2**32 - 1, 2**64 - 1),
             (0x0123456789ABCDEF, 3, (7 << 32) | 5)]
    for _ in range(200):
        cases.append((int(rng.integers(0, 2**63)) * 2 + int(rng.integers(0, 2)),
                      int(rng.integers(0, 2**32)), int(rng.integers(0, 2**63))))
    inp = "".join(f"{s} {g} {r}\n" for s, g, r in cases)
    out = subprocess.run([rocrand_prog], input=inp, capture_output=True, text=True, check=True).stdout
    want = np.array([[int(v) for v in line.split()] for line in out.strip().splitlines()], dtype=np.uint64)
    ctr = np.array([[g, r & 0xFFFFFFFF, r >> 32, 0] for s, g, r in cases], dtype=np.uint64)
    key = np.array([[s & 0xFFFFFFFF, s >> 32] for s, g, r in cases], dtype=np.uint64)
    got = philox.philox4x32_10(ctr, key)
    assert np.array_equal(got.astype(np.uint64), want)


def test_block_words_layout(rocrand_prog):
    """Entry t of block r uses word t & 3 of counter (t >> 2, r_lo, r_hi, 0)."""
    r = (3 << 32) | 77
    w = philox.block_words(5, r, 13)
    inp = "".join(f"5 {g} {r}\n" for g in range(4))
    out = subprocess.run([rocrand_prog], input=inp, capture_output=True, text=True, check=True).stdout
    want = np.array([int(v) for line in out.split("\n") if line for v in line.split()], dtype=np.uint32)
    assert np.array_equal(w, want[:13])


def test_uniform_24bit_distribution():
    """Chi-square of the 24-bit uniforms over 64 equal bins."""
    u = np.concatenate([philox.block_uniforms(0, r, 4096) for r in range(64)])
    assert u.min() >= 0.0 and u.max() < 1.0
    assert np.all(u * 2**24 == np.floor(u * 2**24))
    counts = np.bincount((u * 64).astype(int), minlength=64)
    exp = u.size / 64
    chi2 = np.sum((counts - exp) ** 2 / exp)
    assert chi2 < 120  # 63 dof: mean 63, p(chi2 > 120) ~ 2e-5
    # a different seed gives different draws
    assert not np.array_equal(philox.block_words(0, 0, 64), philox.block_words(1, 0, 64))
