"""Pins of the rANS entropy coder of the oracle (oracle/ans.py).

* a block coded by hand (tests/golden/ans_example.txt);
* decode(encode(codes)) == codes, and every state returns to 2^16, over
  random blocks of many sizes, alphabets and skews;
* the coded length stays within a fixed overhead of the ideal length
  sum_t log2(M / f_{s_t}) of the block's symbols under its own model, and
  that ideal length equals n times the empirical entropy when n = M;
* the model: frequencies sum to 2^k, every present symbol is coded with
  f >= 1, and a one-symbol block codes to the table and the start states.
"""

import math

import numpy as np
import pytest

from oracle import ans


def _golden():
    path = __file__.replace("test_oracle_ans.py", "golden/ans_example.txt")
    env = {}
    for line in open(path):
        line = line.strip()
        if line and not line.startswith("#"):
            k, v = line.split("=", 1)
            env[k.strip()] = eval(v, {})  # literals only
    return env


def test_hand_worked_block():
    g = _golden()
    b = ans.encode_block(g["codes"], g["m"])
    assert b.view("<u2").tolist() == g["words"]
    assert np.array_equal(ans.decode_block(b, g["m"], len(g["codes"])), g["codes"])


@pytest.mark.parametrize("n", [2, 3, 7, 8, 9, 45, 96, 100, 512, 4096])
def test_round_trip_and_length(rng, n):
    for trial in range(6):
        m = int(rng.integers(1, 17))
        p = rng.dirichlet(np.full(m, 0.4))
        codes = rng.choice(m, size=n, p=p)
        b = ans.encode_block(codes, m)
        assert b.size % 4 == 0
        assert np.array_equal(ans.decode_block(b, m, n), codes)
        # table (16 m bits) + ideal bits + at most 32 bits per state + padding
        extra = 8 * b.size - 16 * m - ans.model_bits(codes, m)
        assert -1e-6 <= extra <= 32 * ans.LANES + 16, (n, m, extra)


def test_ideal_length_is_empirical_entropy_at_power_of_two():
    rng = np.random.default_rng(7)
    codes = rng.choice(5, size=4096, p=[0.5, 0.2, 0.15, 0.1, 0.05])
    cnt = np.bincount(codes, minlength=5)
    h = -sum(c / 4096 * math.log2(c / 4096) for c in cnt if c)
    assert ans.model_bits(codes, 5) == pytest.approx(4096 * h, rel=1e-12)


def test_model_frequencies():
    codes = np.array([3, 3, 0, 3, 1, 3, 3])  # n = 7, k = 3, M = 8
    f, k = ans.frequencies(codes, 5)
    assert k == 3 and f.tolist() == [1, 1, 0, 5 + 1, 0]
    assert ans.frequencies(np.array([0, 1]), 2)[0].tolist() == [1, 1]


def test_single_symbol_block():
    b = ans.encode_block(np.zeros(4096, dtype=np.int64), 1)
    w = b.view("<u2").tolist()
    # table (4096) then eight untouched start states (1, 0) and one pad word
    assert w == [4096] + [1, 0] * ans.LANES + [0]
    assert np.array_equal(ans.decode_block(b, 1, 4096), np.zeros(4096))


def test_skewed_block_codes_near_its_entropy():
    rng = np.random.default_rng(3)
    codes = rng.choice(16, size=4096, p=np.r_[0.7, np.full(15, 0.02)])
    b = ans.encode_block(codes, 16)
    cnt = np.bincount(codes, minlength=16)
    h = -sum(c / 4096 * math.log2(c / 4096) for c in cnt if c)  # about 2.08 bits
    # within 0.15 bit of the empirical entropy, about half of fixed-width 4 bits
    assert h <= 8 * b.size / 4096 < h + 0.15
    assert np.array_equal(ans.decode_block(b, 16, 4096), codes)
