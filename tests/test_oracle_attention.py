"""Pins of the decode-attention oracle (oracle/attention.py): closed forms of
softmax attention that a slip in the max shift, the normalisation, the scale
or the grouped-head mapping would break."""

import numpy as np
import pytest

from oracle import attention


def test_uniform_keys_average_the_values(rng):
    """Equal scores make the output the mean of the values."""
    K = np.zeros((1, 2, 7, 4))
    V = rng.standard_normal((1, 2, 7, 4))
    q = rng.standard_normal((1, 2, 4))
    o = attention.decode_attention(K, V, q, 0.5)
    assert np.allclose(o[0, 0], V[0, 0].mean(axis=0), rtol=0, atol=1e-15)
    assert np.allclose(o[0, 1], V[0, 1].mean(axis=0), rtol=0, atol=1e-15)


def test_two_tokens_closed_form():
    """Two tokens: weight of token 1 is the logistic of the score gap."""
    K = np.array([[[[1.0, 0.0], [0.0, 2.0]]]])
    V = np.array([[[[3.0, -1.0], [5.0, 7.0]]]])
    q = np.array([[[0.4, 0.9]]])
    scale = 0.7
    s0, s1 = scale * 0.4, scale * 1.8
    p1 = 1.0 / (1.0 + np.exp(s0 - s1))
    want = (1 - p1) * V[0, 0, 0] + p1 * V[0, 0, 1]
    assert np.allclose(attention.decode_attention(K, V, q, scale)[0, 0], want, rtol=1e-15)


def test_large_scores_select_the_best_token_and_shift_invariance(rng):
    K = rng.standard_normal((1, 1, 9, 8))
    V = rng.standard_normal((1, 1, 9, 8))
    q = rng.standard_normal((1, 1, 8))
    o = attention.decode_attention(K, V, q, 1e4)  # no overflow: the max is shifted out
    best = int(np.argmax(K[0, 0] @ q[0, 0]))
    assert np.allclose(o[0, 0], V[0, 0, best], atol=1e-12)
    # adding a constant to every score (a key component along q) changes nothing
    shift = np.outer(np.ones(9), q[0, 0]) / (q[0, 0] @ q[0, 0])
    o1 = attention.decode_attention(K, V, q, 0.3)
    o2 = attention.decode_attention(K + 2.5 * shift[None, None], V, q, 0.3)
    assert np.allclose(o1, o2, rtol=1e-12, atol=1e-12)


def test_grouped_query_heads_read_their_kv_head(rng):
    """With 4 query heads per KV head, query head g uses KV head g // 4."""
    K = rng.standard_normal((2, 2, 5, 4))
    V = rng.standard_normal((2, 2, 5, 4))
    q = rng.standard_normal((2, 8, 4))
    o = attention.decode_attention(K, V, q, 0.5)
    for g in range(8):
        one = attention.decode_attention(K[:, g // 4:g // 4 + 1], V[:, g // 4:g // 4 + 1],
                                         q[:, g:g + 1], 0.5)
        assert np.array_equal(o[:, g], one[:, 0])
