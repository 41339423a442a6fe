"""Pins for the oracle's compression (softmax-gated pooling with positional bias).

Closed forms and library routines on special cases: m = 1 is the identity for
any gate; zero gates and bias give the block mean (numpy mean); m = 2 gives a
logistic mix (scipy expit); general m equals scipy's softmax weights applied
to the block; a dominant bias picks one token; shifting all gates of a block
changes nothing; entry counts follow non-overlapping blocks (golden fixture
restating the 10100.com article's 1M -> 250K / ~8000 figures).
"""
import os

import numpy as np
import pytest
from scipy.special import expit, softmax

import oracle

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def rnd(seed, *shape):
    return np.random.default_rng(seed).standard_normal(shape)


def test_m1_is_identity_for_any_gate():
    x = rnd(1, 37, 128)
    out = oracle.pool(x, rnd(2, 37) * 5, rnd(3, 1), 1)
    assert np.array_equal(out, x)


def test_zero_gate_gives_block_mean():
    for m in (4, 128):
        x = rnd(4, 3 * m + 1, 64)
        out = oracle.pool(x, np.zeros(len(x)), np.zeros(m), m)
        ref = x[: 3 * m].reshape(3, m, 64).mean(axis=1)
        np.testing.assert_allclose(out, ref, rtol=1e-13, atol=1e-15)


def test_m2_is_logistic_mix():
    x = rnd(5, 40, 32)
    g = rnd(6, 40) * 3
    b = np.array([0.3, -0.2])
    out = oracle.pool(x, g, b, 2)
    a = g.reshape(20, 2) + b
    w0 = expit(a[:, 0] - a[:, 1])[:, None]
    ref = w0 * x[0::2] + (1 - w0) * x[1::2]
    np.testing.assert_allclose(out, ref, rtol=1e-13, atol=1e-15)


@pytest.mark.parametrize("m", [3, 4, 128])
def test_general_m_matches_scipy_softmax_weights(m):
    n = 5
    x = rnd(7, n * m, 128)
    g = rnd(8, n * m) * 2
    b = rnd(9, m) * 0.1
    out = oracle.pool(x, g, b, m)
    for j in range(n):
        w = softmax(g[j * m:(j + 1) * m] + b)
        np.testing.assert_allclose(out[j], w @ x[j * m:(j + 1) * m], rtol=1e-12, atol=1e-14)


def test_dominant_bias_selects_token():
    m = 4
    x = rnd(10, 16, 64)
    b = np.zeros(m)
    b[2] = 60.0
    out = oracle.pool(x, np.zeros(16), b, m)
    np.testing.assert_allclose(out, x[2::4], rtol=0, atol=1e-20)


def test_gate_shift_invariance_and_weights_sum_to_one():
    m = 4
    x = rnd(11, 64, 16)
    g = rnd(12, 64)
    b = rnd(13, m) * 0.1
    base = oracle.pool(x, g, b, m)
    shifted = oracle.pool(x, g + np.repeat(rnd(14, 16) * 50, m), b, m)
    np.testing.assert_allclose(shifted, base, rtol=1e-12, atol=1e-13)
    ones = oracle.pool(np.ones((64, 16)), g, b, m)
    np.testing.assert_allclose(ones, 1.0, rtol=0, atol=4e-16)


def test_tail_block_not_pooled():
    out = oracle.pool(rnd(15, 10, 8), rnd(16, 10), np.zeros(4), 4)
    assert out.shape == (2, 8)


def test_entry_counts_golden():
    rows = [l.split() for l in open(os.path.join(GOLD, "entry_counts.txt")) if l[0] != "#"]
    assert len(rows) >= 9
    for tokens, m, entries, _src in rows:
        T, m = int(tokens), int(m)
        out = oracle.pool(np.zeros((T, 1)), np.zeros(T), np.zeros(m), m)
        assert out.shape[0] == int(entries)
