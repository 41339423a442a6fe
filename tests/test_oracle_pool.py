"""Pins for the oracle's compression (softmax-gated pooling with positional bias).

Closed forms and library routines on special cases: m = 1 is the identity for
any gate; zero gates and bias give the block mean (numpy mean); m = 2 gives a
logistic mix (scipy expit); general m equals scipy's softmax weights applied
to the block; a dominant bias picks one token; shifting all gates of a block
changes nothing; entry counts follow non-overlapping blocks (golden fixture
restating the 10100.com article's 1M -> 250K / ~8000 figures).

Pooling variants (per-channel gates, overlapping blocks): without overlap and
with one logit per token they equal the pinned pooling; per channel they are
scipy's softmax per channel over the existing positions; zero gates give the
numpy mean of the existing positions; a dominant bias row picks the token at
that row's position (which fixes the bias indexing of overlapped blocks);
equal gate columns reduce to one logit per token; a dominant per-channel gate
picks a token per channel; a per-channel shift of all gates changes nothing.
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


# --------------------------------------------------------------------------
# pooling variants: per-channel gates, overlapping blocks
# --------------------------------------------------------------------------
@pytest.mark.parametrize("m", [1, 4, 128])
def test_variant_without_overlap_per_token_is_pool(m):
    x, g, b = rnd(20, 6 * m + 3, 64), rnd(21, 6 * m + 3) * 2, rnd(22, m) * 0.1
    np.testing.assert_array_equal(oracle.pool_variant(x, g, b, m), oracle.pool(x, g, b, m))


@pytest.mark.parametrize("m,o", [(4, 0), (4, 2), (4, 4), (128, 64)])
def test_variant_per_channel_scipy_softmax_per_channel(m, o):
    """Every channel's weights are scipy's softmax over the block's existing
    positions (the first block has no predecessor)."""
    T, D = 5 * m + 1, 16
    x, g, b = rnd(23, T, D), rnd(24, T, D) * 2, rnd(25, m + o, D) * 0.3
    out = oracle.pool_variant(x, g, b, m, o)
    assert out.shape == (5, D)
    for j in range(5):
        t0 = j * m - o
        lo = max(t0, 0)
        for d in range(D):
            w = softmax(g[lo:j * m + m, d] + b[lo - t0:, d])
            np.testing.assert_allclose(out[j, d], w @ x[lo:j * m + m, d], rtol=1e-12, atol=1e-14)


@pytest.mark.parametrize("m,o", [(4, 1), (4, 4), (128, 32)])
def test_overlap_zero_gates_give_mean_of_existing_positions(m, o):
    x = rnd(26, 4 * m, 32)
    out = oracle.pool_variant(x, np.zeros(4 * m), np.zeros(m + o), m, o)
    np.testing.assert_allclose(out[0], x[:m].mean(0), rtol=1e-13, atol=1e-15)
    for j in range(1, 4):
        np.testing.assert_allclose(out[j], x[j * m - o:(j + 1) * m].mean(0), rtol=1e-13, atol=1e-15)


def test_overlap_bias_rows_follow_positions():
    """A dominant bias on row 0 (the oldest overlapped position) picks token
    j*m - o in every block that has it; the first block, which has no
    overlapped positions, averages its own tokens (rows o.. carry no bias)."""
    m, o = 4, 3
    x = rnd(27, 5 * m, 8)
    b = np.zeros(m + o)
    b[0] = 800.0
    out = oracle.pool_variant(x, np.zeros(5 * m), b, m, o)
    np.testing.assert_allclose(out[0], x[:m].mean(0), rtol=1e-13)
    for j in range(1, 5):
        np.testing.assert_allclose(out[j], x[j * m - o], rtol=1e-12)
    b = np.zeros(m + o)
    b[o + m - 1] = 800.0                                 # the newest token of the block
    out = oracle.pool_variant(x, np.zeros(5 * m), b, m, o)
    for j in range(5):
        np.testing.assert_allclose(out[j], x[j * m + m - 1], rtol=1e-12)


def test_per_channel_equal_columns_is_per_token():
    m, o, T, D = 4, 2, 24, 8
    x, g, b = rnd(28, T, D), rnd(29, T) * 2, rnd(30, m + o) * 0.2
    ref = oracle.pool_variant(x, g, b, m, o)
    got = oracle.pool_variant(x, np.repeat(g[:, None], D, 1), np.repeat(b[:, None], D, 1), m, o)
    np.testing.assert_allclose(got, ref, rtol=1e-14, atol=1e-15)


def test_per_channel_gate_picks_a_token_per_channel_and_shift_invariance():
    m, T, D = 4, 16, 4
    x = rnd(31, T, D)
    g = np.zeros((T, D))
    for d in range(D):                    # channel d: token (d + 1) % m of every block dominates
        g[(d + 1) % m::m, d] = 900.0
    out = oracle.pool_variant(x, g, np.zeros((m, D)), m)
    for j in range(T // m):
        for d in range(D):
            np.testing.assert_allclose(out[j, d], x[j * m + (d + 1) % m, d], rtol=1e-12)
    g2 = rnd(32, T, D)
    shift = rnd(33, D) * 5                # the same constant on every token of a channel
    a = oracle.pool_variant(x, g2, np.zeros((m, D)), m)
    bb = oracle.pool_variant(x, g2 + shift, np.zeros((m, D)), m)
    np.testing.assert_allclose(a, bb, rtol=1e-12, atol=1e-14)
