"""Pins for the oracle's lightning-indexer score and top-k selection.

- one indexer head with weight 1 gives ReLU(q.k) (numpy matmul + maximum);
- a one-hot head weight isolates that head (catches transposed / mis-indexed heads);
- the score is linear in the head weights;
- MXFP4 per-head dot products are exact: checked against Python's exact
  rational arithmetic (fractions) on decoded values;
- top-k equals a brute-force full sort by (score desc, index asc) (numpy lexsort);
- k >= n_elig selects everything, padded with -1; equal keys prefer the lower
  index; scaling all head weights by a positive constant keeps the set.
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle


def rnd(seed, *shape):
    return np.random.default_rng(seed).standard_normal(shape).astype(np.float32)


def brute_topk(s, k):
    order = np.lexsort((np.arange(len(s)), -s))
    sel = np.sort(order[:k])
    return np.concatenate([sel, -np.ones(k - len(sel), np.int64)])


def scores_f32(qi, w, keys, n):
    B, Tq, H, d = qi.shape
    idx, sc, alls = oracle.index_topk(qi.astype(np.float64), w, keys, oracle.F32, None,
                                      np.full((B, Tq), n, np.int32), 1, want_scores=True)
    return alls[..., :n]


def test_single_head_is_relu_dot():
    q = rnd(1, 1, 1, 1, 64)
    keys = rnd(2, 1, 300, 64)
    s = scores_f32(q, np.ones((1, 1, 1), np.float32), keys, 300)[0, 0]
    ref = np.maximum(keys[0].astype(np.float64) @ q[0, 0, 0].astype(np.float64), 0)
    np.testing.assert_allclose(s, ref, rtol=1e-13, atol=1e-13)
    assert (s == 0).sum() > 50          # the ReLU is active on about half the entries


def test_one_hot_weights_isolate_heads():
    H = 4
    q = rnd(3, 1, 1, H, 64)
    keys = rnd(4, 1, 200, 64)
    for h in range(H):
        w = np.zeros((1, 1, H), np.float32)
        w[0, 0, h] = 1.0
        s = scores_f32(q, w, keys, 200)[0, 0]
        ref = np.maximum(keys[0].astype(np.float64) @ q[0, 0, h].astype(np.float64), 0)
        np.testing.assert_allclose(s, ref, rtol=1e-13, atol=1e-13)


def test_linear_in_head_weights():
    H = 8
    q = rnd(5, 1, 1, H, 128)
    keys = rnd(6, 1, 150, 128)
    g = np.random.default_rng(7)
    w1 = g.random((1, 1, H), dtype=np.float32)
    w2 = g.random((1, 1, H), dtype=np.float32)
    s1 = scores_f32(q, w1, keys, 150)
    s2 = scores_f32(q, w2, keys, 150)
    s12 = scores_f32(q, (w1 + w2).astype(np.float32), keys, 150)
    # w1 + w2 is rounded to fp32; compare against the exact-weight sum with slack
    np.testing.assert_allclose(s12, s1 + s2, rtol=1e-6, atol=1e-9)
    s3 = scores_f32(q, (w1 * 4).astype(np.float32), keys, 150)
    np.testing.assert_allclose(s3, 4 * s1, rtol=1e-15, atol=0)


def test_mxfp4_dots_are_exact():
    g = np.random.default_rng(8)
    qv = (g.standard_normal((1, 1, 2, 128)) * 2).astype(np.float32)
    kv = (g.standard_normal((1, 64, 128)) * 0.5).astype(np.float32)
    qc, qs = oracle.encode(qv, oracle.MXFP4)
    kc, ks = oracle.encode(kv, oracle.MXFP4)
    qd = oracle.decode(qc, oracle.MXFP4, qs)
    kd = oracle.decode(kc, oracle.MXFP4, ks)
    w = np.array([[[1.0, 0.0]]], np.float32)
    _, _, alls = oracle.index_topk(qd, w, kc, oracle.MXFP4, ks, np.array([[64]], np.int32), 4,
                                   want_scores=True)
    for j in range(64):
        exact = sum(Fraction(float(a)) * Fraction(float(b)) for a, b in zip(qd[0, 0, 0], kd[0, j]))
        exact = max(exact, Fraction(0))
        assert Fraction(alls[0, 0, j]) == exact


@pytest.mark.parametrize("n,k", [(1000, 64), (257, 256), (100, 100), (50, 64), (1, 8), (0, 4)])
def test_topk_matches_brute_force_sort(n, k):
    H = 4
    q = rnd(9, 1, 1, H, 64)
    keys = rnd(10, 1, max(n, 1), 64)
    w = np.random.default_rng(11).random((1, 1, H), dtype=np.float32)
    idx, sc, alls = oracle.index_topk(q.astype(np.float64), w, keys, oracle.F32, None,
                                      np.array([[n]], np.int32), k, want_scores=True)
    s = alls[0, 0, :n]
    assert np.array_equal(idx[0, 0], brute_topk(s, k))
    valid = idx[0, 0] >= 0
    assert np.array_equal(sc[0, 0][valid], s[idx[0, 0][valid]])


def test_k_at_least_n_selects_all_and_pads():
    idx, _ = oracle.select_topk(np.array([3.0, 1.0, 2.0]), 5)
    assert list(idx) == [0, 1, 2, -1, -1]


def test_ties_prefer_lower_index():
    s = np.array([1.0, 5.0, 3.0, 5.0, 5.0, 0.0, 3.0])
    idx, _ = oracle.select_topk(s, 2)
    assert list(idx) == [1, 3]
    idx, _ = oracle.select_topk(s, 4)
    assert list(idx) == [1, 2, 3, 4]
    # duplicated keys in the cache produce equal scores
    keys = rnd(12, 1, 10, 64)
    keys[0, 7] = keys[0, 2]
    q = rnd(13, 1, 1, 1, 64)
    q[0, 0, 0] = keys[0, 2] * 10            # entries 2 and 7 score highest, equally
    idx, _ = oracle.index_topk(q.astype(np.float64), np.ones((1, 1, 1), np.float32), keys,
                               oracle.F32, None, np.array([[10]], np.int32), 1)
    assert list(idx[0, 0]) == [2]


def test_positive_weight_scale_keeps_selection():
    H = 8
    q = rnd(14, 1, 1, H, 128)
    keys = rnd(15, 1, 500, 128)
    w = np.random.default_rng(16).random((1, 1, H), dtype=np.float32)
    n = np.array([[500]], np.int32)
    a, _ = oracle.index_topk(q.astype(np.float64), w, keys, oracle.F32, None, n, 37)
    b, _ = oracle.index_topk(q.astype(np.float64), (w * 8).astype(np.float32), keys, oracle.F32,
                             None, n, 37)
    assert np.array_equal(a, b)


def test_rows_use_their_own_sequence_and_n_elig():
    B, Tq, H, d, N = 2, 3, 2, 64, 40
    q = rnd(17, B, Tq, H, d)
    keys = rnd(18, B, N, d)
    w = np.random.default_rng(19).random((B, Tq, H), dtype=np.float32)
    n = np.array([[40, 10, 3], [25, 0, 40]], np.int32)
    idx, _ = oracle.index_topk(q.astype(np.float64), w, keys, oracle.F32, None, n, 6)
    for b in range(B):
        for t in range(Tq):
            s = np.array([oracle.index_score(q[b, t], w[b, t], keys[b, j]) for j in range(n[b, t])])
            assert np.array_equal(idx[b, t], brute_topk(s, 6))
