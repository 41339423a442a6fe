"""Pins for the oracle's attention over (selected entries U window U sink).

- with the sink at -inf the result is textbook softmax(tau q K^T) V, checked
  against torch's scaled_dot_product_attention in float64 (a library routine);
- a finite sink equals SDPA with one extra zero key/value column whose additive
  mask is the sink logit (the reading: the sink adds to the denominator only);
- sink -> +inf sends the output to 0 and the LSE to the sink logit;
- weights including the sink sum to 1 (V = ones gives 1 - p_sink);
- permuting the attended set, or splitting it and merging by LSE, changes nothing;
- top-k = all entries makes sparse attention equal dense attention (the HCA path);
- k = 0 with a window covering the whole context is full causal attention.

Separate values (the variant with K != V): torch SDPA with different key and
value tensors (sink as an extra zero-value column); values equal to the keys
give the shared-KV result bit for bit; the output is linear in the values
(exactly, on values whose fp32 sums are exact) and the LSE does not depend on
them.
"""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle


def rnd(seed, *shape):
    return np.random.default_rng(seed).standard_normal(shape)


def textbook(q, kv, tau, sink=None):
    """q [H, D], kv [n, D]; optional sink column via an additive float mask."""
    H, D = q.shape
    qt = torch.from_numpy(q).reshape(1, H, 1, D)
    k = torch.from_numpy(kv)
    mask = torch.zeros(1, H, 1, k.shape[0], dtype=torch.float64)
    if sink is not None:
        k = torch.cat([k, torch.zeros(1, D, dtype=torch.float64)])
        mask = torch.cat([mask, torch.from_numpy(sink.astype(np.float64)).reshape(1, H, 1, 1)], -1)
    kt = k.reshape(1, 1, -1, D).expand(1, H, -1, D).contiguous()
    o = F.scaled_dot_product_attention(qt, kt, kt, attn_mask=mask, scale=tau)
    scores = (qt @ kt.transpose(-1, -2)) * tau + mask
    lse = torch.logsumexp(scores, -1)
    return o.reshape(H, D).numpy(), lse.reshape(H).numpy()


def test_no_sink_is_textbook_softmax():
    q = rnd(1, 16, 128)
    ent = rnd(2, 30, 128)
    win = rnd(3, 20, 128)
    tau = 1 / math.sqrt(128)
    o, lse = oracle.attend_row(q, ent, win, np.full(16, -np.inf, np.float32), tau)
    ref, rlse = textbook(q, np.concatenate([ent, win]), tau)
    np.testing.assert_allclose(o, ref, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(lse, rlse, rtol=1e-13, atol=1e-13)


def test_sink_is_extra_zero_value_column():
    q = rnd(4, 8, 64)
    ent = rnd(5, 12, 64)
    win = rnd(6, 5, 64)
    sink = rnd(7, 8).astype(np.float32) * 2
    o, lse = oracle.attend_row(q, ent, win, sink, 0.3)
    ref, rlse = textbook(q, np.concatenate([ent, win]), 0.3, sink)
    np.testing.assert_allclose(o, ref, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(lse, rlse, rtol=1e-13, atol=1e-13)


def test_large_sink_sends_output_to_zero():
    q = rnd(8, 4, 32)
    ent = rnd(9, 10, 32)
    sink = np.full(4, 1e4, np.float32)
    o, lse = oracle.attend_row(q, ent, np.zeros((0, 32)), sink, 0.2)
    assert np.abs(o).max() < 1e-300
    np.testing.assert_allclose(lse, 1e4, rtol=1e-15)


def test_weights_sum_to_one_with_sink():
    q = rnd(10, 8, 16)
    ones = np.ones((25, 16))
    sink = rnd(11, 8).astype(np.float32)
    o, lse = oracle.attend_row(q, ones[:15], ones[15:], sink, 1.0)
    p_sink = np.exp(sink.astype(np.float64) - lse)
    np.testing.assert_allclose(o + p_sink[:, None], 1.0, rtol=0, atol=1e-14)
    assert (p_sink > 0).all() and (o < 1).all()


def test_permutation_and_split_merge():
    q = rnd(13, 8, 64)
    ent = rnd(14, 40, 64)
    sink = rnd(15, 8).astype(np.float32)
    o, lse = oracle.attend_row(q, ent, np.zeros((0, 64)), sink, 0.125)
    perm = np.random.default_rng(16).permutation(40)
    o2, lse2 = oracle.attend_row(q, ent[perm], np.zeros((0, 64)), sink, 0.125)
    np.testing.assert_allclose(o2, o, rtol=1e-13, atol=1e-14)
    # split into two parts, the sink in the first only, merge by LSE
    oa, la = oracle.attend_row(q, ent[:17], np.zeros((0, 64)), sink, 0.125)
    ob, lb = oracle.attend_row(q, ent[17:], np.zeros((0, 64)), np.full(8, -np.inf, np.float32), 0.125)
    M = np.maximum(la, lb)
    wa, wb = np.exp(la - M), np.exp(lb - M)
    om = (wa[:, None] * oa + wb[:, None] * ob) / (wa + wb)[:, None]
    np.testing.assert_allclose(om, o, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(M + np.log(wa + wb), lse, rtol=1e-14)


def test_topk_all_equals_dense_hca_path():
    B, N, D, Hq = 2, 24, 128, 16
    g = np.random.default_rng(17)
    kv = g.standard_normal((B, N, D)).astype(np.float32)
    codes, sc = oracle.encode(kv, oracle.FP8E4M3)
    win = g.standard_normal((B, 8, D)).astype(np.float32)
    q = g.standard_normal((B, 1, Hq, D))
    sink = g.standard_normal(Hq).astype(np.float32)
    n = np.array([[24], [17]], np.int32)
    sel = np.full((B, 1, N), -1, np.int32)
    sel[0, 0, :24] = np.arange(24)
    sel[1, 0, :17] = np.arange(17)
    wb = np.zeros((B, 1), np.int32)
    wl = np.full((B, 1), 8, np.int32)
    o1, l1 = oracle.attend(q, codes, oracle.FP8E4M3, sc, sel, None, win, oracle.F32, wb, wl, sink, 0.09)
    o2, l2 = oracle.attend(q, codes, oracle.FP8E4M3, sc, None, n, win, oracle.F32, wb, wl, sink, 0.09)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(l1, l2)


def test_window_covering_context_is_full_causal_attention():
    # k = 0: only the window branch and the sink; W >= L gives causal attention
    L, D, Hq = 20, 32, 4
    x = rnd(18, L, D)
    xs = x.astype(np.float32)
    sink = rnd(19, Hq).astype(np.float32)
    qall = rnd(20, L, Hq, D)
    for p in (0, 7, L - 1):
        wb = np.array([[0]], np.int32)
        wl = np.array([[p + 1]], np.int32)
        o, lse = oracle.attend(qall[p][None, None], np.zeros((1, 1, D), np.float32), oracle.F32, None,
                               np.full((1, 1, 1), -1, np.int32), None, xs[None], oracle.F32, wb, wl,
                               sink, 0.5)
        # textbook causal attention of row p over all L tokens, sink as extra column
        H = Hq
        qt = torch.from_numpy(qall).permute(1, 0, 2)[None]          # [1,H,L,D]
        kt = torch.from_numpy(xs.astype(np.float64)).expand(1, H, L, D).contiguous()
        causal = torch.full((L, L), -math.inf, dtype=torch.float64).triu(1)
        mask = causal.expand(1, H, L, L)
        kz = torch.cat([kt, torch.zeros(1, H, 1, D, dtype=torch.float64)], 2)
        mz = torch.cat([mask, torch.from_numpy(sink.astype(np.float64)).reshape(1, H, 1, 1).expand(1, H, L, 1)], -1)
        ref = F.scaled_dot_product_attention(qt, kz, kz, attn_mask=mz, scale=0.5)[0, :, p]
        np.testing.assert_allclose(o[0, 0], ref.numpy(), rtol=1e-12, atol=1e-13)


def decode_step(x, xi, gate, gate_i, bias, bias_i, qi, w, q, sink, p, m=4, W=8, k=3, tau=0.3):
    """Oracle decode step for the query at position p, built from raw tokens
    (window = the last W raw tokens up to p; entries j < floor((p+1)/m))."""
    n = (p + 1) // m
    ent = oracle.pool(x[: n * m], gate[: n * m], bias, m)
    keys = oracle.pool(xi[: n * m], gate_i[: n * m], bias_i, m).astype(np.float32)
    keys_full = np.zeros((1, max(n, 1), xi.shape[1]), np.float32)
    keys_full[0, :n] = keys
    idx, _ = oracle.index_topk(qi[None, None], w[None, None], keys_full, oracle.F32, None,
                               np.array([[n]], np.int32), k)
    sel = idx[0, 0][idx[0, 0] >= 0]
    lo = max(0, p - W + 1)
    return oracle.attend_row(q, ent[sel], x[lo:p + 1], sink, tau)


def test_pipeline_is_causal():
    L, D, d_I, H, Hq = 40, 16, 8, 2, 3
    g = np.random.default_rng(21)
    args = dict(x=g.standard_normal((L, D)), xi=g.standard_normal((L, d_I)),
                gate=g.standard_normal(L), gate_i=g.standard_normal(L),
                bias=g.standard_normal(4) * 0.1, bias_i=g.standard_normal(4) * 0.1,
                qi=g.standard_normal((H, d_I)), w=g.random(H).astype(np.float32),
                q=g.standard_normal((Hq, D)), sink=g.standard_normal(Hq).astype(np.float32))
    for p in (3, 17, 26):
        o, lse = decode_step(p=p, **args)
        pert = dict(args)
        for key in ("x", "xi", "gate", "gate_i"):
            a = args[key].copy()
            a[p + 1:] = g.standard_normal(a[p + 1:].shape) * 10
            pert[key] = a
        o2, lse2 = decode_step(p=p, **pert)
        np.testing.assert_array_equal(o, o2)
        np.testing.assert_array_equal(lse, lse2)
        # and a change at or before p does change the result
        pert["x"] = args["x"].copy()
        pert["x"][p] += 1.0
        o3, _ = decode_step(p=p, **pert)
        assert np.abs(o3 - o).max() > 1e-6


# --------------------------------------------------------------------------
# separate values (a variant: keys and values are different vectors)
# --------------------------------------------------------------------------
def batched_inputs(seed, B=2, Tq=2, Hq=4, D=64, N=40, W_buf=24):
    g = np.random.default_rng(seed)
    q = g.standard_normal((B, Tq, Hq, D))
    kv = g.standard_normal((B, N, D)).astype(np.float32)
    v = g.standard_normal((B, N, D)).astype(np.float32)
    win = g.standard_normal((B, W_buf, D)).astype(np.float32)
    win_v = g.standard_normal((B, W_buf, D)).astype(np.float32)
    sel = g.integers(-1, N, (B, Tq, 12)).astype(np.int32)
    wb = g.integers(0, 8, (B, Tq)).astype(np.int32)
    wl = g.integers(0, W_buf - 8 + 1, (B, Tq)).astype(np.int32)
    sink = g.standard_normal(Hq).astype(np.float32)
    return q, kv, v, win, win_v, sel, wb, wl, sink


def test_separate_values_textbook_sdpa():
    """softmax(tau q K^T) V with K != V against torch SDPA (float64), the sink
    as an extra zero-value column with its logit as the mask."""
    q, kv, v, win, win_v, sel, wb, wl, sink = batched_inputs(40)
    tau = 0.125
    o, lse = oracle.attend(q, kv, oracle.F32, None, sel, None, win, oracle.F32, wb, wl, sink, tau, v=v, win_v=win_v)
    B, Tq, Hq, D = q.shape
    for b in range(B):
        for t in range(Tq):
            js = [j for j in sel[b, t] if j >= 0]
            K = np.concatenate([kv[b, js], win[b, wb[b, t]:wb[b, t] + wl[b, t]], np.zeros((1, D))]).astype(np.float64)
            V = np.concatenate([v[b, js], win_v[b, wb[b, t]:wb[b, t] + wl[b, t]], np.zeros((1, D))]).astype(np.float64)
            mask = torch.zeros(1, Hq, 1, K.shape[0], dtype=torch.float64)
            mask[0, :, 0, -1] = torch.from_numpy(sink.astype(np.float64))
            qt = torch.from_numpy(q[b, t]).reshape(1, Hq, 1, D)
            kt = torch.from_numpy(K).reshape(1, 1, -1, D).expand(1, Hq, -1, D).contiguous()
            vt = torch.from_numpy(V).reshape(1, 1, -1, D).expand(1, Hq, -1, D).contiguous()
            ref = F.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask, scale=tau).reshape(Hq, D).numpy()
            np.testing.assert_allclose(o[b, t], ref, rtol=1e-10, atol=1e-12)
            rl = torch.logsumexp((qt @ kt.transpose(-1, -2)) * tau + mask, -1).reshape(Hq).numpy()
            np.testing.assert_allclose(lse[b, t], rl, rtol=1e-12)


def test_separate_values_equal_keys_is_shared_kv():
    q, kv, v, win, win_v, sel, wb, wl, sink = batched_inputs(41)
    a = oracle.attend(q, kv, oracle.F32, None, sel, None, win, oracle.F32, wb, wl, sink, 0.1)
    b = oracle.attend(q, kv, oracle.F32, None, sel, None, win, oracle.F32, wb, wl, sink, 0.1, v=kv, win_v=win)
    np.testing.assert_array_equal(a[0], b[0])
    np.testing.assert_array_equal(a[1], b[1])


def test_separate_values_linear_in_v_and_lse_independent_of_v():
    q, kv, v, win, win_v, sel, wb, wl, sink = batched_inputs(42)
    n_elig = np.full(sel.shape[:2], 30, np.int32)
    args = (q, kv, oracle.F32, None, None, n_elig, win, oracle.F32, wb, wl, sink, 0.1)
    g = np.random.default_rng(43)
    # quarter-integer values: their fp32 sums are exact, so linearity can be tested tightly
    v1, w1 = (g.integers(-8, 9, v.shape) / 4).astype(np.float32), (g.integers(-8, 9, win.shape) / 4).astype(np.float32)
    v2, w2 = (g.integers(-8, 9, v.shape) / 4).astype(np.float32), (g.integers(-8, 9, win.shape) / 4).astype(np.float32)
    o1, l1 = oracle.attend(*args, v=v1, win_v=w1)
    o2, l2 = oracle.attend(*args, v=v2, win_v=w2)
    o12, l12 = oracle.attend(*args, v=v1 + v2, win_v=w1 + w2)
    np.testing.assert_allclose(o12, o1 + o2, rtol=1e-12, atol=1e-13)
    np.testing.assert_array_equal(oracle.attend(*args, v=2 * v1, win_v=2 * w1)[0], 2 * o1)
    np.testing.assert_array_equal(l1, l2)
    np.testing.assert_array_equal(l1, l12)
