"""GPU parity of lca_attend_separate_v (attention with separate key and value
vectors, a variant of the shared-KV reading) against the oracle on the same
encoded inputs.  bf16 queries and windows with bf16 or FP8 entries run on the
matrix-core kernels (key and value tiles staged separately): rtol 2e-2 like
the other bf16/FP8 attention tests; fp32 storage runs on the vector-ALU
kernel: rtol 1e-4.  Covers sparse lists with -1 padding, dense HCA lists,
split rows merged by LSE (long lists), prefill-shaped dense row groups,
ragged and empty windows, FP8 / bf16 / fp32 storage, 16 and 64 heads; values
equal to the keys reproduce the shared-KV call's bytes on both kernels.
Inputs are seeded N(0, 1)."""
import math

import numpy as np
import pytest
import torch

import long_context_attention_13_amd as lca
import oracle
from gpu_util import assert_lse_close, assert_rows_close, dev, empty_ws, to_dev, to_host

pytestmark = pytest.mark.gpu

OD = {lca.F32: oracle.F32, lca.BF16: oracle.BF16, lca.FP8E4M3: oracle.FP8E4M3}
D = 128


def case(seed, sparse, B, Tq, Hq, N_cap, k, W_buf, kv_dt, win_dt, q_dt):
    g = np.random.default_rng(seed)
    K, Ks = oracle.encode(g.standard_normal((B, N_cap, D)).astype(np.float32), OD[kv_dt])
    V, Vs = oracle.encode(g.standard_normal((B, N_cap, D)).astype(np.float32), OD[kv_dt])
    WK, _ = oracle.encode(g.standard_normal((B, W_buf, D)).astype(np.float32), OD[win_dt])
    WV, _ = oracle.encode(g.standard_normal((B, W_buf, D)).astype(np.float32), OD[win_dt])
    qc, _ = oracle.encode(g.standard_normal((B, Tq, Hq, D)).astype(np.float32), OD[q_dt])
    if sparse:
        sel = g.integers(-1, N_cap, (B, Tq, k)).astype(np.int32)
    else:
        sel = g.integers(0, N_cap + 1, (B, Tq)).astype(np.int32)
        sel[0, 0] = 0
    wl = g.integers(0, min(W_buf, 128) + 1, (B, Tq)).astype(np.int32)
    wl[-1, -1] = 0
    wb = np.array([[g.integers(0, W_buf - n + 1) for n in row] for row in wl], np.int32)
    sink = g.standard_normal(Hq).astype(np.float32)
    return qc, K, Ks, V, Vs, WK, WV, sel, wb, wl, sink


def run_gpu(sparse, qc, K, Ks, V, Vs, WK, WV, sel, wb, wl, sink, tau, out_dt=lca.F32):
    B, Tq, Hq, _ = qc.shape
    out = torch.full((B, Tq, Hq, D), float("nan"), device=dev(),
                     dtype=torch.float32 if out_dt == lca.F32 else torch.bfloat16)
    lse = torch.full((B, Tq, Hq), float("nan"), device=dev())
    nmax = sel.shape[-1] if sparse else K.shape[1]
    ws = empty_ws(lca.attend_ws(B, Tq, Hq, D, nmax, WK.shape[1]))
    t = lambda a: None if a is None else to_dev(a)
    lca.attend_separate_v(sparse, t(qc), t(K), t(V), t(Ks), t(Vs), t(sel), t(WK), t(WV), t(wb), t(wl), t(sink), tau,
                          out, lse, ws)
    torch.cuda.synchronize()
    o = to_host(out)
    return (o.astype(np.float64) if out_dt == lca.F32 else oracle.decode(o, oracle.BF16)), to_host(lse)


CASES = [  # sparse, B, Tq, Hq, N_cap, k, W_buf, kv_dt, win_dt, q_dt
    (True, 2, 3, 64, 3000, 512, 300, lca.FP8E4M3, lca.BF16, lca.BF16),
    (True, 3, 2, 16, 500, 1500, 200, lca.BF16, lca.BF16, lca.BF16),
    (True, 1, 4, 64, 200, 0, 160, lca.F32, lca.F32, lca.F32),
    (False, 2, 2, 64, 2500, 0, 256, lca.FP8E4M3, lca.BF16, lca.BF16),
    (False, 2, 3, 16, 700, 0, 130, lca.F32, lca.F32, lca.F32),
    (False, 1, 70, 64, 900, 0, 200, lca.BF16, lca.BF16, lca.BF16),      # dense row groups (prefill shape)
    (True, 1, 66, 32, 1200, 256, 200, lca.FP8E4M3, lca.BF16, lca.BF16),  # one split per row (prefill shape)
]


@pytest.mark.parametrize("sparse,B,Tq,Hq,N_cap,k,W_buf,kv_dt,win_dt,q_dt", CASES)
def test_separate_values_match_oracle(sparse, B, Tq, Hq, N_cap, k, W_buf, kv_dt, win_dt, q_dt):
    qc, K, Ks, V, Vs, WK, WV, sel, wb, wl, sink = case(17 + N_cap, sparse, B, Tq, Hq, N_cap, k, W_buf, kv_dt, win_dt,
                                                       q_dt)
    tau = 1.0 / math.sqrt(D)
    o, l = run_gpu(sparse, qc, K, Ks, V, Vs, WK, WV, sel, wb, wl, sink, tau)
    ro, rl = oracle.attend(oracle.decode(qc, OD[q_dt]), K, OD[kv_dt], Ks, sel if sparse else None,
                           None if sparse else sel, WK, OD[win_dt], wb, wl, sink, tau, v=V, v_scale=Vs, win_v=WV)
    rt = 1e-4 if kv_dt == lca.F32 else 2e-2
    assert_rows_close(o, ro, rt, "out")
    assert_lse_close(l, rl, rt, "lse")


@pytest.mark.parametrize("sparse,kv_dt,Tq", [(True, lca.FP8E4M3, 1), (False, lca.FP8E4M3, 2), (True, lca.BF16, 3)])
def test_values_equal_keys_on_matrix_cores(sparse, kv_dt, Tq):
    """bf16 / FP8 storage at decode shapes (split rows): V = K gives the bytes
    of lca_sparse_mqa_attend / lca_hca_attend."""
    N_cap, k, W_buf, B, Hq = 3000, 700, 200, 2, 64
    qc, K, Ks, V, Vs, WK, WV, sel, wb, wl, sink = case(9 + Tq, sparse, B, Tq, Hq, N_cap, k, W_buf, kv_dt, lca.BF16,
                                                       lca.BF16)
    tau = 0.09
    o, l = run_gpu(sparse, qc, K, Ks, K, Ks, WK, WK, sel, wb, wl, sink, tau, out_dt=lca.BF16)
    out = torch.zeros(B, Tq, Hq, D, dtype=torch.bfloat16, device=dev())
    lse = torch.zeros(B, Tq, Hq, device=dev())
    ws = empty_ws(lca.attend_ws(B, Tq, Hq, D, k if sparse else N_cap, W_buf))
    t = lambda a: None if a is None else to_dev(a)
    (lca.sparse_mqa_attend if sparse else lca.hca_attend)(t(qc), t(K), t(Ks), t(sel), t(WK), t(wb), t(wl), t(sink),
                                                          tau, out, lse, ws)
    torch.cuda.synchronize()
    ref = oracle.decode(to_host(out), oracle.BF16)
    assert np.array_equal(o.view(np.uint64), ref.view(np.uint64))
    assert np.array_equal(l.view(np.uint32), to_host(lse).view(np.uint32))


def test_values_equal_keys_give_the_shared_kv_call():
    """fp32 storage (the shared-KV call also runs the vector-ALU kernel): the
    same bytes as lca_sparse_mqa_attend."""
    qc, K, Ks, V, Vs, WK, WV, sel, wb, wl, sink = case(5, True, 2, 2, 64, 900, 700, 200, lca.F32, lca.F32, lca.F32)
    tau = 0.09
    o, l = run_gpu(True, qc, K, None, K, None, WK, WK, sel, wb, wl, sink, tau)
    out = torch.zeros(2, 2, 64, D, device=dev())
    lse = torch.zeros(2, 2, 64, device=dev())
    ws = empty_ws(lca.attend_ws(2, 2, 64, D, 700, 200))
    lca.sparse_mqa_attend(to_dev(qc), to_dev(K), None, to_dev(sel), to_dev(WK), to_dev(wb), to_dev(wl), to_dev(sink),
                          tau, out, lse, ws)
    torch.cuda.synchronize()
    assert np.array_equal(o.astype(np.float32).view(np.uint32), to_host(out).view(np.uint32))
    assert np.array_equal(l.view(np.uint32), to_host(lse).view(np.uint32))
