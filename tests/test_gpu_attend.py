"""GPU parity of sparse_mqa_attend / hca_attend against the float64 oracle on
the same encoded inputs: rtol 1e-4 for fp32 inputs, 2e-2 for bf16/FP8 inputs
(per element, relative to |ref| plus the row's largest |ref|), outputs and
LSE.  Covers split-KV decode rows, single-split prefill rows with per-row
windows, -1 padding, k = 0, n_elig = 0, empty windows."""
import math

import numpy as np
import pytest
import torch

import long_context_attention_13_amd as lca
import oracle
import synth
from gpu_util import assert_lse_close, assert_rows_close, dev, empty_ws, to_dev, to_host

pytestmark = pytest.mark.gpu

OD = {lca.F32: oracle.F32, lca.BF16: oracle.BF16, lca.FP8E4M3: oracle.FP8E4M3}


def enc(a, dt):
    return oracle.encode(a, OD[dt])


def run(sparse, q, q_dt, kv, kv_dt, kv_sc, sel_or_n, win, win_dt, wb, wl, sink, tau, out_dt):
    B, Tq, Hq, D = q.shape
    qc, _ = enc(q, q_dt)
    N_cap, W_buf = kv.shape[1], win.shape[1]
    out = torch.full((B, Tq, Hq, D), np.nan, device=dev(),
                     dtype=torch.float32 if out_dt == lca.F32 else torch.bfloat16)
    lse = torch.full((B, Tq, Hq), np.nan, device=dev(), dtype=torch.float32)
    nmax = sel_or_n.shape[-1] if sparse else N_cap
    ws = empty_ws(lca.attend_ws(B, Tq, Hq, D, nmax, W_buf))
    args = (to_dev(qc), to_dev(kv), None if kv_sc is None else to_dev(kv_sc), to_dev(sel_or_n), to_dev(win),
            to_dev(wb), to_dev(wl), to_dev(sink), tau, out, lse, ws)
    (lca.sparse_mqa_attend if sparse else lca.hca_attend)(*args)
    torch.cuda.synchronize()
    o = to_host(out)
    o = o.astype(np.float64) if out_dt == lca.F32 else oracle.decode(o, oracle.BF16)
    # oracle on the same stored inputs
    qd = oracle.decode(qc, OD[q_dt])
    ro, rl = oracle.attend(qd, kv, OD[kv_dt], kv_sc, sel_or_n if sparse else None,
                           None if sparse else sel_or_n, win, OD[win_dt], wb, wl, sink, tau)
    return o, to_host(lse).astype(np.float64), ro, rl


def rtol_for(*dts):
    return 1e-4 if all(d == lca.F32 for d in dts) else 2e-2


def make(seed, B, Tq, Hq, N_cap, W_buf, kv_dt, win_dt, D=128):
    g = np.random.default_rng(seed)
    kv32 = g.standard_normal((B, N_cap, D)).astype(np.float32)
    kv, kv_sc = enc(kv32, kv_dt)
    win, _ = enc(g.standard_normal((B, W_buf, D)).astype(np.float32), win_dt)
    q = g.standard_normal((B, Tq, Hq, D)).astype(np.float32)
    sink = g.standard_normal(Hq).astype(np.float32)
    return g, q, kv, kv_sc, win, sink


def test_small_fp32_config():
    """4096-token fp32 decode: 16 heads, top-64 of 1024 entries + 128-token window, tau 1."""
    c = synth.small_csa_decode()
    g = np.random.default_rng(21)
    kv = g.standard_normal((1, 1024, 128)).astype(np.float32)
    win = c["x"][:, -128:, :]
    sel = np.sort(g.choice(1024, 64, replace=False)).astype(np.int32)[None, None]
    o, l, ro, rl = run(True, c["q"], lca.F32, kv, lca.F32, None, sel, win, lca.F32,
                       np.zeros((1, 1), np.int32), np.full((1, 1), 128, np.int32), c["sink"], 1.0, lca.F32)
    assert_rows_close(o, ro, 1e-4, "out")
    assert_lse_close(l, rl, 1e-4, "lse")


@pytest.mark.parametrize("kv_dt,q_dt,out_dt", [(lca.FP8E4M3, lca.BF16, lca.BF16), (lca.BF16, lca.BF16, lca.F32),
                                               (lca.F32, lca.F32, lca.F32)])
def test_sparse_decode_rows(kv_dt, q_dt, out_dt):
    B, Hq, N_cap, k, W = 3, 64, 6000, 512, 128
    g, q, kv, kv_sc, win, sink = make(31 + kv_dt, B, 1, Hq, N_cap, W, kv_dt, lca.BF16 if q_dt == lca.BF16 else lca.F32)
    sel = np.stack([np.sort(g.choice(N_cap, k, replace=False)) for _ in range(B)]).astype(np.int32)[:, None]
    sel[1, 0, 400:] = -1                           # fewer than k selected
    sel[2, 0, :] = -1
    sel[2, 0, :3] = [0, 17, N_cap - 1]
    wl = np.array([[128], [5], [0]], np.int32)
    wdt = lca.BF16 if q_dt == lca.BF16 else lca.F32
    o, l, ro, rl = run(True, q, q_dt, kv, kv_dt, kv_sc, sel, win, wdt, np.zeros((B, 1), np.int32), wl, sink,
                       1 / math.sqrt(128), out_dt)
    rt = rtol_for(kv_dt, q_dt, out_dt)
    assert_rows_close(o, ro, rt, "out")
    assert_lse_close(l, rl, rt, "lse")


@pytest.mark.parametrize("Hq", [16, 32, 64])
@pytest.mark.parametrize("k", [40, 700])
def test_fp32_rows_every_head_count(Hq, k):
    """The fp32 kernel's per-head lane groups (256 / Hq lanes a head, 32 / (256
    / Hq) items a lane and tile) on ragged lists: a partial last tile, -1
    indices inside the list, a short window, an empty window, lists of one
    split (k = 40 with a 64-token window buffer: 104 items at most) and lists
    cut into splits (k = 700 with 128)."""
    B, N_cap = 3, 3000
    W = 64 if k == 40 else 128
    g, q, kv, kv_sc, win, sink = make(91 + Hq + k, B, 1, Hq, N_cap, W, lca.F32, lca.F32)
    sel = np.stack([np.sort(g.choice(N_cap, k, replace=False)) for _ in range(B)]).astype(np.int32)[:, None]
    sel[1, 0, 3::7] = -1
    wl = np.array([[W], [5], [0]], np.int32)
    o, l, ro, rl = run(True, q, lca.F32, kv, lca.F32, None, sel, win, lca.F32, np.zeros((B, 1), np.int32), wl, sink,
                       1 / math.sqrt(128), lca.F32)
    assert_rows_close(o, ro, 1e-4, "out")
    assert_lse_close(l, rl, 1e-4, "lse")


@pytest.mark.parametrize("kv_dt,N_cap", [(lca.BF16, 512), (lca.FP8E4M3, 8192), (lca.FP8E4M3, 1000)])
def test_hca_decode_rows(kv_dt, N_cap):
    B, Hq, W = 3, 64, 128
    g, q, kv, kv_sc, win, sink = make(41 + N_cap, B, 1, Hq, N_cap, W, kv_dt, lca.BF16)
    n = np.array([[N_cap], [N_cap // 3], [0]], np.int32)
    wl = np.array([[128], [128], [40]], np.int32)
    o, l, ro, rl = run(False, q, lca.BF16, kv, kv_dt, kv_sc, n, win, lca.BF16, np.zeros((B, 1), np.int32), wl,
                       sink, 1 / math.sqrt(128), lca.BF16)
    assert_rows_close(o, ro, 2e-2, "out")
    assert_lse_close(l, rl, 2e-2, "lse")


def test_prefill_rows_with_sliding_windows():
    """Tq consecutive queries over one window buffer (W-1 earlier tokens + the
    chunk): row i attends tokens [i, i+W) of the buffer and n_elig grows."""
    B, Tq, Hq, N_cap, W = 1, 300, 32, 600, 128
    g, q, kv, kv_sc, win, sink = make(51, B, Tq, Hq, N_cap, W - 1 + Tq, lca.BF16, lca.BF16)
    wb = np.arange(Tq, dtype=np.int32)[None]
    wl = np.full((1, Tq), W, np.int32)
    n = (np.minimum(500 + np.arange(Tq) // 4, N_cap)).astype(np.int32)[None]
    o, l, ro, rl = run(False, q, lca.BF16, kv, lca.BF16, None, n, win, lca.BF16, wb, wl, sink,
                       1 / math.sqrt(128), lca.BF16)
    assert_rows_close(o, ro, 2e-2, "out")
    sel = np.stack([np.sort(g.choice(N_cap, 200, replace=False)) for _ in range(Tq)]).astype(np.int32)[None]
    o, l, ro, rl = run(True, q, lca.BF16, kv, lca.BF16, None, sel, win, lca.BF16, wb, wl, sink,
                       1 / math.sqrt(128), lca.BF16)
    assert_rows_close(o, ro, 2e-2, "out sparse")
    assert_lse_close(l, rl, 2e-2, "lse sparse")


@pytest.mark.parametrize("out_dt", [lca.BF16, lca.F32])
def test_sparse_prefill_rows_64_heads(out_dt):
    """Sparse rows of a prefill chunk with 64 heads and bf16 entries (one
    workgroup per row, no split): lists of 200 selected entries (not a whole
    number of tiles), -1 padding in some rows and a row with no entry, rows
    of two sequences, windows that slide, start short or are empty."""
    B, Tq, Hq, N_cap, W = 2, 150, 64, 700, 128
    W_buf = W - 1 + Tq
    g, q, kv, kv_sc, win, sink = make(83, B, Tq, Hq, N_cap, W_buf, lca.BF16, lca.BF16)
    wb = np.stack([np.arange(Tq), np.arange(Tq)]).astype(np.int32)
    wl = np.full((B, Tq), W, np.int32)
    wl[1, :30] = np.arange(30)                  # the second sequence starts inside the chunk
    wb[1, :30] += W - 1 - np.arange(30)
    wl[0, 11] = 0                               # an empty window
    sel = np.stack([np.stack([np.sort(g.choice(N_cap, 200, replace=False)) for _ in range(Tq)])
                    for _ in range(B)]).astype(np.int32)
    sel[0, 3, 150:] = -1                        # a short list, padded
    sel[1, 7, :] = -1                           # no selected entry at all
    o, l, ro, rl = run(True, q, lca.BF16, kv, lca.BF16, None, sel, win, lca.BF16, wb, wl, sink,
                       1 / math.sqrt(128), out_dt)
    assert_rows_close(o, ro, 2e-2, "out")
    assert_lse_close(l, rl, 2e-2, "lse")


def test_empty_lists_give_sink_only():
    B, Hq = 2, 16
    g, q, kv, kv_sc, win, sink = make(61, B, 1, Hq, 64, 8, lca.F32, lca.F32)
    sel = np.full((B, 1, 4), -1, np.int32)
    o, l, ro, rl = run(True, q, lca.F32, kv, lca.F32, None, sel, win, lca.F32, np.zeros((B, 1), np.int32),
                       np.zeros((B, 1), np.int32), sink, 0.1, lca.F32)
    assert np.all(o == 0)
    np.testing.assert_allclose(l, np.broadcast_to(sink, l.shape), rtol=1e-6)


@pytest.mark.parametrize("Hq,kv_dt", [(64, lca.FP8E4M3), (64, lca.BF16), (16, lca.BF16)])
def test_dense_row_groups(Hq, kv_dt):
    """Dense prefill rows processed in groups that share staged tiles (64 heads
    with bf16 entries: a wavefront per row and all heads): a ragged last group,
    rows of two sequences, n_elig from 0 up, windows that start short
    (sequence start), an empty window and windows in any order."""
    B, Tq, N_cap, W = 2, 301, 700, 128
    W_buf = W - 1 + Tq
    g, q, kv, kv_sc, win, sink = make(71 + Hq, B, Tq, Hq, N_cap, W_buf, kv_dt, lca.BF16)
    wb = np.stack([np.arange(Tq), np.maximum(np.arange(Tq) - 40, 0)]).astype(np.int32) + W - 1
    wb[1] = np.minimum(wb[1], W_buf - W)
    wl = np.full((B, Tq), W, np.int32)
    wl[1, :40] = np.arange(40)                  # the second sequence starts inside the chunk
    wl[0, 7] = 0                                # an empty window
    wb[0] -= W - 1
    wb[0, 100:104] = wb[0, 100:104][::-1]       # a group with windows out of order
    n = np.stack([np.minimum(np.arange(Tq) // 2, N_cap), np.minimum(300 + np.arange(Tq), N_cap)]).astype(np.int32)
    n[0, :5] = 0
    o, l, ro, rl = run(False, q, lca.BF16, kv, kv_dt, kv_sc, n, win, lca.BF16, wb, wl, sink, 1 / math.sqrt(128),
                       lca.BF16)
    assert_rows_close(o, ro, 2e-2, "out")
    assert_lse_close(l, rl, 2e-2, "lse")


@pytest.mark.parametrize("kv_dt,Hq", [(lca.FP8E4M3, 64), (lca.BF16, 16)])
def test_batch_equals_single_calls(kv_dt, Hq):
    """lca_attend_batch over a sparse job with splits, a dense job with splits,
    a short job without splits and an empty job gives the bytes of the single
    calls (outputs and LSE)."""
    d = dev()
    g = torch.Generator(device=d)
    g.manual_seed(404 + Hq)
    B, D, N_cap, W = 2, 128, 5000, 128
    rn = lambda *s: torch.randn(*s, generator=g, device=d)

    def cache():
        x = rn(B, N_cap, D)
        if kv_dt == lca.BF16:
            return x.to(torch.bfloat16), None
        codes = torch.empty(B, N_cap, D, dtype=torch.uint8, device=d)
        sc = torch.empty(B, N_cap, D // 64, device=d)
        i32 = lambda v: torch.full((B,), v, dtype=torch.int32, device=d)
        lca.csa_compress(x, torch.zeros(B, N_cap, device=d), torch.zeros(1, device=d), 1, i32(0), i32(N_cap),
                         torch.zeros(B, dtype=torch.int64, device=d), N_cap, codes, lca.FP8E4M3, sc)
        return codes, sc

    kv, kv_sc = cache()
    win = rn(B, 3 * W, D).to(torch.bfloat16)
    sink = rn(Hq)
    tau = 1 / math.sqrt(D)
    idx = torch.stack([torch.randperm(N_cap, generator=g, device=d)[:700] for _ in range(B)]).to(torch.int32)
    idx[1, 5:40] = -1
    idx = idx.sort(dim=-1).values.view(B, 1, 700)
    idx_short = idx[:, :, :16].contiguous()
    n = torch.tensor([[N_cap], [3001]], dtype=torch.int32, device=d)
    wb = torch.tensor([[0], [W]], dtype=torch.int32, device=d)
    wl = torch.tensor([[W], [W - 5]], dtype=torch.int32, device=d)
    wl_s = torch.tensor([[40], [0]], dtype=torch.int32, device=d)
    win_s = win[:, :100].contiguous()               # 16 + 100 items: a single split
    wb_s = torch.zeros(B, 1, dtype=torch.int32, device=d)
    specs = [(True, idx, win, wb, wl, True), (False, n, win, wb, wl, False),
             (True, idx_short, win_s, wb_s, wl_s, True)]
    single, batch, jobs = [], [], []
    for sparse, sel, win, wb, wlen, with_lse in specs:
        q = rn(B, 1, Hq, D).to(torch.bfloat16)
        nmax = sel.shape[-1] if sparse else N_cap
        for lst in (single, batch):
            out = torch.full((B, 1, Hq, D), 3.0, device=d).to(torch.bfloat16)
            lse = torch.full((B, 1, Hq), 5.0, device=d) if with_lse else None
            ws = empty_ws(lca.attend_ws(B, 1, Hq, D, nmax, win.shape[1]))
            lst.append((out, lse, ws))
        out, lse, ws = single[-1]
        fn = lca.sparse_mqa_attend if sparse else lca.hca_attend
        fn(q, kv, kv_sc, sel, win, wb, wlen, sink, tau, out, lse, ws=ws)
        out, lse, ws = batch[-1]
        jobs.append(lca.attend_job(sparse, q, kv, kv_sc, sel, win, wb, wlen, sink, tau, out, lse, ws))
    # an empty job (no query rows)
    q0 = torch.empty(0, 1, Hq, D, dtype=torch.bfloat16, device=d)
    assert lca.attend_ws(B, 1, Hq, D, 16, 100) == 0
    jobs.append(lca.attend_job(True, q0, kv, kv_sc, idx[:0], win, wb[:0], wl[:0], sink, tau,
                               torch.empty(0, 1, Hq, D, dtype=torch.bfloat16, device=d)))
    lca.attend_batch(jobs)                      # each job keeps its own query and index arrays alive
    torch.cuda.synchronize()
    del jobs
    for j, (a, b) in enumerate(zip(single, batch)):
        assert torch.equal(a[0].view(torch.int16), b[0].view(torch.int16)), f"job {j} out"
        if a[1] is not None:
            assert torch.equal(a[1], b[1]), f"job {j} lse"
