"""Batch invariance of the attention calls: a sequence's output and LSE bits do
not depend on the other sequences in the call.  A 16-sequence call, the
4-sequence call on sequences 4..7 and the 1-sequence call on sequence 5 must
give equal bytes for the rows they share -- for the sparse (CSA) and dense
(HCA) calls, FP8 and bf16 entries, one and four query tokens per sequence,
through the single calls and through lca_attend_batch (both branches in one
launch).  The same for the indexer's index sets and scores.  [wiki
(chenshi221), 关键技术方法 › 基础设施: batch-invariant, deterministic attention
kernels.]  Inputs are seeded N(0, 1); selected lists are seeded random subsets
of each row's eligible entries, some rows shorter than k."""
import numpy as np
import pytest
import torch

import long_context_attention_13_amd as lca
import oracle
from gpu_util import dev, empty_ws, to_dev

pytestmark = pytest.mark.gpu

B, N, N2, Hq, D, W, K = 16, 6000, 700, 64, 128, 128, 512


def inputs(kv_dt, Tq, seed):
    g = np.random.default_rng(seed)
    ent = g.standard_normal((B, N, D)).astype(np.float32)
    hca = g.standard_normal((B, N2, D)).astype(np.float32)
    if kv_dt == lca.FP8E4M3:
        ent, ent_sc = oracle.encode(ent, oracle.FP8E4M3)
        hca, hca_sc = oracle.encode(hca, oracle.FP8E4M3)
    else:
        ent, _ = oracle.encode(ent, oracle.BF16)
        hca, _ = oracle.encode(hca, oracle.BF16)
        ent_sc = hca_sc = None
    n_csa = g.integers(K // 2, N, size=(B, Tq)).astype(np.int32)
    n_hca = g.integers(1, N2 + 1, size=(B, Tq)).astype(np.int32)
    idx = np.full((B, Tq, K), -1, np.int32)
    for b in range(B):
        for t in range(Tq):
            m = min(K, int(n_csa[b, t])) - (37 if (b + t) % 5 == 0 else 0)
            idx[b, t, :m] = np.sort(g.choice(int(n_csa[b, t]), m, replace=False))
    win, _ = oracle.encode(g.standard_normal((B, W + Tq - 1, D)).astype(np.float32), oracle.BF16)
    q_csa, _ = oracle.encode(g.standard_normal((B, Tq, Hq, D)).astype(np.float32), oracle.BF16)
    q_hca, _ = oracle.encode(g.standard_normal((B, Tq, Hq, D)).astype(np.float32), oracle.BF16)
    wb = np.tile(np.arange(Tq, dtype=np.int32), (B, 1))
    wl = np.full((B, Tq), W, np.int32)
    wl[3, 0] = 17
    sink = g.standard_normal(Hq).astype(np.float32)
    tau = 1 / np.sqrt(128.0)
    dv = lambda a: None if a is None else to_dev(a)
    return dict(ent=dv(ent), ent_sc=dv(ent_sc), hca=dv(hca), hca_sc=dv(hca_sc), idx=dv(idx), n_hca=dv(n_hca),
                win=dv(win), q_csa=dv(q_csa), q_hca=dv(q_hca), wb=dv(wb), wl=dv(wl), sink=dv(sink), tau=tau, Tq=Tq)


def sl(t, b0, b1):
    return None if t is None else t[b0:b1].clone()      # a fresh (aligned) allocation


def run(x, b0, b1, batched):
    """Both attention calls on sequences b0 .. b1-1; returns (out, lse) per call."""
    nb, Tq = b1 - b0, x["Tq"]
    res = []
    jobs = []
    for sparse in (True, False):
        q = sl(x["q_csa" if sparse else "q_hca"], b0, b1)
        kv, sc = (x["ent"], x["ent_sc"]) if sparse else (x["hca"], x["hca_sc"])
        kv, sc = sl(kv, b0, b1), sl(sc, b0, b1)
        sel = sl(x["idx"] if sparse else x["n_hca"], b0, b1)
        out = torch.empty(nb, Tq, Hq, D, dtype=torch.bfloat16, device=dev())
        lse = torch.empty(nb, Tq, Hq, device=dev())
        ws = empty_ws(lca.attend_ws(nb, Tq, Hq, D, K if sparse else N2, W + Tq - 1))
        args = (q, kv, sc, sel, sl(x["win"], b0, b1), sl(x["wb"], b0, b1), sl(x["wl"], b0, b1), x["sink"], x["tau"],
                out, lse, ws)
        if batched:
            jobs.append(lca.attend_job(sparse, *args))
        else:
            (lca.sparse_mqa_attend if sparse else lca.hca_attend)(*args)
        res.append((out, lse))
    if batched:
        lca.attend_batch(jobs)
    torch.cuda.synchronize()
    return res


@pytest.mark.parametrize("batched", [False, True])
@pytest.mark.parametrize("kv_dt,Tq", [(lca.FP8E4M3, 1), (lca.BF16, 1), (lca.FP8E4M3, 4), (lca.BF16, 4)])
def test_attention_batch_invariant(kv_dt, Tq, batched):
    x = inputs(kv_dt, Tq, 60 + Tq + kv_dt)
    full = run(x, 0, B, batched)
    for b0, b1 in [(4, 8), (5, 6)]:
        part = run(x, b0, b1, batched)
        for name, (o, l), (po, pl) in zip(("csa", "hca"), full, part):
            assert torch.equal(o[b0:b1].view(torch.int16), po.view(torch.int16)), f"{name} out, sequences {b0}..{b1 - 1}"
            assert torch.equal(l[b0:b1].view(torch.int32), pl.view(torch.int32)), f"{name} lse, sequences {b0}..{b1 - 1}"


@pytest.mark.parametrize("Tq", [1, 4])
def test_indexer_batch_invariant(Tq):
    g = np.random.default_rng(90 + Tq)
    Nk, H, d, k = 40000, 8, 128, 512
    kc, ks = oracle.encode(g.standard_normal((B, Nk, d)).astype(np.float32), oracle.MXFP4)
    qc, qs = oracle.encode(g.standard_normal((B, Tq, H, d)).astype(np.float32), oracle.MXFP4)
    w = g.random((B, Tq, H)).astype(np.float32)
    n = g.integers(k // 2, Nk + 1, size=(B, Tq)).astype(np.int32)
    xs = [to_dev(a) for a in (qc, qs, w, kc, ks, n)]

    def call(b0, b1):
        nb = b1 - b0
        idx = torch.empty(nb, Tq, k, dtype=torch.int32, device=dev())
        sc = torch.empty(nb, Tq, k, dtype=torch.float64, device=dev())
        ws = empty_ws(lca.index_topk_ws(nb, Tq, H, d, Nk, k))
        a = [t[b0:b1].clone() for t in xs]
        lca.lightning_index_topk(a[0], a[1], a[2], a[3], a[4], a[5], k, idx, ws, score_out=sc)
        torch.cuda.synchronize()
        return idx, sc

    fi, fs = call(0, B)
    for b0, b1 in [(4, 8), (5, 6)]:
        pi, ps = call(b0, b1)
        assert torch.equal(fi[b0:b1], pi)
        assert torch.equal(fs[b0:b1].view(torch.int64), ps.view(torch.int64))
