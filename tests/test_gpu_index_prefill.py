"""GPU parity of lightning_index_topk on the prefill path (64 or more query
rows per sequence, MXFP4 keys of dim 128): sample threshold, MFMA scoring with
an fp32 combine, certified-band selection and the exact fallback queue.

Index sets and selected scores must equal the oracle bit for bit.  The cases
force every fallback reason: a negative head weight, keys outside the exact
MFMA envelope, ties wider than the band, and a candidate list overflow, next
to ordinary causal rows, rows with n_elig <= k, empty rows and a ragged last
row tile."""
import numpy as np
import pytest
import torch

import long_context_attention_13_amd as lca
import oracle
from gpu_util import dev, empty_ws, to_dev, to_host

pytestmark = pytest.mark.gpu


def gpu_topk(qc, qs, w, kc, ks, n_elig, k, scores=True):
    B, Tq = n_elig.shape
    H, d = qc.shape[2], qc.shape[3] * 2
    idx = torch.full((B, Tq, k), -7, dtype=torch.int32, device=dev())
    sc = torch.full((B, Tq, k), np.nan, dtype=torch.float64, device=dev()) if scores else None
    ws = empty_ws(lca.index_topk_ws(B, Tq, H, d, kc.shape[1], k))
    lca.lightning_index_topk(to_dev(qc), to_dev(qs), to_dev(w), to_dev(kc), to_dev(ks), to_dev(n_elig), k, idx, ws,
                             score_out=sc)
    torch.cuda.synchronize()
    return to_host(idx), (to_host(sc) if scores else None)


def check(qc, qs, w, kc, ks, n_elig, k, rows=None):
    gi, gs = gpu_topk(qc, qs, w, kc, ks, n_elig, k)
    gi2, _ = gpu_topk(qc, qs, w, kc, ks, n_elig, k, scores=False)
    assert np.array_equal(gi, gi2), "selection differs with and without score output"
    if rows is None:
        rows = np.arange(n_elig.shape[1])
    qd = oracle.decode(qc[:, rows], oracle.MXFP4, qs[:, rows])
    ri, rs = oracle.index_topk(qd, w[:, rows], kc, oracle.MXFP4, ks, n_elig[:, rows], k)
    for b in range(n_elig.shape[0]):
        for a, t in enumerate(rows):
            assert np.array_equal(gi[b, t], ri[b, a]), (b, t, n_elig[b, t], np.setdiff1d(gi[b, t], ri[b, a])[:8],
                                                        np.setdiff1d(ri[b, a], gi[b, t])[:8])
    assert np.array_equal(gs[:, rows].view(np.uint64), rs.view(np.uint64))
    return gi


def inputs(seed, B, Tq, H, N_cap, d=128):
    g = np.random.default_rng(seed)
    q = g.standard_normal((B, Tq, H, d)).astype(np.float32)
    keys = g.standard_normal((B, N_cap, d)).astype(np.float32)
    w = g.random((B, Tq, H), dtype=np.float32)
    qc, qs = oracle.encode(q, oracle.MXFP4)
    kc, ks = oracle.encode(keys, oracle.MXFP4)
    return qc, qs, w, kc, ks, keys


def causal(Tq, ctx, N_cap):
    p = ctx + np.arange(Tq)
    return np.minimum((p + 1) // 4, N_cap).astype(np.int32)


@pytest.mark.parametrize("H,k", [(8, 1024), (8, 64), (4, 512), (16, 256)])
def test_causal_rows(H, k):
    B, Tq, N_cap = 2, 96, 20480
    qc, qs, w, kc, ks, _ = inputs(100 + H + k, B, Tq, H, N_cap)
    n = np.stack([causal(Tq, 4 * 20000, N_cap), causal(Tq, 4 * 9000, N_cap)])
    check(qc, qs, w, kc, ks, n, k)


@pytest.mark.parametrize("N_cap,k", [(262144, 1024), (131072, 512)])
def test_long_cache_rows(N_cap, k):
    """Key caches of a ~1M-token context (262144 entries) and of 131072: the
    sample workgroups take 8 and 4 rows, the emission makes several bitmap
    passes (rows of 100000 and 245760+ entries cross 122880).  Sampled rows
    against the oracle."""
    B, Tq, H = 1, 64, 8
    qc, qs, w, kc, ks, _ = inputs(300 + k, B, Tq, H, N_cap)
    n = causal(Tq, 4 * (N_cap - 64), N_cap)[None].copy()
    n[0, 5], n[0, 9], n[0, 13] = 100000, 122881, 2000
    check(qc, qs, w, kc, ks, n, k, rows=np.array([0, 5, 9, 13, 40, 63]))


def test_short_and_empty_rows():
    """n_elig of 0, 1, around k, and the sample threshold's small-sample case."""
    B, Tq, N_cap, k = 1, 64, 8192, 512
    qc, qs, w, kc, ks, _ = inputs(7, B, Tq, 8, N_cap)
    n = np.array([0, 1, 5, 511, 512, 513, 700, 1000, 2047, 2048, 2049, 4000] + [8192] * 52, np.int32)[None]
    check(qc, qs, w, kc, ks, n, k)


def test_negative_head_weight_row():
    B, Tq, N_cap, k = 1, 64, 16384, 1024
    qc, qs, w, kc, ks, _ = inputs(8, B, Tq, 8, N_cap)
    w[0, 5, 3] = -0.75
    w[0, 40, :] = 0.0                      # all-zero weights: every score is 0
    check(qc, qs, w, kc, ks, np.full((B, Tq), N_cap, np.int32), k)


def test_keys_outside_envelope():
    """Block scales 2^14 apart inside some keys of one key range: the rows of
    every workgroup that reads them are selected by the exact fallback."""
    B, Tq, N_cap, k = 1, 128, 16384, 512
    g = np.random.default_rng(9)
    qc, qs, w, _, _, keys = inputs(9, B, Tq, 8, N_cap)
    sel = np.zeros(N_cap, bool)
    sel[3000:3100] = g.random(100) < 0.5
    keys[0, sel, :32] *= 2.0 ** 14
    keys[0, 9000:9010, 64:96] = 0.0        # zero blocks (E8M0 code 0)
    kc, ks = oracle.encode(keys, oracle.MXFP4)
    check(qc, qs, w, kc, ks, np.full((B, Tq), N_cap, np.int32), k)


def test_ties_wider_than_band():
    """Hundreds of copies of one key straddle the k-th place."""
    B, Tq, N_cap, k = 1, 64, 16384, 700
    qc, qs, w, kc, ks, _ = inputs(10, B, Tq, 8, N_cap)
    kc[0, 50:16384:9] = kc[0, 7]
    ks[0, 50:16384:9] = ks[0, 7]
    check(qc, qs, w, kc, ks, np.full((B, Tq), N_cap, np.int32), k)


def test_concentrated_candidates_overflow_a_list():
    """The top entries of every row packed into one key range: its candidate
    lists overflow and the rows go to the fallback."""
    B, Tq, N_cap, k = 1, 64, 32768, 1024
    qc, qs, w, kc, ks, _ = inputs(11, B, Tq, 8, N_cap)
    q = oracle.decode(qc, oracle.MXFP4, qs)[0]
    strong = np.clip(q.sum((0, 1)), -6, 6).astype(np.float32)
    g = np.random.default_rng(12)
    blk = (strong[None] * (1 + 0.05 * g.standard_normal((1500, 128)))).astype(np.float32)
    kcs, kss = oracle.encode(blk, oracle.MXFP4)
    kc[0, 4100:5600] = kcs
    ks[0, 4100:5600] = kss
    check(qc, qs, w, kc, ks, np.full((B, Tq), N_cap, np.int32), k, rows=np.arange(0, 64, 7))


def test_matches_decode_path_rows():
    """The same rows through the decode path (one query row per call) select
    the same entries."""
    B, Tq, N_cap, k = 1, 64, 24576, 1024
    qc, qs, w, kc, ks, _ = inputs(13, B, Tq, 8, N_cap)
    n = causal(Tq, 4 * 24000, N_cap)[None]
    gi, gs = gpu_topk(qc, qs, w, kc, ks, n, k)
    for t in (0, 17, 63):
        di, ds = gpu_topk(qc[:, t:t + 1], qs[:, t:t + 1], w[:, t:t + 1], kc, ks, n[:, t:t + 1], k)
        assert np.array_equal(di[0, 0], gi[0, t])
        assert np.array_equal(ds[0, 0].view(np.uint64), gs[0, t].view(np.uint64))
