"""GPU parity of lightning_index_topk against the oracle: selected index sets
bit-exact (ties to the lower index) and the selected scores bit-exact in
float64, on the same encoded inputs.

Covers the fp32 path (64-dim, 4 heads), MXFP4 decode rows on both the
candidate path (many entries) and the direct path (few entries), paired query
rows (prefill), ragged n_elig, k >= n_elig, n_elig = 0, equal keys, keys
outside the exact-MFMA envelope, and inputs that defeat the per-chunk
candidate bound so the exact streamed fallback runs."""
import numpy as np
import pytest
import torch

import long_context_attention_13_amd as lca
import oracle
import synth
from gpu_util import dev, empty_ws, to_dev, to_host

pytestmark = pytest.mark.gpu


def gpu_topk(qc, qs, w, kc, ks, n_elig, k, H, d):
    B, Tq = n_elig.shape
    N_cap = kc.shape[1]
    idx = torch.full((B, Tq, k), -7, dtype=torch.int32, device=dev())
    sc = torch.full((B, Tq, k), np.nan, dtype=torch.float64, device=dev())
    ws = empty_ws(lca.index_topk_ws(B, Tq, H, d, N_cap, k))
    lca.lightning_index_topk(to_dev(qc), None if qs is None else to_dev(qs), to_dev(w), to_dev(kc),
                             None if ks is None else to_dev(ks), to_dev(n_elig), k, idx, ws, score_out=sc,
                             H_I=H, d_I=d)
    torch.cuda.synchronize()
    return to_host(idx), to_host(sc)


def check(qc, qs, w, kc, ks, n_elig, k, H, d, dt):
    gi, gs = gpu_topk(qc, qs, w, kc, ks, n_elig, k, H, d)
    qd = oracle.decode(qc, dt, qs)
    ri, rs = oracle.index_topk(qd, w, kc, dt, ks, n_elig, k)
    for b in range(n_elig.shape[0]):
        for t in range(n_elig.shape[1]):
            assert np.array_equal(gi[b, t], ri[b, t]), (b, t, n_elig[b, t], np.setdiff1d(gi[b, t], ri[b, t])[:8],
                                                        np.setdiff1d(ri[b, t], gi[b, t])[:8])
    assert np.array_equal(gs.view(np.uint64), rs.view(np.uint64))
    return gi


def mx_inputs(seed, B, Tq, H, d, N_cap, key_scale=1.0):
    g = np.random.default_rng(seed)
    q = g.standard_normal((B, Tq, H, d)).astype(np.float32)
    keys = (g.standard_normal((B, N_cap, d)) * key_scale).astype(np.float32)
    w = g.random((B, Tq, H), dtype=np.float32)
    qc, qs = oracle.encode(q, oracle.MXFP4)
    kc, ks = oracle.encode(keys, oracle.MXFP4)
    return qc, qs, w, kc, ks


def test_small_fp32_config():
    """4096-token fp32 decode: 1024 entries, 4 heads x 64, top-64."""
    c = synth.small_csa_decode()
    g = np.random.default_rng(7)
    keys = g.standard_normal((1, 1024, 64)).astype(np.float32)
    n = np.array([[1024]], np.int32)
    check(c["qi"], None, c["w"], keys, None, n, 64, 4, 64, oracle.F32)


def test_fp32_chunk_path():
    g = np.random.default_rng(8)
    B, N, H, d = 2, 12000, 4, 64
    q = g.standard_normal((B, 1, H, d)).astype(np.float32)
    keys = g.standard_normal((B, N, d)).astype(np.float32)
    w = g.random((B, 1, H), dtype=np.float32)
    check(q, None, w, keys, None, np.array([[12000], [9001]], np.int32), 100, H, d, oracle.F32)


@pytest.mark.parametrize("N_cap,n_list,k", [
    (20000, [20000, 15123, 9000], 512),          # candidate path, ragged
    (8192, [8192, 5000, 3], 512),                # direct path
    (40000, [40000, 33333], 2048),
    (2000, [2000, 0, 1999], 2048),               # k >= n_elig, empty row
])
def test_mxfp4_decode_rows(N_cap, n_list, k):
    B = len(n_list)
    qc, qs, w, kc, ks = mx_inputs(N_cap + k, B, 1, 8, 128, N_cap)
    check(qc, qs, w, kc, ks, np.array(n_list, np.int32)[:, None], k, 8, 128, oracle.MXFP4)


@pytest.mark.parametrize("H,d", [(4, 64), (16, 128), (1, 128), (5, 64)])
def test_mxfp4_head_shapes(H, d):
    qc, qs, w, kc, ks = mx_inputs(H * d, 2, 3, H, d, 12000)
    n = np.array([[12000, 11000, 9000], [8000, 12000, 100]], np.int32)
    check(qc, qs, w, kc, ks, n, 256, H, d, oracle.MXFP4)


def test_prefill_rows_causal():
    """Chunked-prefill style: consecutive queries, n_elig = floor((p+1)/4)."""
    B, Tq, N_cap, k = 1, 7, 16384, 1024
    qc, qs, w, kc, ks = mx_inputs(3, B, Tq, 8, 128, N_cap)
    p = 40000 + np.arange(Tq) * 2300
    n = np.minimum((p + 1) // 4, N_cap).astype(np.int32)[None]
    check(qc, qs, w, kc, ks, n, k, 8, 128, oracle.MXFP4)


def test_equal_keys_prefer_lower_index():
    qc, qs, w, kc, ks = mx_inputs(11, 1, 1, 8, 128, 16000)
    # many copies of one strong key: ties straddle the k-th place
    kc[0, 100:16000:7] = kc[0, 5]
    ks[0, 100:16000:7] = ks[0, 5]
    gi = check(qc, qs, w, kc, ks, np.array([[16000]], np.int32), 300, 8, 128, oracle.MXFP4)
    # and in the direct path
    check(qc, qs, w, kc[:, :6000], ks[:, :6000], np.array([[6000]], np.int32), 300, 8, 128, oracle.MXFP4)


def test_keys_outside_exact_envelope():
    """Block scales 2^14 apart inside one key: those keys take the exact
    float64 path; zero blocks (E8M0 code 0) too."""
    g = np.random.default_rng(12)
    qc, qs, w, kc, ks = mx_inputs(12, 1, 2, 8, 128, 12000)
    keys = g.standard_normal((1, 12000, 128)).astype(np.float32)
    sel = g.random(12000) < 0.3
    keys[0, sel, :32] *= 2.0 ** 14
    keys[0, g.random(12000) < 0.05, 64:96] = 0.0
    kc, ks = oracle.encode(keys, oracle.MXFP4)
    check(qc, qs, w, kc, ks, np.array([[12000, 11999]], np.int32), 700, 8, 128, oracle.MXFP4)


def test_concentrated_top_entries_force_fallback():
    """All top-k entries packed into two adjacent chunks: the per-chunk
    candidate bound cannot hold them, so the certified check must reject the
    candidates and the exact streamed pass must produce the result."""
    qc, qs, w, kc, ks = mx_inputs(13, 1, 1, 8, 128, 30000)
    q = oracle.decode(qc, oracle.MXFP4, qs)[0, 0]
    strong = np.clip(q.sum(0), -6, 6).astype(np.float32)       # aligned with every head
    g = np.random.default_rng(14)
    blk = (strong[None] * (1 + 0.01 * g.standard_normal((1500, 128)))).astype(np.float32)
    kcs, kss = oracle.encode(blk, oracle.MXFP4)
    kc[0, 20000:21500] = kcs
    ks[0, 20000:21500] = kss
    gi = check(qc, qs, w, kc, ks, np.array([[30000]], np.int32), 1024, 8, 128, oracle.MXFP4)
    assert ((gi[0, 0] >= 20000) & (gi[0, 0] < 21500)).sum() == 1024


def test_run_twice_and_batch_invariant():
    qc, qs, w, kc, ks = mx_inputs(15, 3, 1, 8, 128, 20000)
    n = np.array([[20000], [19000], [12345]], np.int32)
    a, sa = gpu_topk(qc, qs, w, kc, ks, n, 512, 8, 128)
    b, sb = gpu_topk(qc, qs, w, kc, ks, n, 512, 8, 128)
    assert np.array_equal(a, b) and np.array_equal(sa.view(np.uint64), sb.view(np.uint64))
    one, _ = gpu_topk(qc[1:2], qs[1:2], w[1:2], kc[1:2], ks[1:2], n[1:2], 512, 8, 128)
    assert np.array_equal(one[0], a[1])
