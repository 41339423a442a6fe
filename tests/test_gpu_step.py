"""lca_decode_step gives the bytes of lca_compress_batch, lca_lightning_index_topk
and lca_attend_batch issued in that order: with the compress jobs and the HCA
attention running inside the indexer's scan launch (the scan workgroup and the
attention split that read a row the step compresses compute it themselves;
FP8 entries, one query row per sequence; bf16 entries, two rows per sequence
so that two rows share a scan wavefront),
with an indexer that has no scan (a short cache: the unfused order), with
rows written by the step's own compress jobs that decide its results, and
captured in a graph.  Inputs are seeded N(0, 1)."""
import math

import pytest
import torch

import long_context_attention_13_amd as lca
from gpu_util import dev, empty_ws

pytestmark = pytest.mark.gpu


class Step:
    def __init__(self, seed, kv_dt=lca.FP8E4M3, Tq=1, N=40000, N2=320, k=512, B=2, Hq=64, D=128, H_I=8, W=128):
        d = dev()
        g = torch.Generator(device=d)
        g.manual_seed(seed)
        rn = lambda *s: torch.randn(*s, generator=g, device=d)
        i32 = lambda v: torch.full((B,), v, dtype=torch.int32, device=d)
        i64 = lambda v: torch.full((B,), v, dtype=torch.int64, device=d)
        zb = torch.zeros(1, device=d)

        def cache(rows, dim, dt):
            if dt == lca.BF16:
                return rn(B, rows, dim).to(torch.bfloat16), None
            dst = torch.empty(B, rows, dim if dt == lca.FP8E4M3 else dim // 2, dtype=torch.uint8, device=d)
            sc = torch.empty(B, rows, dim // 64 if dt == lca.FP8E4M3 else dim // 32,
                             dtype=torch.float32 if dt == lca.FP8E4M3 else torch.uint8, device=d)
            lca.csa_compress(rn(B, rows, dim), torch.zeros(B, rows, device=d), zb, 1, i32(0), i32(rows), i64(0), rows,
                             dst, dt, sc)
            return dst, sc

        self.ent, self.ent_sc = cache(N, D, kv_dt)
        self.key, self.key_sc = cache(N, 128, lca.MXFP4)
        self.hca, self.hca_sc = cache(N2, D, kv_dt)
        qi32 = rn(B, Tq * H_I, 128)
        self.qi = torch.empty(B, Tq, H_I, 64, dtype=torch.uint8, device=d)
        self.qi_sc = torch.empty(B, Tq, H_I, 4, dtype=torch.uint8, device=d)
        lca.csa_compress(qi32, torch.zeros(B, Tq * H_I, device=d), zb, 1, i32(0), i32(Tq * H_I), i64(0), Tq * H_I,
                         self.qi.view(B, Tq * H_I, 64), lca.MXFP4, self.qi_sc.view(B, Tq * H_I, 4))
        self.w = torch.rand(B, Tq, H_I, generator=g, device=d)
        self.n_csa = torch.tensor([[N - t for t in range(Tq - 1, -1, -1)], [N - 777 - t for t in range(Tq - 1, -1, -1)]],
                                  dtype=torch.int32, device=d)
        self.n_hca = torch.tensor([[N2] * Tq, [N2 - 5] * Tq], dtype=torch.int32, device=d)
        self.win = rn(B, 2 * W, D).to(torch.bfloat16)
        self.win_keys = rn(B, 2 * W, 128).to(torch.bfloat16)
        self.wb = torch.stack([torch.arange(Tq, device=d)] * B).to(torch.int32)
        self.wl = torch.full((B, Tq), W, dtype=torch.int32, device=d)
        self.q_csa = rn(B, Tq, Hq, D).to(torch.bfloat16)
        self.q_hca = rn(B, Tq, Hq, D).to(torch.bfloat16)
        self.sink = rn(Hq)
        gate, gate_i, gate_h = rn(B, 2 * W), rn(B, 2 * W), rn(B, 2 * W)
        bias4, bias128 = rn(4), rn(128)
        tau = 1 / math.sqrt(D)
        self.idx = torch.empty(B, Tq, k, dtype=torch.int32, device=d)
        self.out_csa = torch.empty(B, Tq, Hq, D, dtype=torch.bfloat16, device=d)
        self.out_hca = torch.empty(B, Tq, Hq, D, dtype=torch.bfloat16, device=d)
        self.lse_csa = torch.empty(B, Tq, Hq, device=d)
        self.lse_hca = torch.empty(B, Tq, Hq, device=d)
        ws_i = empty_ws(lca.index_topk_ws(B, Tq, H_I, 128, N, k))
        ws_c = empty_ws(lca.attend_ws(B, Tq, Hq, D, k, 2 * W))
        ws_h = empty_ws(lca.attend_ws(B, Tq, Hq, D, N2, 2 * W))
        ent_dt = lca.FP8E4M3 if kv_dt == lca.FP8E4M3 else lca.BF16
        self.cjobs = [lca.compress_job(self.win, gate, bias4, 4, i32(W - 4), i32(1), i64(N - 1), 1, self.ent, ent_dt,
                                       self.ent_sc),
                      lca.compress_job(self.win_keys, gate_i, bias4, 4, i32(W - 4), i32(1), i64(N - 1), 1, self.key,
                                       lca.MXFP4, self.key_sc),
                      lca.compress_job(self.win, gate_h, bias128, 128, i32(0), i32(1), i64(N2 - 1), 1, self.hca, ent_dt,
                                       self.hca_sc)]
        self.ijob = lca.index_job(self.qi, self.qi_sc, self.w, self.key, self.key_sc, self.n_csa, k, self.idx, ws_i)
        self.ajobs = [lca.attend_job(True, self.q_csa, self.ent, self.ent_sc, self.idx, self.win, self.wb, self.wl,
                                     self.sink, tau, self.out_csa, self.lse_csa, ws_c),
                      lca.attend_job(False, self.q_hca, self.hca, self.hca_sc, self.n_hca, self.win, self.wb, self.wl,
                                     self.sink, tau, self.out_hca, self.lse_hca, ws_h)]
        self.k = k

    def outputs(self):
        ts = [self.ent, self.key, self.key_sc, self.hca, self.idx, self.out_csa, self.out_hca, self.lse_csa,
              self.lse_hca]
        ts += [t for t in (self.ent_sc, self.hca_sc) if t is not None]
        return [t.clone() for t in ts]

    def clobber(self):
        for t in (self.idx, self.out_csa, self.out_hca, self.lse_csa, self.lse_hca):
            t.zero_()

    def three_calls(self):
        J = self.ijob
        lca.compress_batch(self.cjobs)
        lca.load().lca_lightning_index_topk(J.qi, J.qi_dt, J.qi_scale, J.w, J.ki, J.ki_dt, J.ki_scale, J.n_elig, J.B,
                                            J.Tq, J.H_I, J.d_I, J.N_cap, J.k, J.idx_out, J.score_out, J.ws,
                                            J.ws_bytes, lca._stream(None))
        lca.attend_batch(self.ajobs)

    def step(self):
        lca.decode_step(self.cjobs, self.ijob, self.ajobs)


@pytest.mark.parametrize("kv_dt,Tq,N", [(lca.FP8E4M3, 1, 40000), (lca.BF16, 2, 40000), (lca.FP8E4M3, 1, 6000)])
def test_step_equals_three_calls(kv_dt, Tq, N):
    st = Step(700 + Tq + N % 7, kv_dt, Tq, N)
    st.three_calls()
    torch.cuda.synchronize()
    ref = st.outputs()
    assert int((ref[4] >= 0).sum()) == 2 * Tq * st.k
    st.clobber()
    st.step()
    torch.cuda.synchronize()
    for i, (a, b) in enumerate(zip(st.outputs(), ref)):
        assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), f"output {i}"


def test_step_graph_replays():
    st = Step(811)
    st.step()
    torch.cuda.synchronize()
    ref = st.outputs()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        st.step()
    torch.cuda.synchronize()
    x = torch.randn(1 << 20, device=dev())
    for rep in range(3):
        st.clobber()
        x.mul_(0.5).add_(1.0)
        g.replay()
        torch.cuda.synchronize()
        for i, (a, b) in enumerate(zip(st.outputs(), ref)):
            assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), f"replay {rep}: output {i}"


@pytest.mark.parametrize("kv_dt,Tq", [(lca.FP8E4M3, 1), (lca.BF16, 2)])
def test_step_reads_rows_written_in_the_step(kv_dt, Tq):
    """The newest indexer key row and HCA row are written by the step's own
    compress jobs: before the step they hold zeros, and their raw tokens are
    scaled so that the new rows decide the results (the key row is selected,
    the HCA row dominates the HCA attention).  A scan or HCA split that read
    the rows before they were written would differ from the three calls.
    With two query rows per sequence (bf16 entries) the rows share each scan
    wavefront, and only the second row sees the new key row."""
    st = Step(919 + Tq, kv_dt, Tq)
    N, N2, W = st.key.shape[1], st.hca.shape[1], 128
    st.win_keys[:, W - 4:W] *= 40.0
    st.win[:, :128] *= 8.0

    def stale():
        st.key[:, N - 1].zero_()
        st.key_sc[:, N - 1].fill_(127)
        st.hca[:, N2 - 1].zero_()
        if st.hca_sc is not None:
            st.hca_sc[:, N2 - 1].fill_(1.0)

    stale()
    st.three_calls()
    torch.cuda.synchronize()
    ref = st.outputs()
    assert bool((ref[4][0, Tq - 1] == N - 1).any()), "the new key row is selected"
    stale()
    st.clobber()
    for rep in range(2):
        st.step()
        torch.cuda.synchronize()
        for i, (a, b) in enumerate(zip(st.outputs(), ref)):
            assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), f"step {rep}: output {i}"
        stale()
        st.clobber()


def test_step_compress_into_key_cache_at_an_offset():
    """A compress job that writes into the indexer's key cache through an
    offset pointer (a different row layout: sequence b's row r lands at key
    row b * (N - 4) + r + 4) is not run beside the scan, which reads those
    rows: the step still gives the bytes of the three calls in order.  The
    raw keys of the block are scaled so that the rows it writes are selected."""
    st = Step(933)
    N = st.key.shape[1]
    kv = st.key.view(-1)[4 * 64:].view(st.key.shape[0] * N - 4, 64)[: 2 * (N - 4)].view(2, N - 4, 64)
    ks = st.key_sc.view(-1)[4 * 4:].view(st.key.shape[0] * N - 4, 4)[: 2 * (N - 4)].view(2, N - 4, 4)
    d = dev()
    st.win_keys[:, 128 - 4:128] *= 40.0
    st.cjobs[1] = lca.compress_job(st.win_keys, torch.randn(2, 256, device=d), torch.randn(4, device=d), 4,
                                   torch.full((2,), 124, dtype=torch.int32, device=d),
                                   torch.ones(2, dtype=torch.int32, device=d),
                                   torch.tensor([N - 40, N - 90], dtype=torch.int64, device=d), 1, kv, lca.MXFP4, ks)
    key0, ksc0 = st.key.clone(), st.key_sc.clone()
    st.three_calls()
    torch.cuda.synchronize()
    ref = st.outputs()
    assert bool((ref[4][0, 0] == N - 36).any()), "a row the offset job wrote is selected"
    st.key.copy_(key0)
    st.key_sc.copy_(ksc0)
    st.clobber()
    st.step()
    torch.cuda.synchronize()
    for i, (a, b) in enumerate(zip(st.outputs(), ref)):
        assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), f"output {i}"
