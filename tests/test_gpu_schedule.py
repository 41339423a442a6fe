"""The attention layers of the 61-layer V4-Pro model and its MTP block as a
decode loop (layers 0-1 HCA, layers 2..60 alternating CSA and HCA, then the
MTP block with window-only attention).  Per layer and step: one
lca_decode_append (the layer's raw-token rings) and one lca_decode_step (CSA:
two compress jobs, the indexer, the sparse attention; HCA: one compress job and
the dense attention, no indexer; MTP block: the window-only attention job).

Two sequences near 40K tokens, five steps; the first step completes a 4-block
and a 128-block in every layer.  At every step every layer's index set and
scores are bit-exact and its attention is within rtol 2e-2 of the oracle on
caches the host assembles (oracle codecs, oracle pooling of the host-held
token history) and windows cut from that history; the captured schedule step
replayed five times ends with the eager loop's bytes, issued per layer as
the two calls and as one lca_decode_loop_step.  lca_window_attend is
also checked on its own against the oracle on ragged windows."""
import math

import numpy as np
import pytest
import torch

import long_context_attention_13_amd as lca
import oracle
import synth
from gpu_util import assert_lse_close, assert_rows_close, dev, empty_ws, to_dev, to_host

pytestmark = [pytest.mark.gpu, pytest.mark.timeout(900)]

B, Hq, D, H_I, d_I, W = 2, 64, 128, 8, 128, 128
TAU = 1.0 / math.sqrt(D)
HIST = 128                       # raw tokens before the loop kept by the host


def bf16(a):
    return oracle.encode(np.asarray(a, np.float32), oracle.BF16)[0]


class Stream:
    """Host history of one raw-token stream (block m, ring R, window W)."""

    def __init__(self, g, L0, S, dim, m, R, W_, exact=False):
        self.L0, self.dim, self.m, self.R, self.W = L0, dim, m, R, W_
        self.base = [max(0, l - HIST) for l in L0]
        n = [l + S - b0 for l, b0 in zip(L0, self.base)]
        if exact:           # multiples of 1/16 with equal gates: fp32 pooling is exact
            self.x = [bf16(g.integers(-48, 49, (t, dim)) / 16.0) for t in n]
            self.gate = [np.zeros(t, np.float32) for t in n]
            self.bias = np.zeros(max(m, 1), np.float32)
        else:
            self.x = [bf16(g.standard_normal((t, dim))) for t in n]
            self.gate = [g.standard_normal(t).astype(np.float32) for t in n]
            self.bias = (g.standard_normal(max(m, 1)) * 0.1).astype(np.float32)
        self.rows = {}
        if m > 0:
            for b in range(B):
                for e in range(L0[b] + 1, L0[b] + S + 1):
                    if e % m == 0:
                        t0 = e - m - self.base[b]
                        xd = oracle.decode(self.x[b][t0:t0 + m], oracle.BF16)
                        self.rows[(b, e // m - 1)] = oracle.pool(xd, self.gate[b][t0:t0 + m], self.bias, m)[0]

    def tok(self, b, p):
        return self.x[b][p - self.base[b]]

    def new(self, i):
        return (np.stack([self.tok(b, self.L0[b] + i) for b in range(B)]),
                np.array([self.gate[b][self.L0[b] + i - self.base[b]] for b in range(B)], np.float32))

    def ring0(self):
        ring = np.zeros((B, 2 * self.R, self.dim), np.uint16)
        gring = np.zeros((B, 2 * self.R), np.float32)
        for b in range(B):
            for p in range(max(self.base[b], self.L0[b] - self.R), self.L0[b]):
                r = p % self.R
                ring[b, r] = ring[b, r + self.R] = self.tok(b, p)
                gring[b, r] = gring[b, r + self.R] = self.gate[b][p - self.base[b]]
        return ring, gring

    def window(self, L):
        win = np.zeros((B, W, self.dim), np.uint16)
        wl = np.zeros((B, 1), np.int32)
        for b in range(B):
            n = min(L[b], W)
            for j in range(n):
                win[b, j] = self.tok(b, L[b] - n + j)
            wl[b, 0] = n
        return win, wl

    def cache_at(self, codes, scales, dt, L):
        codes, scales = codes.copy(), scales.copy()
        for (b, r), v in self.rows.items():
            if (r + 1) * self.m <= L[b]:
                rc, rs = oracle.encode(v.astype(np.float32)[None], dt)
                codes[b, r], scales[b, r] = rc[0], rs[0]
        return codes, scales


class Layer:
    """Host data of one attention layer of the schedule."""

    def __init__(self, kind, seed, L0, S, N, N2, k):
        g = np.random.default_rng(seed)
        self.kind, self.S, self.k = kind, S, k
        if kind == "csa":
            self.kv = Stream(g, L0, S, D, 4, 128, W)
            self.key = Stream(g, L0, S, d_I, 4, 6, 0, exact=True)
            self.ent, self.ent_sc = oracle.encode(g.standard_normal((B, N, D)).astype(np.float32), oracle.FP8E4M3)
            self.kc, self.ks = oracle.encode(g.standard_normal((B, N, d_I)).astype(np.float32), oracle.MXFP4)
            self.qc, self.qs = oracle.encode(g.standard_normal((S, B, 1, H_I, d_I)).astype(np.float32),
                                             oracle.MXFP4)
            self.w = g.random((S, B, 1, H_I)).astype(np.float32)
        elif kind == "hca":
            self.kv = Stream(g, L0, S, D, 128, 128, W)
            self.ent, self.ent_sc = oracle.encode(g.standard_normal((B, N2, D)).astype(np.float32), oracle.FP8E4M3)
        else:
            self.kv = Stream(g, L0, S, D, 0, 128, W)
        self.q = bf16(g.standard_normal((S, B, 1, Hq, D)))
        self.sink = g.standard_normal(Hq).astype(np.float32)

    def streams(self):
        return [self.kv, self.key] if self.kind == "csa" else [self.kv]


class LayerDev:
    """Device buffers and prebuilt jobs of one layer; issue() = append + step."""

    def __init__(self, ly: Layer):
        d = dev()
        self.ly = ly
        i32 = lambda *s: torch.zeros(*s, dtype=torch.int32, device=d)
        self.st = []
        for s in ly.streams():
            ring, gring = s.ring0()
            t = dict(ring=to_dev(ring), len=torch.tensor(s.L0, dtype=torch.int64, device=d),
                     xn=torch.zeros(B, s.dim, dtype=torch.bfloat16, device=d),
                     all_x=to_dev(np.stack([s.new(i)[0] for i in range(ly.S)])))
            if s.m > 0:
                t.update(gring=to_dev(gring), gn=torch.zeros(B, device=d), tok0=i32(B), nblk=i32(B),
                         row0=torch.zeros(B, dtype=torch.int64, device=d), bias=to_dev(s.bias),
                         all_g=to_dev(np.stack([s.new(i)[1] for i in range(ly.S)])))
            self.st.append(t)
        kv = self.st[0]
        self.n, self.wb, self.wl = i32(B, 1), i32(B, 1), i32(B, 1)
        apps = []
        for s, t in zip(ly.streams(), self.st):
            kw = dict(m=s.m, W=s.W)
            if s.m > 0:
                kw.update(g_new=t["gn"], gring=t["gring"], x_tok0=t["tok0"], nblk=t["nblk"], dst_row0=t["row0"])
            if t is kv:
                kw.update(win_begin=self.wb, win_len=self.wl)
                if s.m > 0:
                    kw.update(n_elig=self.n)
            apps.append(lca.append_job(t["xn"], t["ring"], t["len"], **kw))
        self.appends = (lca.AppendJob * len(apps))(*apps)
        self._apps = apps
        self.q = torch.zeros(B, 1, Hq, D, dtype=torch.bfloat16, device=d)
        self.all_q = to_dev(ly.q)
        self.sink = to_dev(ly.sink)
        self.out = torch.zeros(B, 1, Hq, D, dtype=torch.bfloat16, device=d)
        self.lse = torch.zeros(B, 1, Hq, device=d)
        self.cjobs, self.ijob, self.idx, self.score = [], None, None, None
        if ly.kind == "csa":
            key = self.st[1]
            self.ent, self.ent_sc = to_dev(ly.ent), to_dev(ly.ent_sc)
            self.kc, self.ks = to_dev(ly.kc), to_dev(ly.ks)
            self.cjobs = [lca.compress_job(kv["ring"], kv["gring"], kv["bias"], 4, kv["tok0"], kv["nblk"], kv["row0"],
                                           1, self.ent, lca.FP8E4M3, self.ent_sc),
                          lca.compress_job(key["ring"], key["gring"], key["bias"], 4, key["tok0"], key["nblk"],
                                           key["row0"], 1, self.kc, lca.MXFP4, self.ks)]
            self.qi = torch.zeros(B, 1, H_I, d_I // 2, dtype=torch.uint8, device=d)
            self.qi_sc = torch.zeros(B, 1, H_I, d_I // 32, dtype=torch.uint8, device=d)
            self.w = torch.zeros(B, 1, H_I, device=d)
            self.all_qi, self.all_qs, self.all_w = to_dev(ly.qc), to_dev(ly.qs), to_dev(ly.w)
            self.idx = torch.zeros(B, 1, ly.k, dtype=torch.int32, device=d)
            self.score = torch.zeros(B, 1, ly.k, dtype=torch.float64, device=d)
            ws_i = empty_ws(lca.index_topk_ws(B, 1, H_I, d_I, self.kc.shape[1], ly.k))
            self.ijob = lca.index_job(self.qi, self.qi_sc, self.w, self.kc, self.ks, self.n, ly.k, self.idx, ws_i,
                                      score_out=self.score)
            ws = empty_ws(lca.attend_ws(B, 1, Hq, D, ly.k, 256))
            self.ajob = lca.attend_job(True, self.q, self.ent, self.ent_sc, self.idx, kv["ring"], self.wb, self.wl,
                                       self.sink, TAU, self.out, self.lse, ws)
        elif ly.kind == "hca":
            self.ent, self.ent_sc = to_dev(ly.ent), to_dev(ly.ent_sc)
            self.cjobs = [lca.compress_job(kv["ring"], kv["gring"], kv["bias"], 128, kv["tok0"], kv["nblk"],
                                           kv["row0"], 1, self.ent, lca.FP8E4M3, self.ent_sc)]
            ws = empty_ws(lca.attend_ws(B, 1, Hq, D, self.ent.shape[1], 256))
            self.ajob = lca.attend_job(False, self.q, self.ent, self.ent_sc, self.n, kv["ring"], self.wb, self.wl,
                                       self.sink, TAU, self.out, self.lse, ws)
        else:
            ws = empty_ws(lca.attend_ws(B, 1, Hq, D, 0, 256))
            self.ajob = lca.attend_job(True, self.q, None, None, None, kv["ring"], self.wb, self.wl, self.sink, TAU,
                                       self.out, self.lse, ws)

    def load_inputs(self, i):
        for t in self.st:
            t["xn"].copy_(t["all_x"][i])
            if "gn" in t:
                t["gn"].copy_(t["all_g"][i])
        self.q.copy_(self.all_q[i])
        if self.ly.kind == "csa":
            self.qi.copy_(self.all_qi[i])
            self.qi_sc.copy_(self.all_qs[i])
            self.w.copy_(self.all_w[i])

    def issue(self, fused=False):
        if fused:
            lca.decode_loop_step(self.appends, self.cjobs, self.ijob, [self.ajob])
        else:
            lca.decode_append(self.appends)
            lca.decode_step(self.cjobs, self.ijob, [self.ajob])

    def state(self):
        ts = [self.out, self.lse] + [t["ring"] for t in self.st] + [t["len"] for t in self.st]
        if self.ly.kind != "window":
            ts += [self.ent, self.ent_sc]
        if self.ly.kind == "csa":
            ts += [self.kc, self.ks, self.idx, self.score]
        return [t.clone() for t in ts]


def check_layer(ly: Layer, dv: LayerDev, i, L, what):
    win, wl = ly.kv.window(L)
    wb0 = np.zeros((B, 1), np.int32)
    q = oracle.decode(ly.q[i], oracle.BF16)
    if ly.kind == "csa":
        ent, ent_sc = ly.kv.cache_at(ly.ent, ly.ent_sc, oracle.FP8E4M3, L)
        kc, ks = ly.key.cache_at(ly.kc, ly.ks, oracle.MXFP4, L)
        n = np.array(L, np.int32)[:, None] // 4
        ri, rs = oracle.index_topk(oracle.decode(ly.qc[i], oracle.MXFP4, ly.qs[i]), ly.w[i], kc, oracle.MXFP4, ks, n,
                                   ly.k)
        assert np.array_equal(to_host(dv.idx), ri), f"{what}: index set"
        assert np.array_equal(to_host(dv.score).view(np.uint64), rs.view(np.uint64)), f"{what}: index scores"
        ro, rl = oracle.attend(q, ent, oracle.FP8E4M3, ent_sc, ri, None, win, oracle.BF16, wb0, wl, ly.sink, TAU)
    elif ly.kind == "hca":
        ent, ent_sc = ly.kv.cache_at(ly.ent, ly.ent_sc, oracle.FP8E4M3, L)
        n = np.array(L, np.int32)[:, None] // 128
        ro, rl = oracle.attend(q, ent, oracle.FP8E4M3, ent_sc, None, n, win, oracle.BF16, wb0, wl, ly.sink, TAU)
    else:
        empty = np.zeros((B, 0, D), np.uint16)
        ro, rl = oracle.attend(q, empty, oracle.BF16, None, np.zeros((B, 1, 0), np.int32), None, win, oracle.BF16,
                               wb0, wl, ly.sink, TAU)
    assert_rows_close(oracle.decode(to_host(dv.out), oracle.BF16), ro, 2e-2, f"{what}: out")
    assert_lse_close(to_host(dv.lse), rl, 2e-2, f"{what}: lse")


def test_v4_pro_schedule_loop():
    L0, S, N, N2, k = [40959, 36991], 5, 10304, 322, 256
    kinds = synth.v4_pro_layer_kinds()
    layers = [Layer(kd, 500 + j, L0, S, N, N2, k) for j, kd in enumerate(kinds)]
    devs = [LayerDev(ly) for ly in layers]
    for i in range(S):
        for dv in devs:
            dv.load_inputs(i)
            dv.issue()
        torch.cuda.synchronize()
        L = [l + i + 1 for l in L0]
        for j, (ly, dv) in enumerate(zip(layers, devs)):
            check_layer(ly, dv, i, L, f"step {i} layer {j} ({ly.kind})")
    eager = [dv.state() for dv in devs]

    for fused in (False, True):
        devs2 = [LayerDev(ly) for ly in layers]
        for dv in devs2:
            dv.load_inputs(0)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for dv in devs2:
                dv.issue(fused)
        torch.cuda.synchronize()
        for i in range(S):
            for dv in devs2:
                dv.load_inputs(i)
            graph.replay()
        torch.cuda.synchronize()
        for j, dv in enumerate(devs2):
            for a, b in zip(dv.state(), eager[j]):
                assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), f"graph (fused={fused}): layer {j}"
        del graph, devs2


@pytest.mark.parametrize("Hq_,q_dt", [(64, "bf16"), (16, "f32")])
def test_window_attend_ragged(Hq_, q_dt):
    """Window-only attention: windows of every length 0..W at any offset in a
    buffer, several query rows per sequence."""
    g = np.random.default_rng(77 + Hq_)
    Bq, Tq, W_buf = 3, 5, 300
    win = g.standard_normal((Bq, W_buf, D)).astype(np.float32)
    q = g.standard_normal((Bq, Tq, Hq_, D)).astype(np.float32)
    wl = g.integers(0, W + 1, (Bq, Tq)).astype(np.int32)
    wl[0, 0], wl[1, 1] = 0, W
    wb = np.array([[g.integers(0, W_buf - n + 1) for n in row] for row in wl], np.int32)
    sink = g.standard_normal(Hq_).astype(np.float32)
    if q_dt == "bf16":
        qb, winb = bf16(q), bf16(win)
        qd, wdt = oracle.decode(qb, oracle.BF16), oracle.BF16
        qt, wt = to_dev(qb), to_dev(winb)
        rtol = 2e-2
    else:
        qd, winb, wdt = q.astype(np.float64), win, oracle.F32
        qt, wt = to_dev(q), to_dev(win)
        rtol = 1e-4
    out = torch.zeros(Bq, Tq, Hq_, D, dtype=torch.float32, device=dev())
    lse = torch.zeros(Bq, Tq, Hq_, device=dev())
    ws = empty_ws(lca.attend_ws(Bq, Tq, Hq_, D, 0, W_buf))
    lca.window_attend(qt, wt, to_dev(wb), to_dev(wl), to_dev(sink), TAU, out, lse, ws)
    torch.cuda.synchronize()
    empty = np.zeros((Bq, 0, D), np.float32)
    ro, rl = oracle.attend(qd, empty, oracle.F32, None, np.zeros((Bq, Tq, 0), np.int32), None, winb, wdt, wb, wl,
                           sink, TAU)
    assert_rows_close(to_host(out), ro, rtol, "out")
    assert_lse_close(to_host(lse), rl, rtol, "lse")
