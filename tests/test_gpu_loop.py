"""A decode loop of the CSA+HCA layer pair: per step, lca_decode_append puts
each sequence's new raw token into three doubled rings (CSA KV, indexer keys,
HCA KV; token t at rows t % R and t % R + R) and derives the step's arguments,
then lca_decode_step compresses the blocks that just completed, runs the
indexer and both attentions.  The host keeps the whole token history and
checks:

- every step: the derived arguments (block flags, ring rows, cache rows,
  eligible counts, window rows) against the definitions, exactly;
- sampled steps: the top-k index set and its scores against the oracle's
  indexer, bit-exact, and both attentions against the oracle within rtol 2e-2,
  all on caches the host assembles itself (pre-loop rows encoded with the
  oracle's codecs, loop rows pooled by the oracle from the host history) and a
  window cut from the host history, not from the rings;
- the end: ring bytes, lengths, and every cache row the loop wrote (indexer
  keys bit-exact: their raw values are multiples of 1/16 with equal gates, so
  fp32 pooling is exact; FP8 rows a correct rounding of the oracle's pooling);
- the same loop captured once as a graph (append + step) and replayed with
  new inputs copied in before each replay ends with the eager loop's bytes,
  both as the two calls and as one lca_decode_loop_step (the appends inside
  the compress launch).

Two cases: long sequences (the indexer's chunked scan runs beside the HCA
attention) starting at different phases of the 4- and 128-token blocks, and
sequences that start empty (windows and caches fill up during the loop).
"""
import math

import numpy as np
import pytest
import torch

import long_context_attention_13_amd as lca
import oracle
from gpu_util import assert_lse_close, assert_rows_close, dev, empty_ws, to_dev, to_host

pytestmark = [pytest.mark.gpu, pytest.mark.timeout(600)]

B, Hq, D, H_I, d_I, W = 2, 64, 128, 8, 128, 128
M, M2 = 4, 128
R_CSA, R_KEY, R_HCA = 128, 6, 128          # R_KEY: not a multiple of 4, so blocks wrap into the second copy
TAU = 1.0 / math.sqrt(D)


class Loop:
    """Host history + device state of one loop case."""

    def __init__(self, seed, L0, S, N, N2, k):
        g = np.random.default_rng(seed)
        self.L0, self.S, self.N, self.N2, self.k = list(L0), S, N, N2, k
        self.base = [max(0, l - 128) for l in L0]
        n_tok = [l + S - b0 for l, b0 in zip(L0, self.base)]

        def bf16(a):
            return oracle.encode(a.astype(np.float32), oracle.BF16)[0]

        # raw token histories (bf16 bits) and gate logits, per sequence
        self.x = {"csa": [bf16(g.standard_normal((n, D))) for n in n_tok],
                  "key": [bf16(g.integers(-48, 49, (n, d_I)) / 16.0) for n in n_tok],
                  "hca": [bf16(g.standard_normal((n, D))) for n in n_tok]}
        self.gate = {"csa": [g.standard_normal(n).astype(np.float32) for n in n_tok],
                     "key": [np.zeros(n, np.float32) for n in n_tok],
                     "hca": [g.standard_normal(n).astype(np.float32) for n in n_tok]}
        self.bias = {"csa": (g.standard_normal(M) * 0.1).astype(np.float32), "key": np.zeros(M, np.float32),
                     "hca": (g.standard_normal(M2) * 0.1).astype(np.float32)}
        self.R = {"csa": R_CSA, "key": R_KEY, "hca": R_HCA}
        self.m = {"csa": M, "key": M, "hca": M2}
        # pre-loop caches (all rows N(0,1), oracle codecs)
        self.ent, self.ent_sc = oracle.encode(g.standard_normal((B, N, D)).astype(np.float32), oracle.FP8E4M3)
        self.key, self.key_sc = oracle.encode(g.standard_normal((B, N, d_I)).astype(np.float32), oracle.MXFP4)
        self.hca, self.hca_sc = oracle.encode(g.standard_normal((B, N2, D)).astype(np.float32), oracle.FP8E4M3)
        # per-step queries
        self.qc, self.qs = oracle.encode(g.standard_normal((S, B, 1, H_I, d_I)).astype(np.float32), oracle.MXFP4)
        self.w = g.random((S, B, 1, H_I)).astype(np.float32)
        self.q_csa = bf16(g.standard_normal((S, B, 1, Hq, D)))
        self.q_hca = bf16(g.standard_normal((S, B, 1, Hq, D)))
        self.sink_csa = g.standard_normal(Hq).astype(np.float32)
        self.sink_hca = g.standard_normal(Hq).astype(np.float32)
        # cache rows the loop writes, pooled by the oracle from the history
        self.rows = {"csa": {}, "key": {}, "hca": {}}
        for s in self.rows:
            m = self.m[s]
            for b in range(B):
                for e in range(L0[b] + 1, L0[b] + S + 1):
                    if e % m == 0:
                        t0 = e - m - self.base[b]
                        xd = oracle.decode(self.x[s][b][t0:t0 + m], oracle.BF16)
                        self.rows[s][(b, e // m - 1)] = oracle.pool(xd, self.gate[s][b][t0:t0 + m], self.bias[s], m)[0]

    def tok(self, s, b, p):
        return self.x[s][b][p - self.base[b]]

    def new_tokens(self, s, i):
        return np.stack([self.tok(s, b, self.L0[b] + i) for b in range(B)])

    def new_gates(self, s, i):
        return np.array([self.gate[s][b][self.L0[b] + i - self.base[b]] for b in range(B)], np.float32)

    def ring0(self, s):
        R, dim = self.R[s], self.x[s][0].shape[1]
        ring = np.zeros((B, 2 * R, dim), np.uint16)
        gring = np.zeros((B, 2 * R), np.float32)
        for b in range(B):
            for p in range(max(self.base[b], self.L0[b] - R), self.L0[b]):
                ring[b, p % R] = ring[b, p % R + R] = self.tok(s, b, p)
                gring[b, p % R] = gring[b, p % R + R] = self.gate[s][b][p - self.base[b]]
        return ring, gring

    def caches_at(self, L):
        """Host caches after the step that reaches lengths L."""
        out = []
        for s, c, sc, dt in (("csa", self.ent, self.ent_sc, oracle.FP8E4M3),
                             ("key", self.key, self.key_sc, oracle.MXFP4),
                             ("hca", self.hca, self.hca_sc, oracle.FP8E4M3)):
            c, sc = c.copy(), sc.copy()
            for (b, r), v in self.rows[s].items():
                if (r + 1) * self.m[s] <= L[b]:
                    rc, rs = oracle.encode(v.astype(np.float32)[None], dt)
                    c[b, r], sc[b, r] = rc[0], rs[0]
            out += [c, sc]
        return out

    def window(self, s, L):
        """[B, W, dim] bf16 bits of the last min(L, W) tokens (front-aligned) and their counts."""
        dim = self.x[s][0].shape[1]
        win = np.zeros((B, W, dim), np.uint16)
        wl = np.zeros((B, 1), np.int32)
        for b in range(B):
            n = min(L[b], W)
            for j in range(n):
                win[b, j] = self.tok(s, b, L[b] - n + j)
            wl[b, 0] = n
        return win, wl


class Device:
    """Device buffers and job arrays of the loop (append jobs + step jobs)."""

    def __init__(self, lp: Loop):
        d = dev()
        self.lp = lp
        i32 = lambda *s: torch.zeros(*s, dtype=torch.int32, device=d)
        self.ring, self.gring, self.len, self.xn, self.gn = {}, {}, {}, {}, {}
        for s in ("csa", "key", "hca"):
            ring, gring = lp.ring0(s)
            self.ring[s], self.gring[s] = to_dev(ring), to_dev(gring)
            self.len[s] = torch.tensor(lp.L0, dtype=torch.int64, device=d)
            self.xn[s] = torch.zeros(B, ring.shape[2], dtype=torch.bfloat16, device=d)
            self.gn[s] = torch.zeros(B, dtype=torch.float32, device=d)
        self.tok0 = {s: i32(B) for s in self.ring}
        self.nblk = {s: i32(B) for s in self.ring}
        self.row0 = {s: torch.zeros(B, dtype=torch.int64, device=d) for s in self.ring}
        self.n_csa, self.n_hca = i32(B, 1), i32(B, 1)
        self.wb_csa, self.wl_csa, self.wb_hca, self.wl_hca = i32(B, 1), i32(B, 1), i32(B, 1), i32(B, 1)
        self.ent, self.ent_sc = to_dev(lp.ent), to_dev(lp.ent_sc)
        self.key, self.key_sc = to_dev(lp.key), to_dev(lp.key_sc)
        self.hca, self.hca_sc = to_dev(lp.hca), to_dev(lp.hca_sc)
        self.bias = {s: to_dev(lp.bias[s]) for s in lp.bias}
        self.qi = torch.zeros(B, 1, H_I, d_I // 2, dtype=torch.uint8, device=d)
        self.qi_sc = torch.zeros(B, 1, H_I, d_I // 32, dtype=torch.uint8, device=d)
        self.w = torch.zeros(B, 1, H_I, dtype=torch.float32, device=d)
        self.q_csa = torch.zeros(B, 1, Hq, D, dtype=torch.bfloat16, device=d)
        self.q_hca = torch.zeros(B, 1, Hq, D, dtype=torch.bfloat16, device=d)
        self.sink_csa, self.sink_hca = to_dev(lp.sink_csa), to_dev(lp.sink_hca)
        # every step's inputs, resident; copied into the fixed buffers before the step
        self.all_x = {s: to_dev(np.stack([lp.new_tokens(s, i) for i in range(lp.S)])) for s in self.ring}
        self.all_g = {s: to_dev(np.stack([lp.new_gates(s, i) for i in range(lp.S)])) for s in self.ring}
        self.all_qi, self.all_qs, self.all_w = to_dev(lp.qc), to_dev(lp.qs), to_dev(lp.w)
        self.all_qc, self.all_qh = to_dev(lp.q_csa), to_dev(lp.q_hca)
        k, N, N2 = lp.k, lp.N, lp.N2
        self.idx = torch.zeros(B, 1, k, dtype=torch.int32, device=d)
        self.score = torch.zeros(B, 1, k, dtype=torch.float64, device=d)
        self.out_csa = torch.zeros(B, 1, Hq, D, dtype=torch.bfloat16, device=d)
        self.out_hca = torch.zeros(B, 1, Hq, D, dtype=torch.bfloat16, device=d)
        self.lse_csa = torch.zeros(B, 1, Hq, device=d)
        self.lse_hca = torch.zeros(B, 1, Hq, device=d)
        ws_i = empty_ws(lca.index_topk_ws(B, 1, H_I, d_I, N, k))
        ws_c = empty_ws(lca.attend_ws(B, 1, Hq, D, k, 2 * R_CSA))
        ws_h = empty_ws(lca.attend_ws(B, 1, Hq, D, N2, 2 * R_HCA))
        A = lambda s, **kw: lca.append_job(self.xn[s], self.ring[s], self.len[s], m=lp.m[s], g_new=self.gn[s],
                                           gring=self.gring[s], x_tok0=self.tok0[s], nblk=self.nblk[s],
                                           dst_row0=self.row0[s], **kw)
        self.appends = [A("csa", W=W, n_elig=self.n_csa, win_begin=self.wb_csa, win_len=self.wl_csa),
                        A("key"),
                        A("hca", W=W, n_elig=self.n_hca, win_begin=self.wb_hca, win_len=self.wl_hca)]
        C = lambda s, dst, dt, sc: lca.compress_job(self.ring[s], self.gring[s], self.bias[s], lp.m[s], self.tok0[s],
                                                    self.nblk[s], self.row0[s], 1, dst, dt, sc)
        self.cjobs = [C("csa", self.ent, lca.FP8E4M3, self.ent_sc), C("key", self.key, lca.MXFP4, self.key_sc),
                      C("hca", self.hca, lca.FP8E4M3, self.hca_sc)]
        self.ijob = lca.index_job(self.qi, self.qi_sc, self.w, self.key, self.key_sc, self.n_csa, k, self.idx, ws_i,
                                  score_out=self.score)
        self.ajobs = [lca.attend_job(True, self.q_csa, self.ent, self.ent_sc, self.idx, self.ring["csa"], self.wb_csa,
                                     self.wl_csa, self.sink_csa, TAU, self.out_csa, self.lse_csa, ws_c),
                      lca.attend_job(False, self.q_hca, self.hca, self.hca_sc, self.n_hca, self.ring["hca"],
                                     self.wb_hca, self.wl_hca, self.sink_hca, TAU, self.out_hca, self.lse_hca, ws_h)]

    def load_inputs(self, i):
        for s in self.ring:
            self.xn[s].copy_(self.all_x[s][i])
            self.gn[s].copy_(self.all_g[s][i])
        self.qi.copy_(self.all_qi[i])
        self.qi_sc.copy_(self.all_qs[i])
        self.w.copy_(self.all_w[i])
        self.q_csa.copy_(self.all_qc[i])
        self.q_hca.copy_(self.all_qh[i])

    def step(self, fused=False):
        if fused:
            lca.decode_loop_step(self.appends, self.cjobs, self.ijob, self.ajobs)
        else:
            lca.decode_append(self.appends)
            lca.decode_step(self.cjobs, self.ijob, self.ajobs)

    def state(self):
        ts = [self.ent, self.ent_sc, self.key, self.key_sc, self.hca, self.hca_sc, self.idx, self.score,
              self.out_csa, self.out_hca, self.lse_csa, self.lse_hca]
        ts += [self.ring[s] for s in self.ring] + [self.gring[s] for s in self.ring] + [self.len[s] for s in self.ring]
        return [t.clone() for t in ts]


def expected_args(lp, L):
    """The step arguments that the definitions give for lengths L (after the append)."""
    e = {}
    for s in ("csa", "key", "hca"):
        m, R = lp.m[s], lp.R[s]
        e[s + ".nblk"] = [int(l % m == 0) for l in L]
        e[s + ".tok0"] = [(l - m) % R if l >= m else 0 for l in L]
        e[s + ".row0"] = [max(l // m - 1, 0) for l in L]
    e["n_csa"] = [l // M for l in L]
    e["n_hca"] = [l // M2 for l in L]
    e["wl"] = [min(l, W) for l in L]
    e["wb_csa"] = [(l - min(l, W)) % R_CSA for l in L]
    e["wb_hca"] = [(l - min(l, W)) % R_HCA for l in L]
    return e


def check_against_oracle(lp, dv, i, L):
    ent, ent_sc, key, key_sc, hca, hca_sc = lp.caches_at(L)
    qd = oracle.decode(lp.qc[i], oracle.MXFP4, lp.qs[i])
    n_csa = np.array(L, np.int32)[:, None] // M
    n_hca = np.array(L, np.int32)[:, None] // M2
    ri, rs = oracle.index_topk(qd, lp.w[i], key, oracle.MXFP4, key_sc, n_csa, lp.k)
    gi, gs = to_host(dv.idx), to_host(dv.score)
    assert np.array_equal(gi, ri), f"step {i}: index set"
    assert np.array_equal(gs.view(np.uint64), rs.view(np.uint64)), f"step {i}: index scores"
    wb0 = np.zeros((B, 1), np.int32)
    for name, q, kv, sc, sel, n, s, sink, out, lse in (
            ("csa", lp.q_csa[i], ent, ent_sc, ri, None, "csa", lp.sink_csa, dv.out_csa, dv.lse_csa),
            ("hca", lp.q_hca[i], hca, hca_sc, None, n_hca, "hca", lp.sink_hca, dv.out_hca, dv.lse_hca)):
        win, wl = lp.window(s, L)
        ro, rl = oracle.attend(oracle.decode(q, oracle.BF16), kv, oracle.FP8E4M3, sc, sel, n, win, oracle.BF16,
                               wb0, wl, sink, TAU)
        o = oracle.decode(to_host(out), oracle.BF16)
        assert_rows_close(o, ro, 2e-2, f"step {i}: {name} out")
        assert_lse_close(to_host(lse), rl, 2e-2, f"step {i}: {name} lse")


def check_final_state(lp, dv):
    L = [l + lp.S for l in lp.L0]
    for s in ("csa", "key", "hca"):
        assert to_host(dv.len[s]).tolist() == L, s
        R = lp.R[s]
        ring, gring = to_host(dv.ring[s]), to_host(dv.gring[s])
        for b in range(B):
            for p in range(max(0, L[b] - R), L[b]):
                for row in (p % R, p % R + R):
                    assert np.array_equal(ring[b, row], lp.tok(s, b, p)), (s, b, p, row)
                    assert gring[b, row] == lp.gate[s][b][p - lp.base[b]], (s, b, p, row)
    # indexer key rows: bit-exact (exact pooling)
    key, key_sc = to_host(dv.key), to_host(dv.key_sc)
    assert lp.rows["key"], "the loop completes key blocks"
    for (b, r), v in lp.rows["key"].items():
        c, sc = oracle.encode(v.astype(np.float32)[None], oracle.MXFP4)
        assert np.array_equal(key[b, r], c[0]) and np.array_equal(key_sc[b, r], sc[0]), ("key row", b, r)
    # FP8 rows: a correctly rounded value of the oracle's pooled row (FP8 quantisation
    # bound: 2^-4 relative in the normal range, 2^-10 * scale below, plus 1e-5 of the row max)
    for s, c, sc in (("csa", dv.ent, dv.ent_sc), ("hca", dv.hca, dv.hca_sc)):
        c, sc = to_host(c), to_host(sc)
        assert lp.rows[s], f"the loop completes {s} blocks"
        for (b, r), v in lp.rows[s].items():
            got = oracle.decode(c[b, r], oracle.FP8E4M3, sc[b, r])
            s_ref = np.repeat(np.abs(v).reshape(-1, 64).max(-1) / 448.0, 64)
            tol = np.maximum(np.abs(v) / 16, s_ref * 2.0 ** -10) * 1.001 + 1e-5 * np.abs(v).max()
            assert (np.abs(got - v) <= tol).all(), (s, b, r)


CASES = {"long": dict(seed=31, L0=[40003, 36862], S=300, N=10240, N2=320, k=256),
         "from_empty": dict(seed=32, L0=[0, 5], S=140, N=64, N2=4, k=32)}


@pytest.mark.parametrize("case", list(CASES))
def test_decode_loop(case):
    lp = Loop(**CASES[case])
    dv = Device(lp)
    S = lp.S
    hca_done = {i for i in range(S) for b in range(B) if (lp.L0[b] + i + 1) % M2 == 0}
    sample = set(range(0, S, 25)) | {S - 1} | hca_done | {min(i + 1, S - 1) for i in hca_done}
    for i in range(S):
        dv.load_inputs(i)
        dv.step()
        L = [l + i + 1 for l in lp.L0]
        e = expected_args(lp, L)
        got = {}
        for s in ("csa", "key", "hca"):
            got[s + ".nblk"] = to_host(dv.nblk[s]).tolist()
            got[s + ".tok0"] = to_host(dv.tok0[s]).tolist()
            got[s + ".row0"] = to_host(dv.row0[s]).tolist()
        got["n_csa"], got["n_hca"] = to_host(dv.n_csa)[:, 0].tolist(), to_host(dv.n_hca)[:, 0].tolist()
        got["wl"] = to_host(dv.wl_csa)[:, 0].tolist()
        assert to_host(dv.wl_hca)[:, 0].tolist() == got["wl"]
        got["wb_csa"], got["wb_hca"] = to_host(dv.wb_csa)[:, 0].tolist(), to_host(dv.wb_hca)[:, 0].tolist()
        for key_ in e:
            assert got[key_] == e[key_], (i, key_, got[key_], e[key_])
        if i in sample:
            check_against_oracle(lp, dv, i, L)
    torch.cuda.synchronize()
    check_final_state(lp, dv)
    eager = dv.state()

    # the same loop as one captured step replayed S times: the two calls, and
    # decode_loop_step (the appends inside the compress launch)
    for fused in (False, True):
        dv2 = Device(lp)
        dv2.load_inputs(0)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            dv2.step(fused)
        torch.cuda.synchronize()
        for i in range(S):
            dv2.load_inputs(i)
            graph.replay()
        torch.cuda.synchronize()
        for j, (a, b) in enumerate(zip(dv2.state(), eager)):
            assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), f"graph loop (fused={fused}): state {j}"
        del graph, dv2
