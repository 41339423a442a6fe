"""GPU parity of the pooling variants (per-channel gates, overlapping blocks;
alone and together) against the oracle's pool_variant:

- blocks from the start of a sequence, where the overlap rows of the first
  block do not exist (they hold NaN here, so reading or weighting them would
  show), ragged block counts, both input types and widths;
- blocks in the middle of a sequence (their overlap rows are real tokens);
- a decode loop over a ring (lca_decode_append with per-channel gate rings
  and overlap), issued as the two calls and as lca_decode_loop_step, whose
  cache rows (fp32, so the pooled values themselves) match the oracle's
  pooling of the whole token history, and whose two forms give equal bytes.

Pooled rows are compared within rtol 1e-4 (fp32 accumulation against the
float64 oracle).  Inputs are seeded N(0,1) tokens and gates, bias N(0, 0.3^2).
"""
import numpy as np
import pytest
import torch

import long_context_attention_13_amd as lca
import oracle
from gpu_util import assert_rows_close, dev, to_dev, to_host

pytestmark = pytest.mark.gpu


def as_input(x, x_dt):
    """float32 -> (device tensor, float64 values the kernel reads)."""
    if x_dt == "bf16":
        bits = oracle.encode(x.astype(np.float32), oracle.BF16)[0]
        return to_dev(bits), oracle.decode(bits, oracle.BF16)
    return to_dev(x.astype(np.float32)), x.astype(np.float64)


def compress(xt, gate, bias, m, o, tok0, nblk, row0, nblk_max, dst_rows):
    B, _, D = xt.shape
    d = dev()
    dst = torch.zeros(B, dst_rows, D, device=d)
    pooled = torch.zeros(B, nblk_max, D, device=d)
    job = lca.compress_job(xt, to_dev(gate), to_dev(bias), m, to_dev(np.array(tok0, np.int32)),
                           to_dev(np.array(nblk, np.int32)), to_dev(np.array(row0, np.int64)), nblk_max, dst, lca.F32,
                           pooled=pooled, overlap=o)
    lca.compress_batch([job])
    torch.cuda.synchronize()
    return to_host(dst), to_host(pooled)


CASES = [(4, 0, 1, 128, "bf16"), (4, 4, 0, 128, "bf16"), (4, 2, 1, 128, "bf16"), (4, 3, 1, 64, "f32"),
         (128, 64, 0, 128, "bf16"), (128, 128, 1, 128, "bf16"), (7, 5, 0, 128, "f32")]


@pytest.mark.parametrize("m,o,pc,D,x_dt", CASES)
def test_variant_from_sequence_start(m, o, pc, D, x_dt):
    g = np.random.default_rng(1000 + 7 * m + o + pc)
    B, n = 2, 9
    T = n * m + 2                                   # a tail that is not pooled
    nblk = [n, n - 3]
    x = g.standard_normal((B, o + T, D)).astype(np.float32)
    x[:, :o] = np.nan                               # rows before the first token
    gate = g.standard_normal((B, o + T, D) if pc else (B, o + T)).astype(np.float32)
    gate[:, :o] = np.nan
    bias = (g.standard_normal((m + o, D) if pc else (m + o,)) * 0.3).astype(np.float32)
    xt, xd = as_input(x, x_dt)
    dst, pooled = compress(xt, gate, bias, m, o, [0, 0], nblk, [0, 0], n, n)
    for b in range(B):
        ref = oracle.pool_variant(xd[b, o:], gate[b, o:], bias, m, o)[:nblk[b]]
        assert_rows_close(pooled[b, :nblk[b]], ref, 1e-4, f"pooled b={b}")
        assert np.array_equal(dst[b, :nblk[b]].view(np.uint32), pooled[b, :nblk[b]].view(np.uint32))
        assert (dst[b, nblk[b]:] == 0).all()


@pytest.mark.parametrize("m,o,pc,D,x_dt", CASES)
def test_variant_mid_sequence(m, o, pc, D, x_dt):
    g = np.random.default_rng(2000 + 7 * m + o + pc)
    B, j0, n = 2, 3, 6
    T = (j0 + n) * m
    x = g.standard_normal((B, T, D)).astype(np.float32)
    gate = g.standard_normal((B, T, D) if pc else (B, T)).astype(np.float32)
    bias = (g.standard_normal((m + o, D) if pc else (m + o,)) * 0.3).astype(np.float32)
    xt, xd = as_input(x, x_dt)
    # block j0 + i of sequence b pools from buffer row (j0 + i) * m - o
    dst, pooled = compress(xt, gate, bias, m, o, [j0 * m - o] * B, [n, n - 1], [j0, j0], n, j0 + n)
    for b, nb in enumerate([n, n - 1]):
        ref = oracle.pool_variant(xd[b], gate[b], bias, m, o)[j0:j0 + nb]
        assert_rows_close(pooled[b, :nb], ref, 1e-4, f"pooled b={b}")
        assert np.array_equal(dst[b, j0:j0 + nb].view(np.uint32), pooled[b, :nb].view(np.uint32))
        assert (dst[b, :j0] == 0).all()


@pytest.mark.parametrize("o,pc", [(4, 1), (2, 0), (0, 1)])
def test_variant_decode_loop(o, pc):
    """One raw-token stream with m = 4 in a ring of R = 4 + o + 3 rows (R not a
    multiple of m): 60 steps from lengths 0 and 9."""
    g = np.random.default_rng(3000 + 10 * o + pc)
    d = dev()
    B, D, m, S = 2, 128, 4, 60
    R = m + o + 3
    L0 = [0, 9]
    hist = [oracle.encode(g.standard_normal((l + S, D)).astype(np.float32), oracle.BF16)[0] for l in L0]
    gates = [g.standard_normal((l + S, D) if pc else (l + S,)).astype(np.float32) for l in L0]
    bias = (g.standard_normal((m + o, D) if pc else (m + o,)) * 0.3).astype(np.float32)
    N = (max(L0) + S) // m + 1

    def state():
        ring = np.zeros((B, 2 * R, D), np.uint16)
        gring = np.zeros((B, 2 * R, D) if pc else (B, 2 * R), np.float32)
        for b in range(B):
            for p in range(max(0, L0[b] - R), L0[b]):
                ring[b, p % R] = ring[b, p % R + R] = hist[b][p]
                gring[b, p % R] = gring[b, p % R + R] = gates[b][p]
        st = dict(ring=to_dev(ring), gring=to_dev(gring), len=torch.tensor(L0, dtype=torch.int64, device=d),
                  xn=torch.zeros(B, D, dtype=torch.bfloat16, device=d),
                  gn=torch.zeros((B, D) if pc else (B,), device=d),
                  tok0=torch.zeros(B, dtype=torch.int32, device=d), nblk=torch.zeros(B, dtype=torch.int32, device=d),
                  row0=torch.zeros(B, dtype=torch.int64, device=d), cache=torch.zeros(B, N, D, device=d))
        st["app"] = lca.append_job(st["xn"], st["ring"], st["len"], m=m, g_new=st["gn"], gring=st["gring"],
                                   x_tok0=st["tok0"], nblk=st["nblk"], dst_row0=st["row0"], overlap=o)
        st["cj"] = lca.compress_job(st["ring"], st["gring"], to_dev(bias), m, st["tok0"], st["nblk"], st["row0"], 1,
                                    st["cache"], lca.F32, overlap=o)
        return st

    xs = to_dev(np.stack([np.stack([hist[b][L0[b] + i] for b in range(B)]) for i in range(S)]))
    gs = to_dev(np.stack([np.stack([gates[b][L0[b] + i] for b in range(B)]) for i in range(S)]))
    two, one = state(), state()
    for i in range(S):
        for st, fused in ((two, False), (one, True)):
            st["xn"].copy_(xs[i])
            st["gn"].copy_(gs[i])
            if fused:
                lca.decode_loop_step([st["app"]], [st["cj"]], None, [])
            else:
                lca.decode_append([st["app"]])
                lca.compress_batch([st["cj"]])
    torch.cuda.synchronize()
    for k in ("ring", "gring", "len", "cache"):
        assert torch.equal(two[k].view(torch.uint8), one[k].view(torch.uint8)), k
    cache = to_host(one["cache"])
    for b in range(B):
        ref = oracle.pool_variant(oracle.decode(hist[b], oracle.BF16), gates[b], bias, m, o)
        r0 = L0[b] // m                                  # rows completed during the loop
        r1 = (L0[b] + S) // m
        assert_rows_close(cache[b, r0:r1], ref[r0:r1], 1e-4, f"cache b={b}")
        assert (cache[b, r1:] == 0).all() and (cache[b, :r0] == 0).all()
