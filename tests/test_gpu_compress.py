"""GPU parity of csa_compress / hca_compress against the oracle.

m = 1 with zero gate and bias is an exact copy, so the device encoders
(FP8 E4M3 + per-64 scale, MXFP4, bf16) must equal the oracle codecs bit for
bit on the same fp32 values.  For real pooling (m = 4, 128) the pooled fp32
row must match the float64 oracle within rtol 1e-4, and encoded outputs must
be correct roundings of the oracle's pooled values."""
import numpy as np
import pytest
import torch

import long_context_attention_13_amd as lca
import oracle
import synth
from gpu_util import assert_rows_close, bf16_bits_to_f64, dev, to_dev, to_host

pytestmark = pytest.mark.gpu


def run_compress(x, gate, bias, m, dst_dt, nblk=None, x_tok0=None, dst_row0=None, dst_rows=None,
                 hca=False, bf16_in=False):
    """x: numpy f32 [B,T,D] (or uint16 bf16 bits); returns (codes, scales, pooled) numpy."""
    B, T, D = x.shape
    nb = T // m
    nblk = np.full(B, nb, np.int32) if nblk is None else nblk
    nblk_max = int(nblk.max()) if nblk.size else 0
    x_tok0 = np.zeros(B, np.int32) if x_tok0 is None else x_tok0
    dst_row0 = np.zeros(B, np.int64) if dst_row0 is None else dst_row0
    rows = nblk_max if dst_rows is None else dst_rows
    xd = to_dev(x)
    if dst_dt == lca.F32:
        dst = torch.zeros(B, rows, D, dtype=torch.float32, device=dev()); sc = None
    elif dst_dt == lca.BF16:
        dst = torch.zeros(B, rows, D, dtype=torch.bfloat16, device=dev()); sc = None
    elif dst_dt == lca.FP8E4M3:
        dst = torch.zeros(B, rows, D, dtype=torch.uint8, device=dev())
        sc = torch.zeros(B, rows, D // 64, dtype=torch.float32, device=dev())
    else:
        dst = torch.zeros(B, rows, D // 2, dtype=torch.uint8, device=dev())
        sc = torch.zeros(B, rows, D // 32, dtype=torch.uint8, device=dev())
    pooled = torch.full((B, max(nblk_max, 1), D), np.nan, dtype=torch.float32, device=dev())
    fn = lca.hca_compress if hca else lca.csa_compress
    fn(xd, to_dev(gate), to_dev(bias), m, to_dev(x_tok0), to_dev(nblk), to_dev(dst_row0), nblk_max,
       dst, dst_dt, sc, pooled)
    torch.cuda.synchronize()
    return to_host(dst), (None if sc is None else to_host(sc)), to_host(pooled)


def special_rows(D=128):
    rows = []
    g = np.random.default_rng(99)
    rows.append(np.zeros(D, np.float32))
    # amax 448 -> FP8 scale exactly 1; every E4M3 midpoint pattern (ties -> even)
    mags = np.array([oracle.e4m3_value(c) for c in range(127)])
    mids = ((mags[:-1] + mags[1:]) / 2).astype(np.float32)
    for i in range(0, len(mids), D - 1):
        r = np.zeros(D, np.float32)
        r[0] = 448.0
        chunk = mids[i:i + D - 1]
        r[1:1 + len(chunk)] = chunk * np.where(g.random(len(chunk)) < 0.5, -1, 1)
        rows.append(r)
    # amax in [4, 8): MX scale 2^0, E2M1 midpoints
    r = np.zeros(D, np.float32)
    r[:9] = [6.0, 0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, -0.1]
    rows.append(r)
    r = np.zeros(D, np.float32)
    r[3] = 1e-40                       # subnormal amax
    r[70] = -3e-39
    rows.append(r)
    # FP8 groups whose amax / 448 rounds to 0 in fp32 (scale 2^-149), and a
    # group where it rounds up to 2^-149 instead
    t = np.float32(2.0) ** -149
    r = np.zeros(D, np.float32)
    r[3], r[10], r[64 + 5], r[64 + 9] = t, -t, 224 * t, -100 * t
    rows.append(r)
    r = np.zeros(D, np.float32)
    r[0], r[1], r[64], r[65] = 100 * t, 3 * t, 225 * t, 7 * t
    rows.append(r)
    rows.append((g.standard_normal(D) * 1e30).astype(np.float32))
    rows.append((g.standard_normal(D) * 1e-30).astype(np.float32))
    rows.append(g.standard_normal(D).astype(np.float32) * np.float32(2.0) ** g.integers(-20, 20, D).astype(np.float32))
    return np.stack(rows)


@pytest.mark.parametrize("dst_dt", [lca.F32, lca.BF16, lca.FP8E4M3, lca.MXFP4])
def test_encoders_bit_exact(dst_dt):
    g = np.random.default_rng(1)
    vals = np.concatenate([special_rows(), g.standard_normal((3000, 128)).astype(np.float32)])
    x = vals[None]
    T = x.shape[1]
    codes, sc, pooled = run_compress(x, np.zeros((1, T), np.float32), np.zeros(1, np.float32), 1, dst_dt)
    assert np.array_equal(pooled.view(np.uint32), x.view(np.uint32))
    ref_codes, ref_sc = oracle.encode(x, {lca.F32: oracle.F32, lca.BF16: oracle.BF16,
                                          lca.FP8E4M3: oracle.FP8E4M3, lca.MXFP4: oracle.MXFP4}[dst_dt])
    if dst_dt == lca.F32:
        assert np.array_equal(codes.view(np.uint32), ref_codes.view(np.uint32))
    else:
        assert np.array_equal(codes, ref_codes)
    if sc is not None:
        assert np.array_equal(sc.view(np.uint8), ref_sc.view(np.uint8))


def test_fp8_hardware_decode_is_ocp():
    # the attention kernels decode E4M3 with the hardware conversion; check all
    # 256 codes through a 1-entry attention: q = e_d picks element d
    import math
    D = 128
    codes = np.arange(256, dtype=np.uint8)
    codes[0x7F] = 0
    codes[0xFF] = 0                                  # NaN codes are not valid inputs
    kv = codes.reshape(2, 128)[:, None, :].copy()    # B=2 sequences, one entry each
    sc = np.ones((2, 1, 2), np.float32)
    ref = oracle.decode(kv, oracle.FP8E4M3, sc)      # [2,1,128]
    Hq = 16
    q = np.zeros((2, 1, Hq, D), np.float32)
    out = torch.zeros(2, 1, Hq, D, dtype=torch.float32, device=dev())
    lca.hca_attend(to_dev(q), to_dev(kv), to_dev(sc), to_dev(np.ones((2, 1), np.int32)),
                   to_dev(np.zeros((2, 1, D), np.float32)), to_dev(np.zeros((2, 1), np.int32)),
                   to_dev(np.zeros((2, 1), np.int32)), to_dev(np.full(Hq, -1e30, np.float32)), 1.0, out)
    torch.cuda.synchronize()
    got = to_host(out)[:, 0, 0, :]      # q = 0: uniform weight 1 over the single entry
    assert np.array_equal(got, ref[:, 0, :].astype(np.float32))


@pytest.mark.parametrize("m,D,bf16_in", [(4, 128, False), (4, 64, False), (128, 128, True), (7, 128, True)])
def test_pooling_matches_oracle(m, D, bf16_in):
    g = np.random.default_rng(m * 10 + D)
    B, T = 3, 40 * m + m - 1          # ragged tail block not pooled
    x = g.standard_normal((B, T, D)).astype(np.float32)
    if bf16_in:
        x, _ = oracle.encode(x, oracle.BF16)
    gate = g.standard_normal((B, T)).astype(np.float32)
    bias = (g.standard_normal(m) * 0.1).astype(np.float32)
    nblk = np.array([40, 17, 0], np.int32)
    x_tok0 = np.array([0, m - 1, 5], np.int32)        # sequence 1 starts mid-buffer
    dst_row0 = np.array([0, 3, 0], np.int64)
    codes, _, pooled = run_compress(x, gate, bias, m, lca.F32, nblk=nblk, x_tok0=x_tok0,
                                    dst_row0=dst_row0, dst_rows=45, hca=(m > 64))
    xd = oracle.decode(x, oracle.BF16) if bf16_in else x.astype(np.float64)
    for b in range(B):
        n = nblk[b]
        t0 = x_tok0[b]
        ref = oracle.pool(xd[b, t0:t0 + n * m], gate[b, t0:t0 + n * m], bias, m)
        if n:
            assert_rows_close(pooled[b, :n], ref, 1e-4, f"pooled b={b}")
            assert np.array_equal(codes[b, dst_row0[b]:dst_row0[b] + n], pooled[b, :n])
        # rows outside [dst_row0, dst_row0 + n) untouched
        mask = np.ones(45, bool)
        mask[dst_row0[b]:dst_row0[b] + n] = False
        assert (codes[b, mask] == 0).all()


def test_small_config_cache_build():
    """4096 fp32 tokens, m=4 -> 1024 entries (and the 64-dim indexer keys)."""
    c = synth.small_csa_decode()
    codes, _, pooled = run_compress(c["x"], c["gate"], c["bias"], 4, lca.F32)
    ref = oracle.pool(c["x"][0].astype(np.float64), c["gate"][0], c["bias"], 4)
    assert codes.shape == (1, 1024, 128)
    assert_rows_close(codes[0], ref, 1e-4, "entries")
    kcodes, _, _ = run_compress(c["xi"], c["gate_i"], c["bias_i"], 4, lca.F32)
    kref = oracle.pool(c["xi"][0].astype(np.float64), c["gate_i"][0], c["bias_i"], 4)
    assert_rows_close(kcodes[0], kref, 1e-4, "indexer keys")


@pytest.mark.parametrize("dst_dt", [lca.BF16, lca.FP8E4M3, lca.MXFP4])
def test_pooled_encoding_is_a_correct_rounding(dst_dt):
    """Encoded pooled rows decode to a correctly rounded value of (a value within
    rtol of) the oracle's pooled row; codes equal the oracle codec applied to
    the oracle's own pooled values except at near-ties."""
    g = np.random.default_rng(5 + dst_dt)
    B, T, D, m = 2, 128 * 24, 128, 128
    x, _ = oracle.encode(g.standard_normal((B, T, D)).astype(np.float32), oracle.BF16)
    gate = g.standard_normal((B, T)).astype(np.float32)
    bias = (g.standard_normal(m) * 0.1).astype(np.float32)
    codes, sc, _ = run_compress(x, gate, bias, m, dst_dt, hca=True)
    xd = oracle.decode(x, oracle.BF16)
    ref = np.stack([oracle.pool(xd[b], gate[b], bias, m) for b in range(B)])
    odt = {lca.BF16: oracle.BF16, lca.FP8E4M3: oracle.FP8E4M3, lca.MXFP4: oracle.MXFP4}[dst_dt]
    rc, rs = oracle.encode(ref.astype(np.float32), odt)
    got = oracle.decode(codes, odt, sc)
    exp = oracle.decode(rc, odt, rs)
    # quantisation bound (bf16: half an ulp <= 2^-8 relative; FP8: 2^-4 relative in
    # the normal range, 2^-10 * scale below it; MXFP4: saturation at 6X can cost up
    # to 2X <= amax/2) plus the fp32 pooling error, an absolute 1e-5 of the row max
    rowmax = np.abs(ref).max(-1, keepdims=True)
    if dst_dt == lca.BF16:
        qb = np.abs(ref) * 2.0 ** -8
    elif dst_dt == lca.FP8E4M3:
        s = np.repeat(rs.astype(np.float64), 64, axis=-1)
        qb = np.maximum(np.abs(ref) / 16, s * 2.0 ** -10)
    else:
        amax = np.abs(ref).reshape(B, -1, D // 32, 32).max(-1)
        qb = np.repeat(amax / 2, 32, axis=-1).reshape(ref.shape)
    tol = qb * 1.001 + 1e-5 * rowmax
    err = np.abs(got - ref)
    i = np.unravel_index(np.argmax(err - tol), err.shape)
    assert (err <= tol).all(), (i, got[i], ref[i], tol[i])
    frac_equal = (codes == rc).mean()
    assert frac_equal > 0.999, frac_equal


def test_batch_equals_single_calls():
    """lca_compress_batch: CSA FP8 (m = 4), indexer keys MXFP4 with pooled rows
    (m = 4), HCA FP8 (m = 128) and a bf16 cache (m = 16) in one launch give
    the bytes of the four single calls; rows no job writes are untouched."""
    d = dev()
    g = torch.Generator(device=d)
    g.manual_seed(91)
    B, D, rows = 3, 128, 12
    x = torch.randn(B, 2048, D, generator=g, device=d).to(torch.bfloat16)
    gate = torch.randn(B, 2048, generator=g, device=d)
    i32 = lambda v: torch.tensor(v, dtype=torch.int32, device=d)
    i64 = lambda v: torch.tensor(v, dtype=torch.int64, device=d)
    specs = [  # (m, dst_dt, nblk, tok0, row0, pooled)
        (4, lca.FP8E4M3, [5, 0, 3], [0, 7, 100], [0, 4, 9], False),
        (4, lca.MXFP4, [1, 5, 2], [3, 0, 64], [11, 0, 2], True),
        (128, lca.FP8E4M3, [2, 1, 0], [0, 129, 5], [1, 10, 0], False),
        (16, lca.BF16, [4, 4, 4], [16, 0, 33], [0, 8, 3], True),
    ]

    def dst_of(dt):
        if dt == lca.FP8E4M3:
            return (torch.full((B, rows, D), 0x5A, dtype=torch.uint8, device=d),
                    torch.full((B, rows, D // 64), -3.0, device=d))
        if dt == lca.MXFP4:
            return (torch.full((B, rows, D // 2), 0x5A, dtype=torch.uint8, device=d),
                    torch.full((B, rows, D // 32), 7, dtype=torch.uint8, device=d))
        return torch.full((B, rows, D), -2.0, device=d).to(torch.bfloat16), None

    single, batch, jobs = [], [], []
    for m, dt, nb, t0, r0, pooled in specs:
        bias = torch.randn(m, generator=g, device=d)
        args = (x, gate, bias, m, i32(t0), i32(nb), i64(r0), max(nb))
        outs = []
        for dst_list in (single, batch):
            dst, sc = dst_of(dt)
            pl = torch.full((B, max(nb), D), 9.0, device=d) if pooled else None
            dst_list.append((dst, sc, pl))
        dst, sc, pl = single[-1]
        (lca.hca_compress if m > 64 else lca.csa_compress)(*args, dst, dt, sc, pl)
        dst, sc, pl = batch[-1]
        jobs.append(lca.compress_job(*args, dst, dt, sc, pl))
    lca.compress_batch(jobs)                    # each job keeps its own index arrays and bias alive
    torch.cuda.synchronize()
    del jobs
    for j, (a, b) in enumerate(zip(single, batch)):
        for ta, tb in zip(a, b):
            if ta is not None:
                assert torch.equal(ta.view(torch.uint8), tb.view(torch.uint8)), f"job {j}"
