"""Pins for the oracle's storage codecs (CPU only).

FP8 E4M3 is checked against torch's float8_e4m3fn conversions (a library
routine) on all 256 codes and on dense sweeps of fp32 values; E2M1 against the
OCP MX table in tests/golden/e2m1_values.txt; bf16 against torch's bfloat16
rounding; the MXFP4 shared exponent against exact powers of two and numpy's
log2 away from powers of two; "FP4 to FP8 dequantisation is lossless" (wiki
page, 基础设施) against the FP8 encoder.
"""
import math
import os

import numpy as np
import pytest
import torch

import oracle

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def torch_e4m3_codes(v: np.ndarray) -> np.ndarray:
    return torch.from_numpy(np.ascontiguousarray(v, np.float32)).to(torch.float8_e4m3fn).view(
        torch.uint8).numpy()


def test_e4m3_decode_all_codes_match_torch():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = np.array([oracle.e4m3_value(c) for c in range(256)])
    nan = np.isnan(ref)
    assert list(np.nonzero(nan)[0]) == [0x7F, 0xFF]
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    assert oracle.e4m3_value(0x7E) == 448.0
    assert oracle.e4m3_value(0x01) == 2.0 ** -9


def test_e4m3_encode_matches_torch_rne_in_range():
    g = np.random.default_rng(7)
    vals = [g.standard_normal(20000).astype(np.float32) * s for s in (1e-3, 0.1, 1, 30, 200)]
    # every exact midpoint between neighbouring finite codes (ties -> even code)
    mags = np.array([oracle.e4m3_value(c) for c in range(127)])
    mids = ((mags[:-1] + mags[1:]) / 2).astype(np.float32)
    vals += [mids, -mids, mags.astype(np.float32)]
    v = np.concatenate(vals)
    v = v[np.abs(v) < 464.0]               # torch does not saturate beyond 464
    got = np.array([oracle.e4m3_encode(float(x)) for x in v], np.uint8)
    assert np.array_equal(got, torch_e4m3_codes(v))


def test_e4m3_encode_saturates():
    for x, c in [(464.0, 0x7E), (1e6, 0x7E), (-1e30, 0xFE), (448.0, 0x7E)]:
        assert oracle.e4m3_encode(x) == c


def test_e2m1_table_matches_ocp_golden():
    rows = [l.split() for l in open(os.path.join(GOLD, "e2m1_values.txt")) if l[0] != "#"]
    for code, val in rows:
        assert oracle.e2m1_value(int(code)) == float(val)
        assert oracle.e2m1_value(int(code) | 8) == -float(val)


def test_e2m1_encode_rne_and_saturation():
    # midpoints go to the even code
    cases = {0.25: 0, 0.75: 2, 1.25: 2, 1.75: 4, 2.5: 4, 3.5: 6, 5.0: 6, 7.0: 7, 100.0: 7, -0.1: 8,
             0.2: 0, 0.3: 1, 2.6: 5, 5.1: 7, -0.75: 10, -6.5: 15}
    for y, c in cases.items():
        assert oracle.e2m1_encode(y) == c, y


def test_fp4_to_fp8_is_lossless():
    # wiki page, 基础设施: dequantising FP4 to FP8 loses nothing, i.e. every E2M1
    # value is an E4M3 value (scale 1).
    for c in range(16):
        v = oracle.e2m1_value(c)
        assert oracle.e4m3_value(oracle.e4m3_encode(v)) == v


def test_fp8_scale_rule_and_roundtrip():
    g = np.random.default_rng(3)
    v = g.standard_normal((64, 128)).astype(np.float32) * np.float32(3.0)
    v[5] = 0.0
    codes, sc = oracle.encode(v, oracle.FP8E4M3)
    amax = np.abs(v.reshape(64, 2, 64)).max(-1)
    exp_sc = np.where(amax == 0, np.float32(1), (amax / np.float32(448)).astype(np.float32))
    assert np.array_equal(sc, exp_sc)
    # the element of largest magnitude maps to +-448
    dec = oracle.decode(codes, oracle.FP8E4M3, sc)
    nz = amax.reshape(-1) > 0
    dmax = np.abs(dec.reshape(-1, 64)).max(-1)
    assert np.allclose(dmax[nz], (448.0 * sc.reshape(-1).astype(np.float64))[nz], rtol=0, atol=0)
    # each code is the RNE code of fl32(v / s)
    q = (v.reshape(-1, 64) / sc.reshape(-1, 1)).astype(np.float32)
    q = np.clip(q, -447.99, 447.99)
    assert np.array_equal(codes.reshape(-1, 64), torch_e4m3_codes(q))
    # exact round trip of decoded values with power-of-two scales
    c2 = g.integers(0, 127, size=(8, 64)).astype(np.uint8) | (g.integers(0, 2, (8, 64)) << 7).astype(np.uint8)
    c2[:, 0] = 0x7E
    s2 = np.float32(2.0) ** g.integers(-6, 6, size=(8, 1)).astype(np.float32)
    vals = np.array([[oracle.e4m3_value(c) for c in row] for row in c2], np.float32) * s2
    back, sb = oracle.encode(vals, oracle.FP8E4M3)
    assert np.array_equal(sb.reshape(-1), s2.reshape(-1))
    assert np.array_equal(back, c2)


def test_fp8_scale_underflow_branch():
    """Reading of the FP8 scale rule for groups whose amax / 448 rounds to 0 in
    fp32: the scale is the smallest fp32 subnormal, s = 2^-149, so the group's
    values become integer multiples of s and their codes are those integers
    rounded to E4M3 (ties to the even code).  Closed forms, one per group."""
    t = np.float32(2.0) ** -149
    v = np.zeros((3, 128), np.float32)
    v[0, 3], v[0, 10] = t, -t                        # amax = s: codes of +-1
    v[0, 64 + 5], v[0, 64 + 9] = 224 * t, -100 * t    # 224/448 = 1/2: ties to 0
    v[1, 0], v[1, 1] = 100 * t, 3 * t                 # 100/448 < 1/2: rounds to 0
    v[1, 64], v[1, 65] = 225 * t, 7 * t               # 225/448 > 1/2: s = 2^-149 without the branch
    v[2, 0] = 448 * t                                 # s = fl32(448 s / 448) = s exactly
    assert np.float32(v[0, 64 + 5] / np.float32(448)) == 0 and np.float32(v[1, 64] / np.float32(448)) == t
    codes, sc = oracle.encode(v, oracle.FP8E4M3)
    assert np.array_equal(sc[:, 0], [t, t, t]) and np.array_equal(sc[:, 1], [t, t, np.float32(1)])
    # E4M3 codes of the integers 1, 3, 7, 100 (a tie between 96 and 104), 224, 225 and 448
    assert (codes[0, 3], codes[0, 10]) == (0x38, 0xB8)
    assert (codes[0, 64 + 5], codes[0, 64 + 9]) == (0x76, 0xEC)
    assert (codes[1, 0], codes[1, 1]) == (0x6C, 0x44)
    assert (codes[1, 64], codes[1, 65]) == (0x76, 0x4E)
    assert codes[2, 0] == 0x7E
    assert np.count_nonzero(codes) == 9
    # the same codes from torch's E4M3 conversion of v / s
    q = (v.reshape(-1, 64).astype(np.float64) / sc.reshape(-1, 1).astype(np.float64)).astype(np.float32)
    assert np.array_equal(codes.reshape(-1, 64), torch_e4m3_codes(q))
    # decoded values: the code's value times 2^-149 (exact in float64)
    dec = oracle.decode(codes, oracle.FP8E4M3, sc)
    assert dec[0, 64 + 9] == -96 * 2.0 ** -149 and dec[1, 64] == 224 * 2.0 ** -149


def test_mxfp4_shared_exponent():
    g = np.random.default_rng(5)
    blocks = g.standard_normal((400, 32)).astype(np.float32) * np.float32(4.0) ** g.integers(
        -8, 8, size=(400, 1)).astype(np.float32)
    blocks[0] = 0.0
    blocks[1] = 0.0
    blocks[1, 7] = 8.0            # amax exactly 2^3 -> X = 1
    blocks[2] = 0.0
    blocks[2, 3] = -0.5           # amax 2^-1 -> X = -3
    _, sc = oracle.encode(blocks, oracle.MXFP4)
    X = sc.reshape(-1).astype(int) - 127
    amax = np.abs(blocks).max(-1).astype(np.float64)
    assert X[0] == -127 and X[1] == 1 and X[2] == -3
    for b in range(3, 400):
        lg = math.log2(amax[b])
        if abs(lg - round(lg)) > 1e-9:
            assert X[b] == math.floor(lg) - 2


def test_mxfp4_elements_and_packing():
    # a block with amax in [4, 8) has scale 2^0, so elements are RNE(v) directly
    v = np.zeros((1, 32), np.float32)
    v[0, :8] = [0.25, 0.75, 1.25, 5.0, -7.0, 6.0, 2.9, -0.1]
    codes, sc = oracle.encode(v, oracle.MXFP4)
    assert sc[0, 0] == 127
    expect = [0, 2, 2, 6, 15, 7, 5, 8]
    got = [(codes[0, i // 2] >> (4 * (i % 2))) & 15 for i in range(8)]
    assert got == expect
    dec = oracle.decode(codes, oracle.MXFP4, sc)
    assert list(dec[0, :8]) == [0.0, 1.0, 1.0, 4.0, -6.0, 6.0, 3.0, -0.0]


def test_bf16_encode_matches_torch():
    g = np.random.default_rng(11)
    v = np.concatenate([g.standard_normal(20000).astype(np.float32) * s for s in (1e-20, 1, 1e20)])
    # exact halfway cases between neighbouring bf16 values
    base = torch.from_numpy(g.standard_normal(2000).astype(np.float32)).to(torch.bfloat16)
    bits = base.view(torch.int16).numpy().astype(np.uint32) << 16
    half = (bits | 0x8000).view(np.float32)
    v = np.concatenate([v, half])
    ref = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got, _ = oracle.encode(v, oracle.BF16)
    assert np.array_equal(got, ref)
    dec = oracle.decode(ref, oracle.BF16)
    assert np.array_equal(dec, torch.from_numpy(ref.view(np.int16)).view(torch.bfloat16).double().numpy())
