"""Pins of the oracle's number formats (CPU only).

Each check compares the oracle with something other than itself: the format
definition's anchor table, an independent nearest-value search, and torch's
own float8_e4m3fn / bfloat16 conversions.
"""
import math
import os

import numpy as np
import pytest
import torch

from oracle import codec

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "e4m3_ocp_anchors.txt")


def _anchors():
    rows = []
    for line in open(GOLDEN):
        line = line.split("#")[0].strip()
        if line:
            c, v = line.split()
            rows.append((int(c, 16), float(v)))
    return rows


def test_decode_anchor_table():
    dec = codec.e4m3_decode_table()
    for c, v in _anchors():
        if math.isnan(v):
            assert math.isnan(dec[c]), hex(c)
        else:
            assert dec[c] == v, hex(c)
            assert math.copysign(1.0, dec[c]) == math.copysign(1.0, v), hex(c)


def test_decode_all_256_against_torch():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float32).double().numpy()
    dec = codec.e4m3_decode_table()
    nan = np.isnan(ref)
    assert (np.isnan(dec) == nan).all()
    assert np.array_equal(dec[~nan], ref[~nan])
    assert np.array_equal(np.signbit(dec[~nan]), np.signbit(ref[~nan]))
    assert nan.sum() == 2 and nan[0x7F] and nan[0xFF]


def test_decode_closed_form_counts():
    dec = codec.e4m3_decode_table()
    fin = dec[~np.isnan(dec)]
    assert fin.size == 254
    assert fin.max() == 448.0 and fin.min() == -448.0
    pos = np.unique(fin[fin > 0])
    assert pos.size == 126 and pos[0] == 2.0 ** -9
    # consecutive positive magnitudes: spacing 2^-9 below 2^-5, then 2^(e-3) per binade
    for a, b in zip(pos[:-1], pos[1:]):
        e = max(math.floor(math.log2(a)), -6)
        assert b - a == 2.0 ** (e - 3)


def test_encode_roundtrip_all_finite_codes():
    dec = codec.e4m3_decode_table()
    codes = np.arange(256, dtype=np.uint8)
    fin = ~np.isnan(dec)
    assert np.array_equal(codec.e4m3_encode(dec[fin]), codes[fin])


def _nearest_search(p):
    """Independent encoder: nearest of the 127 non-negative finite magnitudes, ties to the even code."""
    p = np.asarray(p, dtype=np.float64)
    mags = np.array([(1 + (c & 7) / 8) * 2.0 ** (((c >> 3) & 15) - 7) if (c >> 3) & 15 else (c & 7) * 2.0 ** -9
                     for c in range(0x7F)])
    a = np.abs(p)
    out = np.zeros(p.shape, dtype=np.int64)
    fin = ~np.isnan(a)
    af = np.where(fin, a, 0.0)
    dist = np.abs(af[:, None] - mags[None, :])
    best = dist.min(axis=1, keepdims=True)
    cand = dist == best
    codes = np.arange(0x7F)
    # among equally near codes prefer the even one
    even_pref = np.where(cand & (codes[None, :] % 2 == 0), codes[None, :], 10 ** 6).min(axis=1)
    any_pref = np.where(cand, codes[None, :], 10 ** 6).min(axis=1)
    out = np.where(even_pref < 10 ** 6, even_pref, any_pref)
    out = np.where(af > 448.0, 0x7E, out)        # saturate (beyond 448, incl. inf)
    out = np.where(fin, out, 0x7F)
    return (out | (np.signbit(p).astype(np.int64) << 7)).astype(np.uint8)


ALL_BF16 = np.arange(65536, dtype=np.uint32).astype(np.uint16)


@pytest.mark.parametrize("scale", [1.0, 2.0 ** -3, 2.0 ** -6, 4.5 / 448, 5.3125 / 448, 3.0e-3])
def test_encode_brute_force_all_bf16(scale):
    scale = np.float32(scale)
    x = codec.f32_from_bf16(ALL_BF16)
    with np.errstate(over="ignore"):
        prod = (x * (np.float32(1) / scale)).astype(np.float32)
    got = codec.e4m3_encode(prod)
    for a in range(0, 65536, 8192):
        ref = _nearest_search(prod[a:a + 8192])
        assert np.array_equal(got[a:a + 8192], ref), scale
    assert np.array_equal(codec.quantize_e4m3(ALL_BF16, scale), got)


def test_encode_against_torch_in_range():
    x = codec.f32_from_bf16(ALL_BF16)
    m = np.abs(x) <= 448.0
    got = codec.e4m3_encode(x[m])
    ref = torch.from_numpy(x[m]).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(got, ref)


def test_encode_saturation_and_specials():
    assert codec.e4m3_encode([448.0, 449.0, 463.9, 464.0, 1e30, np.inf])[:].tolist() == [0x7E] * 6
    assert codec.e4m3_encode([-448.0, -500.0, -np.inf]).tolist() == [0xFE] * 3
    assert codec.e4m3_encode([np.nan]).tolist() == [0x7F]
    assert codec.e4m3_encode([-np.nan]).tolist() == [0xFF]
    assert codec.e4m3_encode([-1e-30, -0.0, 0.0]).tolist() == [0x80, 0x80, 0x00]
    # ties: halfway between 0 and 2^-9 -> 0 (even); between 0x01 and 0x02 -> 0x02
    assert codec.e4m3_encode([2.0 ** -10, 3 * 2.0 ** -10]).tolist() == [0x00, 0x02]
    # 1 + 1/16 is halfway between 1.0 (0x38) and 1.125 (0x39): even -> 0x38
    assert codec.e4m3_encode([1.0625, 1.1875]).tolist() == [0x38, 0x3A]
    # the carry from the top of a binade into the next exponent
    assert codec.e4m3_encode([1.96875]).tolist() == [0x40]


def test_encode_monotone():
    x = np.linspace(0, 460, 200001)
    c = codec.e4m3_encode(x).astype(np.int64)
    assert (np.diff(c) >= 0).all()


def test_bf16_rne_against_torch():
    rng = np.random.Generator(np.random.PCG64(7))
    x = np.concatenate([
        rng.standard_normal(200000).astype(np.float32),
        (rng.standard_normal(20000) * 1e-39).astype(np.float32),     # subnormals
        np.array([0.0, -0.0, np.inf, -np.inf, 3.3895314e38, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8,
                  1.0 + 2 ** -8 + 2 ** -20], dtype=np.float32),
        rng.integers(0, 2 ** 32, 200000, dtype=np.uint64).astype(np.uint32).view(np.float32),
    ])
    got = codec.bf16_from_f32(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    nan = np.isnan(x)
    assert np.array_equal(got[~nan], ref[~nan])
    assert (((got[nan] & 0x7FFF) > 0x7F80)).all()


def test_bf16_widen_exact():
    b = ALL_BF16
    f = codec.f32_from_bf16(b)
    fin = ~np.isnan(f)
    assert np.array_equal(codec.bf16_from_f32(f[fin]), b[fin])


def test_scale_calibration():
    x = codec.bf16_from_f32(np.array([0.5, -3.0, 2.0, -0.25], dtype=np.float32))
    s = codec.calibrate_scale(x)
    assert s == np.float32(3.0) / np.float32(448.0)
    # the largest magnitude lands on the top code, and nothing saturates
    q = codec.quantize_e4m3(x, s)
    assert q[1] == 0xFE
    assert codec.absmax_bits(x) == np.float32(3.0).view(np.uint32)
    # NaN is ignored by absmax, inf is not
    nanx = np.array([0x7FC0, 0x4000], dtype=np.uint16)
    assert codec.absmax_bits(nanx) == np.float32(2.0).view(np.uint32)


def test_dequantize_exact():
    codes = np.arange(256, dtype=np.uint8)
    scale = np.float32(0.0123)
    d = codec.dequantize_e4m3(codes, scale)
    fin = ~np.isnan(d)
    # dec(c) has 4 significant bits and scale 24: the fp64 product is exact
    ref = np.array([float(np.float64(v)) * float(scale) for v in codec.e4m3_decode_table()])
    assert np.array_equal(d[fin], ref[fin])
