"""Number formats of the KV cache: bfloat16 and FP8 e4m3 (oracle; test infrastructure).

The Cloudflare post "Smaller, faster, safer: running Kimi and GLM at scale",
section "Quantized KV cache", stores the cache as "FP8, e4m3" instead of
BF16.  It does not say which e4m3; the reading taken here is the OCP 8-bit
floating point format E4M3 ("E4M3FN"): sign bit, 4 exponent bits with bias 7,
3 mantissa bits, no infinities, NaN = S.1111.111, largest finite 448 =
S.1111.110, subnormals m * 2^-9 for exponent field 0.

Readings where the pages are silent:
* rounding is to nearest, ties to even, never stochastic;
* magnitudes above 448 (including infinity) saturate to +-448;
* NaN encodes to 0x7F with the input's sign bit;
* a tiny negative value keeps its sign (rounds to 0x80, -0);
* a per-tensor scale is applied by multiplying with inv = fl32(1/scale),
  and the encoded value is fl32(x * inv) (one fp32 rounding, then the
  e4m3 rounding); decoding is dec(c) * scale;
* the scale is fl32(max|x| / 448) over the whole tensor.
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0
_TWO_M9 = 2.0 ** -9          # smallest subnormal
_TWO_M6 = 2.0 ** -6          # smallest normal


# ----------------------------------------------------------------------------- bfloat16

def bf16_from_f32(x) -> np.ndarray:
    """float32 -> bfloat16 bits, round to nearest even, by integer arithmetic.

    NaN keeps its sign and becomes the quiet NaN 0x7FC0 (or 0xFFC0).
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    is_nan = ((u >> 23) & 0xFF == 0xFF) & (u & 0x7FFFFF != 0)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16) & 0xFFFF
    r = np.where(is_nan, ((u >> 16) & 0x8000) | 0x7FC0, r)
    return r.astype(np.uint16)


def f32_from_bf16(b) -> np.ndarray:
    """bfloat16 bits -> float32 (exact)."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def f64_from_bf16(b) -> np.ndarray:
    return f32_from_bf16(b).astype(np.float64)


# ----------------------------------------------------------------------------- e4m3

def e4m3_decode(c) -> np.ndarray:
    """e4m3 code(s) -> float64 values (NaN for S.1111.111)."""
    c = np.asarray(c, dtype=np.uint8).astype(np.int64)
    s = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    normal = (1.0 + m / 8.0) * np.ldexp(1.0, e - 7)
    sub = m * _TWO_M9
    v = s * np.where(e == 0, sub, normal)
    return np.where((e == 15) & (c & 7 == 7), np.nan, v)


def e4m3_decode_table() -> np.ndarray:
    """float64[256]: value of every code."""
    return e4m3_decode(np.arange(256, dtype=np.uint8))


def e4m3_encode(p) -> np.ndarray:
    """float value(s) -> e4m3 codes (uint8), RNE with saturation.

    Steps: take the sign; NaN -> 0x7F; |p| > 448 -> 0x7E; |p| below the
    smallest normal -> the subnormal count n = RNE(|p| / 2^-9) (n = 8 is the
    smallest normal's code 0x08); otherwise split |p| = f * 2^e with f in
    [1, 2), take n = RNE(|p| / 2^(e-3)) in [8, 16], carry n = 16 into the
    exponent, and emit (e+7) << 3 | (n-8).  Every division is by a power of
    two and so exact in fp64; np.rint rounds half to even.
    """
    p = np.asarray(p, dtype=np.float64)
    sign = np.signbit(p).astype(np.int64) << 7
    a = np.abs(p)
    nan = np.isnan(a)
    a_f = np.where(nan, 0.0, a)
    sat = a_f > E4M3_MAX
    a_c = np.where(sat, 0.0, a_f)

    sub = a_c < _TWO_M6
    n_sub = np.rint(a_c / _TWO_M9).astype(np.int64)          # 0..8

    _, x = np.frexp(np.where(sub, 1.0, a_c))                  # a = f * 2^x, f in [0.5, 1)
    e = x.astype(np.int64) - 1                                # a = (2f) * 2^e
    n = np.rint(a_c / np.ldexp(1.0, e - 3)).astype(np.int64)  # 8..16
    carry = n == 16
    e = np.where(carry, e + 1, e)
    n = np.where(carry, 8, n)
    code_norm = ((e + 7) << 3) | (n - 8)

    code = np.where(sub, n_sub, code_norm)
    code = np.where(sat, 0x7E, code)
    code = np.where(nan, 0x7F, code)
    return (code | sign).astype(np.uint8)


def scale_from_absmax(absmax) -> np.float32:
    """Per-tensor scale fl32(max|x| / 448), the division done in fp32."""
    return np.float32(absmax) / np.float32(E4M3_MAX)


def calibrate_scale(x_bf16_bits) -> np.float32:
    """Scale of a bf16 tensor: fl32(max|x| / 448).  max|x| is exact (a bf16 value); NaN is ignored."""
    return scale_from_absmax(np.uint32(absmax_bits(x_bf16_bits)).view(np.float32))


def absmax_bits(x_bf16_bits) -> np.uint32:
    """max|x| of a bf16 tensor as float32 bits (NaN inputs ignored)."""
    a = np.abs(f32_from_bf16(np.asarray(x_bf16_bits).ravel()))
    a = a[~np.isnan(a)]
    m = a.max() if a.size else np.float32(0)
    return np.float32(m).view(np.uint32)


def inv_scale(scale) -> np.float32:
    return np.float32(1.0) / np.float32(scale)


def quantize_e4m3(x_bf16_bits, scale) -> np.ndarray:
    """bf16 tensor -> e4m3 codes with a per-tensor scale: E(fl32(x * fl32(1/scale)))."""
    x = f32_from_bf16(x_bf16_bits)
    with np.errstate(over="ignore", invalid="ignore"):
        prod = (x * inv_scale(scale)).astype(np.float32)      # one fp32 rounding
    return e4m3_encode(prod)


def dequantize_e4m3(codes, scale) -> np.ndarray:
    """codes -> float64 dec(c) * scale (exact in fp64)."""
    return e4m3_decode(codes) * np.float64(np.float32(scale))
