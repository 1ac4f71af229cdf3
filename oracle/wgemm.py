"""Weight-only quantised decode GEMM, INT4 (W4A16) and FP8 (W8A16) weights (oracle; test infrastructure).

The pages (Cloudflare post "Smaller, faster, safer: running Kimi and GLM at scale", section
"Compressed model weights" (压缩模型权重); agentlenshq summary, section "模型权重压缩以降低延迟"; xujun.org
note, section "INT4 权重：40% 更小的 checkpoint，一样的精度") compress GLM's weights from FP8 to INT4:
decode reads every weight once per token, so it is bound by memory bandwidth and gets faster with fewer
bytes; the INT4 weights are expanded to a wider type before the multiply, which is why prefill gets
slower.  They give neither the grouping nor the scale format.  Readings taken here:

* a weight matrix W is [N][K] (output channel n, input channel k); y[m][n] = sum_k x[m][k] * W[n][k]
  with bf16 activations x [M][K] and a bf16 result (fp64 here, rounded fp64 -> fp32 -> bf16);
* weights are quantised in groups of G = 128 consecutive input channels of one output channel, with
  one scale per group stored as bf16;
* INT4: symmetric signed codes q in [-8, 7]; scale s = bf16(fl32(max|w| / 7)) over the group;
  q = clamp(rint(fl32(w * fl32(1/s))), -8, 7) with ties to even; a group whose scale is 0 gets codes 0;
  the weight the GEMM uses is s * q;
* FP8 (the pages' baseline weights): e4m3 codes under the same grouping, s = bf16(fl32(max|w| / 448)),
  code = E(fl32(w * fl32(1/s))) with the KV cache's e4m3 encoder (RNE, saturating); weight s * dec(code);
* weights are finite (the offline quantiser is not defined on NaN or infinity).

Storage (the pages fix none; this is the library's layout, written out here as plain index rules):
* codes are grouped in tiles of 16 output channels x 128 input channels, tile (t, g) for channels
  n in [16t, 16t+16), k in [128g, 128g+128), tiles ordered t-major: tile index t * (K/128) + g;
* inside a tile, 64 lanes l = 16*qq + nn (qq in 0..3, nn in 0..15) each own output channel 16t + nn
  and, for j in 0..3 and e in 0..7, input channel k = 128g + 32j + 8qq + e;
* INT4: 16 bytes per lane, dword j holds the 8 codes of (j, e) as unsigned nibbles q + 8, e = 2*(s%4)
  + s//4 in nibble slot s (bits 4s..4s+3 of the little-endian dword);
* FP8: 32 bytes per lane, byte 8j + e holds the code of (j, e);
* scales: bf16 [N/16][K/128][16], element (t, g, nn) = scale of output channel 16t + nn in group g.
"""
from __future__ import annotations

import numpy as np

from . import codec

G = 128                 # input channels per quantisation group
TILE_N = 16             # output channels per storage tile
INT4_MAX = 7.0


def _groups(w_bits):
    """bf16 bits [N][K] -> fl32 values [N][K/G][G]."""
    w = codec.f32_from_bf16(np.asarray(w_bits, dtype=np.uint16))
    N, K = w.shape
    if K % G:
        raise ValueError(f"K = {K} is not a multiple of {G}")
    return w.reshape(N, K // G, G)


def _group_scale(wg, qmax):
    """bf16 scale bits [N][K/G]: bf16(fl32(max|w| / qmax))."""
    amax = np.max(np.abs(wg), axis=2).astype(np.float32)
    return codec.bf16_from_f32(amax / np.float32(qmax))


def _inv(s_bits):
    """fl32(1/s) per group, 0 where s = 0 (those groups get code 0)."""
    s = codec.f32_from_bf16(s_bits)
    with np.errstate(divide="ignore"):
        inv = np.where(s > 0, np.float32(1.0) / s, np.float32(0.0)).astype(np.float32)
    return inv


def quantize_w4(w_bits):
    """bf16 weights [N][K] -> (q int8 [N][K] in [-8, 7], scale bf16 bits [N][K/G])."""
    wg = _groups(w_bits)
    s = _group_scale(wg, INT4_MAX)
    prod = (wg * _inv(s)[:, :, None]).astype(np.float32)           # one fp32 rounding
    q = np.clip(np.rint(prod.astype(np.float64)), -8, 7).astype(np.int8)
    return q.reshape(wg.shape[0], -1), s


def quantize_w8(w_bits):
    """bf16 weights [N][K] -> (e4m3 codes uint8 [N][K], scale bf16 bits [N][K/G])."""
    wg = _groups(w_bits)
    s = _group_scale(wg, codec.E4M3_MAX)
    prod = (wg * _inv(s)[:, :, None]).astype(np.float32)
    return codec.e4m3_encode(prod).reshape(wg.shape[0], -1), s


def dequant_w4(q, s_bits):
    """fp64 [N][K] weights s * q."""
    N, K = q.shape
    s = codec.f64_from_bf16(s_bits)
    return (q.astype(np.float64).reshape(N, K // G, G) * s[:, :, None]).reshape(N, K)


def dequant_w8(codes, s_bits):
    N, K = codes.shape
    s = codec.f64_from_bf16(s_bits)
    return (codec.e4m3_decode(codes).reshape(N, K // G, G) * s[:, :, None]).reshape(N, K)


# ----------------------------------------------------------------------------- storage layout

def _lane_index(N, K):
    """For every (n, k): (tile index, lane, j, e) of the storage rule."""
    n = np.arange(N)[:, None]
    k = np.arange(K)[None, :]
    t, nn = n // TILE_N, n % TILE_N
    g, kk = k // G, k % G
    j, qq, e = kk // 32, (kk % 32) // 8, kk % 8
    tile = t * (K // G) + g
    lane = 16 * qq + nn
    return np.broadcast_arrays(tile, lane, j, e)


def _check_shape(N, K):
    if N % TILE_N or K % G:
        raise ValueError(f"N = {N} must be a multiple of {TILE_N} and K = {K} of {G}")


def pack_w4(q):
    """int8 codes [N][K] -> packed bytes (N*K/2) in the library's INT4 layout."""
    N, K = q.shape
    _check_shape(N, K)
    tile, lane, j, e = _lane_index(N, K)
    slot = (e % 2) * 4 + e // 2                     # inverse of e = 2*(s%4) + s//4
    nib = (q.astype(np.int64) + 8) & 0xF
    byte = (tile * 64 + lane) * 16 + 4 * j + slot // 2
    shift = 4 * (slot % 2)
    out = np.zeros(N * K // 2, dtype=np.int64)
    np.add.at(out, byte.ravel(), (nib << shift).ravel())
    return out.astype(np.uint8)


def unpack_w4(packed, N, K):
    _check_shape(N, K)
    tile, lane, j, e = _lane_index(N, K)
    slot = (e % 2) * 4 + e // 2
    byte = (tile * 64 + lane) * 16 + 4 * j + slot // 2
    nib = (np.asarray(packed, dtype=np.uint8)[byte].astype(np.int64) >> (4 * (slot % 2))) & 0xF
    return (nib - 8).astype(np.int8)


def pack_w8(codes):
    N, K = codes.shape
    _check_shape(N, K)
    tile, lane, j, e = _lane_index(N, K)
    out = np.zeros(N * K, dtype=np.uint8)
    out[((tile * 64 + lane) * 32 + 8 * j + e).ravel()] = np.asarray(codes, dtype=np.uint8).ravel()
    return out


def unpack_w8(packed, N, K):
    _check_shape(N, K)
    tile, lane, j, e = _lane_index(N, K)
    return np.asarray(packed, dtype=np.uint8)[(tile * 64 + lane) * 32 + 8 * j + e]


def pack_scales(s_bits):
    """bf16 bits [N][K/G] -> [N/16][K/G][16]."""
    N, KG = s_bits.shape
    return np.ascontiguousarray(np.asarray(s_bits, dtype=np.uint16).reshape(N // TILE_N, TILE_N, KG)
                                .transpose(0, 2, 1))


def unpack_scales(s_packed, N, K):
    return np.ascontiguousarray(np.asarray(s_packed, dtype=np.uint16).reshape(N // TILE_N, K // G, TILE_N)
                                .transpose(0, 2, 1).reshape(N, K // G))


# ----------------------------------------------------------------------------- the GEMM

def gemm(x_bits, w_f64):
    """y [M][N] = x W^T in fp64 (x bf16 bits [M][K], W fp64 [N][K])."""
    return codec.f64_from_bf16(x_bits) @ np.asarray(w_f64, dtype=np.float64).T


def output_bf16(y_f64):
    """The GEMM's bf16 result: fp64 -> fp32 -> bf16 (round to nearest even at each step)."""
    return codec.bf16_from_f32(np.asarray(y_f64, dtype=np.float64).astype(np.float32))
