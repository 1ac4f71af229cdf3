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

Codes and scales are held in their logical order (codes [N][K], scales [N][K/128]); how the library
packs them for its loads is not the oracle's concern.
"""
from __future__ import annotations

import numpy as np

from . import codec

G = 128                 # input channels per quantisation group
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


# ----------------------------------------------------------------------------- the GEMM

def gemm(x_bits, w_f64):
    """y [M][N] = x W^T in fp64 (x bf16 bits [M][K], W fp64 [N][K])."""
    return codec.f64_from_bf16(x_bits) @ np.asarray(w_f64, dtype=np.float64).T


def output_bf16(y_f64):
    """The GEMM's bf16 result: fp64 -> fp32 -> bf16 (round to nearest even at each step)."""
    return codec.bf16_from_f32(np.asarray(y_f64, dtype=np.float64).astype(np.float32))
