"""Decode attention over a paged FP8 or BF16 KV cache, in fp64 (oracle; test infrastructure).

The Cloudflare post "Smaller, faster, safer: running Kimi and GLM at scale",
section "Quantized KV cache": at decode, the attention kernel reads the
cached K and V of every earlier token, and with an FP8 cache it converts the
stored values as it reads them.  What that computes has a plain definition,
written out here without blocking, split-K or online softmax (those are
exact rewrites of it up to floating-point rounding):

  K^_t = dec(K_t) * k_scale,  V^_t = dec(V_t) * v_scale        (FP8 cache)
  K^_t = K_t,                 V^_t = V_t                        (BF16 cache)
  s_t  = sm_scale * <q_h, K^_t>     for every token t < L of the request
  o_h  = sum_t softmax(s)_t * V^_t

Readings where the pages are silent: query head h reads KV head
g = h // (Hq / Hkv) (contiguous groups); sm_scale is passed in (1/sqrt(D) by
default); the request attends to positions [0, L) with L counting the token
appended this step; a request whose abort flag is set produces an all-zero
output row and reads no pages.  Latent cache: one vector c_t of width Dl per
token shared by every query head; K^_t = dec(c_t) * scale (all Dl dims) and
V^_t = the first Dv dims of it.
"""
from __future__ import annotations

import math

import numpy as np

from . import codec, paged


def softmax_attention(q, k, v, sm_scale):
    """q [H][D], k [L][D], v [L][Dv] in fp64 -> [H][Dv]; every query head reads the same k and v."""
    s = sm_scale * (q @ k.T)                      # [H][L]
    s = s - s.max(axis=1, keepdims=True)
    p = np.exp(s)
    return (p @ v) / p.sum(axis=1, keepdims=True)


def dequant_rows(codes_or_bits, dtype: str, scale):
    if dtype == "fp8":
        return codec.dequantize_e4m3(codes_or_bits, scale)
    return codec.f64_from_bf16(codes_or_bits)


def request_attention(q_r, k_rows, v_rows, num_kv_heads, sm_scale):
    """One request, GQA: q_r [Hq][D] fp64, k_rows [L][Hkv][D] fp64, v_rows [L][Hkv][Dv] fp64."""
    Hq = q_r.shape[0]
    G = Hq // num_kv_heads
    out = np.empty((Hq, v_rows.shape[2]), dtype=np.float64)
    for g in range(num_kv_heads):
        out[g * G:(g + 1) * G] = softmax_attention(q_r[g * G:(g + 1) * G], k_rows[:, g, :],
                                                   v_rows[:, g, :], sm_scale)
    return out


def decode_attention(q_bits, k_pool, v_pool, page_table, ctx_lens, *, num_kv_heads, page_size,
                     head_dim, v_dim, dtype, k_scale=1.0, v_scale=1.0, sm_scale=None,
                     flags=None, requests=None, latent=False):
    """Paged decode attention for the listed requests (all by default).

    q_bits: bf16 bits [B][Hq][D].  Pools: logical [P][Hkv][S][D] element arrays
    (e4m3 codes when dtype == "fp8", bf16 bits when "bf16"), as oracle.paged keeps them.
    Returns {r: fp64 [Hq][Dv]}; aborted requests (flags[r] != 0) and L <= 0
    give zero rows.
    """
    B, Hq, D = q_bits.shape
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(D)
    if requests is None:
        requests = range(B)
    out = {}
    for r in requests:
        L = int(ctx_lens[r])
        if L <= 0 or (flags is not None and int(flags[r]) != 0):
            out[r] = np.zeros((Hq, v_dim), dtype=np.float64)
            continue
        q = codec.f64_from_bf16(q_bits[r])
        if latent:
            c, _ = paged.gather(k_pool, None, page_table, r, L)
            c = dequant_rows(c, dtype, k_scale)[:, 0, :]            # [L][Dl]
            out[r] = softmax_attention(q, c, c[:, :v_dim], sm_scale)
        else:
            k, v = paged.gather(k_pool, v_pool, page_table, r, L)
            out[r] = request_attention(q, dequant_rows(k, dtype, k_scale), dequant_rows(v, dtype, v_scale),
                                       num_kv_heads, sm_scale)
    return out


def row_rel_error(got, ref):
    """Per (request, head) row: max|got - ref| / max|ref| (0 when both rows are zero)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    num = np.abs(got - ref).max(axis=-1)
    den = np.abs(ref).max(axis=-1)
    with np.errstate(invalid="ignore", divide="ignore"):
        e = np.where(den > 0, num / np.where(den > 0, den, 1.0), np.where(num > 0, np.inf, 0.0))
    return e
