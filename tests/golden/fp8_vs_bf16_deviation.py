#!/usr/bin/env python3
"""How far attention over the FP8 (e4m3) cache lands from attention over the BF16 cache, per workload
(information only: the Cloudflare post judges the FP8 cache by model evaluations, section "Quantized KV
cache", which no kernel test can stand in for; the agentlenshq summary notes that model families differ in
how much KV quantisation costs them).

Both sides are the oracle's fp64 attention: over K^ = dec(e4m3(K)) * k_scale, V^ = dec(e4m3(V)) * v_scale
with the per-tensor scales of the whole workload, and over the bf16 K, V themselves.  For sampled requests
of each workload: the row error max|o_fp8 - o_bf16| / max|o_bf16| per (request, head), its maximum and mean.

    python tests/golden/fp8_vs_bf16_deviation.py [--quick]   # writes tests/golden/fp8_vs_bf16_deviation.txt

Only the oracle and the seeded input generators are used.
"""
from __future__ import annotations

import argparse
import math
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

from kvsynth import workloads as wl  # noqa: E402
from oracle import attention, codec  # noqa: E402

OUT = os.path.join(os.path.dirname(os.path.abspath(__file__)), "fp8_vs_bf16_deviation.txt")


def scales(w, lens, outliers_in_k_scale):
    """Per-tensor scales over every request of the workload (absmax taken request by request)."""
    kmax = vmax = 0.0
    for r in range(w.batch):
        L = int(lens[r])
        k = wl.request_k(w, r, L, outliers=outliers_in_k_scale or w.outlier_frac == 0)
        kmax = max(kmax, float(np.uint32(codec.absmax_bits(k)).view(np.float32)))
        if not w.latent:
            vmax = max(vmax, float(np.uint32(codec.absmax_bits(wl.request_v(w, r, L))).view(np.float32)))
    ks = codec.scale_from_absmax(np.float32(kmax))
    vs = ks if w.latent else codec.scale_from_absmax(np.float32(vmax))
    return ks, vs


def request_rows(w, r, L, q, ks, vs):
    """(o over the FP8 cache, o over the BF16 cache), fp64 [Hq][Dv], for request r."""
    sm = 1.0 / math.sqrt(w.head_dim)
    k = wl.request_k(w, r, L)
    qr = codec.f64_from_bf16(q[r])
    if w.latent:
        c8 = codec.dequantize_e4m3(codec.quantize_e4m3(k, ks), ks)[:, 0, :]
        c16 = codec.f64_from_bf16(k)[:, 0, :]
        return (attention.softmax_attention(qr, c8, c8[:, :w.v_dim], sm),
                attention.softmax_attention(qr, c16, c16[:, :w.v_dim], sm))
    v = wl.request_v(w, r, L)
    o8 = attention.request_attention(qr, codec.dequantize_e4m3(codec.quantize_e4m3(k, ks), ks),
                                     codec.dequantize_e4m3(codec.quantize_e4m3(v, vs), vs), w.num_kv_heads, sm)
    o16 = attention.request_attention(qr, codec.f64_from_bf16(k), codec.f64_from_bf16(v), w.num_kv_heads, sm)
    return o8, o16


def run(name, w, requests, outliers_in_k_scale=False):
    lens = wl.ctx_lens(w)
    ks, vs = scales(w, lens, outliers_in_k_scale)
    q = wl.queries(w)
    errs = []
    for r in requests:
        o8, o16 = request_rows(w, r, int(lens[r]), q, ks, vs)
        errs.append(attention.row_rel_error(o8, o16))
    e = np.concatenate(errs)
    return (f"{name:34s} {len(requests):3d} req  L {int(min(lens[requests])):6d}-{int(max(lens[requests])):6d}  "
            f"row error max {e.max():.3e}  mean {e.mean():.3e}  k_scale {float(ks):.6g}")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--quick", action="store_true", help="the tiny workload only, printed, nothing written")
    args = ap.parse_args()
    W = wl.WORKLOADS
    lines = [run("tiny (1 x 256)", W["tiny"], [0])]
    if args.quick:
        print(lines[0])
        return
    g = W["gqa_batch"]
    order = np.argsort(wl.ctx_lens(g), kind="stable")
    lines.append(run("gqa_batch (32 x 1024-8192)", g, sorted({int(order[0]), int(order[len(order) // 2]),
                                                               int(order[-1])})))
    lines.append(run("sweep (B x 8192, requests 0, 17)", W["sweep_b64"], [0, 17]))
    lines.append(run("long (4 x 131072), outliers saturate", W["long"], [3]))
    lines.append(run("long, K scale over the outliers", W["long"], [3], outliers_in_k_scale=True))
    lines.append(run("latent (64 x 4096, 576 / 512)", W["latent"], [0, 31, 63]))
    text = ("# FP8 (e4m3) cache against BF16 cache: fp64 attention on both, row error max|o8 - o16| / max|o16|\n"
            "# written by tests/golden/fp8_vs_bf16_deviation.py (oracle only); information, not a pass bar\n" +
            "\n".join(lines) + "\n")
    open(OUT, "w").write(text)
    print(text, end="")


if __name__ == "__main__":
    main()
