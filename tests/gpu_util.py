"""Helpers for the GPU parity tests: upload seeded inputs, build oracle and device caches side by side.

The oracle side and the device side read the same kvsynth arrays and share
nothing else: the oracle quantises, scatters and attends with oracle.*, the
device with the HIP library through its C ABI.
"""
from __future__ import annotations

import math
import sys

import numpy as np
import torch

import fp8_paged_kv_append_amd as kv
from kvsynth import workloads as wl
from oracle import attention, codec, paged
from tests import layout


def note(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def dev(a: np.ndarray) -> torch.Tensor:
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    elif a.dtype == np.uint32:
        a = a.view(np.int32)
    return torch.from_numpy(a).cuda()


def host(t: torch.Tensor, dtype) -> np.ndarray:
    return t.detach().cpu().numpy().view(dtype)


class Case:
    """One workload, filled into an oracle cache (numpy) and a device cache (HIP), plus a decode step's inputs."""

    def __init__(self, w: wl.Workload, kv_dtype: str, lens=None, stride=None, oracle_fill=True, stale=None,
                 calib_outliers=False):
        """calib_outliers: with K outliers in the workload, take the K scale over K as drawn (outliers
        included, nothing saturates) instead of over the outlier-free draw (outliers saturate)."""
        self.w, self.kv_dtype = w, kv_dtype
        self.lens = wl.ctx_lens(w) if lens is None else np.asarray(lens, dtype=np.int32)
        self.pt, self.stride = wl.page_table(w, self.lens, stride)
        self.k, self.v = wl.all_kv(w, self.lens)
        self.k_calib = self.k
        if w.outlier_frac > 0 and not calib_outliers:
            self.k_calib, _ = wl.all_kv(w, self.lens, outliers=False)
        self.req, self.pos = wl.token_index(self.lens)
        self.tags = wl.page_tags(w)
        self.stale = wl.stale_requests(w) if stale is None else np.asarray(stale)
        self.exp = wl.expected_tags(w, self.pt, self.lens, self.tags, self.stale)
        self.q = wl.queries(w)
        self.elt = 1 if kv_dtype == "fp8" else 2
        self.max_ctx = int(max(1, self.lens.max()))
        off = np.concatenate([[0], np.cumsum(self.lens.astype(np.int64))])
        self.off = off
        self.last = off[1:] - 1                       # each request's newest token (appended by the step)
        self.sm_scale = 1.0 / math.sqrt(w.head_dim)

        # ---- oracle
        self.o_k_scale = codec.calibrate_scale(self.k_calib) if kv_dtype == "fp8" else np.float32(1)
        if kv_dtype == "fp8" and not w.latent:
            self.o_v_scale = codec.calibrate_scale(self.v)
        else:
            self.o_v_scale = self.o_k_scale
        # the device pools start as random bytes in the library's layout; the oracle's logical pools
        # start as the same elements, mapped by the test-side layout rules
        self.kind_k = "latent" if w.latent else "k"
        self.kp0 = wl.pool_bytes(w, "k", self.elt)
        self.vp0 = None if w.latent else wl.pool_bytes(w, "v", self.elt)
        self.et = np.uint8 if self.elt == 1 else np.uint16
        self.k_shape = (w.num_pages, w.num_kv_heads, w.page_size, w.head_dim)
        self.v_shape = (w.num_pages, w.num_kv_heads, w.page_size, w.v_dim)
        if oracle_fill:
            self.okp = layout.from_device(self.kp0.view(self.et), self.kind_k, self.k_shape, self.elt)
            self.ovp = None if w.latent else layout.from_device(self.vp0.view(self.et), "v", self.v_shape, self.elt)
            if kv_dtype == "fp8":
                paged.append_fp8(self.okp, self.ovp, self.k, self.v, self.req, self.pos, self.pt, self.o_k_scale,
                                 self.o_v_scale)
            else:
                paged.append(self.okp, self.ovp, self.k, self.v, self.req, self.pos, self.pt)

        # ---- device
        self.desc = kv.pool_desc(w.num_pages, w.page_size, w.num_kv_heads, w.head_dim, w.v_dim)
        if kv_dtype == "fp8":
            self.dkp = dev(self.kp0)
            self.dvp = None if w.latent else dev(self.vp0)
        else:
            self.dkp = dev(self.kp0.view(np.uint16))
            self.dvp = None if w.latent else dev(self.vp0.view(np.uint16))
        self.dpt = dev(self.pt)
        self.dlens = dev(self.lens)
        self.dq = dev(self.q)
        self.dk = dev(self.k)
        self.dv = None if w.latent else dev(self.v)
        self.dreq, self.dpos = dev(self.req), dev(self.pos)
        self.dtags, self.dexp = dev(self.tags), dev(self.exp)
        if kv_dtype == "fp8":
            separate = w.outlier_frac > 0 and not calib_outliers
            dkc = dev(self.k_calib) if separate else self.dk
            self.d_k_scale = kv.calibrate_scale(dkc)
            self.d_v_scale = self.d_k_scale if w.latent else kv.calibrate_scale(self.dv)
            del dkc
        else:
            self.d_k_scale = self.d_v_scale = 1.0

    def device_k(self, t=None) -> np.ndarray:
        """The device K (or latent) pool mapped to the oracle's logical order [P][Hkv][S][D]."""
        return layout.from_device(host(self.dkp if t is None else t, self.et), self.kind_k, self.k_shape, self.elt)

    def device_v(self, t=None) -> np.ndarray:
        return layout.from_device(host(self.dvp if t is None else t, self.et), "v", self.v_shape, self.elt)

    def pools_match(self) -> bool:
        """Device pools equal the oracle's, element by element (pages never written included)."""
        if not np.array_equal(self.device_k(), self.okp):
            return False
        return self.w.latent or np.array_equal(self.device_v(), self.ovp)

    def fill_device(self):
        if self.kv_dtype == "fp8":
            kv.kv_append_fp8(self.desc, self.dkp, self.dvp, self.dk, self.dv, self.dreq, self.dpos, self.dpt,
                             k_scale=self.d_k_scale, v_scale=self.d_v_scale)
        else:
            kv.kv_append_bf16(self.desc, self.dkp, self.dvp, self.dk, self.dv, self.dreq, self.dpos, self.dpt)

    def step_inputs(self):
        """The decode step's new rows: each request re-appends its last token (same data, same slot)."""
        lr = np.maximum(self.last, 0)
        k_new = self.k[lr]
        v_new = None if self.w.latent else self.v[lr]
        req = np.arange(self.w.batch, dtype=np.int32)
        pos = (self.lens - 1).astype(np.int32)
        return k_new, v_new, req, pos

    def out_tensor(self):
        return torch.empty((self.w.batch, self.w.num_q_heads, self.w.v_dim), dtype=torch.int16, device="cuda")

    def workspace(self, splits):
        n = kv.paged_decode_attn_workspace_bytes(self.w.batch, self.w.num_q_heads, self.w.v_dim, splits)
        return torch.zeros(max(n, 16) // 4 + 4, dtype=torch.float32, device="cuda")   # zeroed once, as the library asks

    def attend(self, flags=None, num_splits=0, max_ctx=None):
        out = self.out_tensor()
        mc = self.max_ctx if max_ctx is None else max_ctx
        splits = num_splits or kv.paged_decode_attn_auto_splits(self.w.batch, self.w.num_kv_heads, mc)
        ws = self.workspace(splits)
        if self.kv_dtype == "fp8":
            kv.paged_decode_attn_fp8(self.desc, self.dq, self.dkp, self.dvp, self.dpt, self.dlens, mc, out, flags,
                                     k_scale=self.d_k_scale, v_scale=self.d_v_scale, sm_scale=self.sm_scale,
                                     num_splits=num_splits, workspace=ws)
        else:
            kv.paged_decode_attn_bf16(self.desc, self.dq, self.dkp, self.dvp, self.dpt, self.dlens, mc, out, flags,
                                      sm_scale=self.sm_scale, num_splits=num_splits, workspace=ws)
        torch.cuda.synchronize()
        return host(out, np.uint16)

    def oracle_attend(self, flags=None, requests=None):
        w = self.w
        return attention.decode_attention(self.q, self.okp, self.ovp, self.pt, self.lens,
                                          num_kv_heads=w.num_kv_heads, page_size=w.page_size, head_dim=w.head_dim,
                                          v_dim=w.v_dim, dtype=self.kv_dtype, k_scale=self.o_k_scale,
                                          v_scale=self.o_v_scale, sm_scale=self.sm_scale, flags=flags,
                                          requests=requests, latent=w.latent)

    def oracle_request(self, r):
        """fp64 attention for one request straight from its own rows (no pool), for large workloads."""
        w = self.w
        a, b = int(self.off[r]), int(self.off[r + 1])
        q = codec.f64_from_bf16(self.q[r])
        if self.kv_dtype == "fp8":
            kh = codec.dequantize_e4m3(codec.quantize_e4m3(self.k[a:b], self.o_k_scale), self.o_k_scale)
            vh = None if w.latent else codec.dequantize_e4m3(codec.quantize_e4m3(self.v[a:b], self.o_v_scale),
                                                             self.o_v_scale)
        else:
            kh = codec.f64_from_bf16(self.k[a:b])
            vh = None if w.latent else codec.f64_from_bf16(self.v[a:b])
        if w.latent:
            c = kh[:, 0, :]
            return attention.softmax_attention(q, c, c[:, :w.v_dim], self.sm_scale)
        return attention.request_attention(q, kh, vh, w.num_kv_heads, self.sm_scale)


def attn_error(got_bits: np.ndarray, ref: dict) -> float:
    """Largest row-normalised error over the requests in ref (bf16 device rows vs fp64 oracle rows)."""
    worst = 0.0
    for r, o in ref.items():
        g = codec.f64_from_bf16(got_bits[r])
        e = attention.row_rel_error(g, o)
        worst = max(worst, float(np.max(e)) if e.size else 0.0)
    return worst


ATTN_TOL = 1e-2   # max relative error per (request, head) row, bf16 output
