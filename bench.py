#!/usr/bin/env python3
"""Decode-step benchmark on one MI355X: FP8 (e4m3) vs BF16 paged KV cache.

A step is one pass of the whole hot path for one attention layer over one
batch: the batched page-tag check, the append of every request's new token
(quantised to e4m3 for the FP8 cache) and paged decode attention (split
kernel + log-sum-exp merge when the context is split).  By default the step
is kv_decode_step_* over that one layer, which is a single
launch: every attention block checks its request's page tags before reading
any page, and the block holding position L-1 writes the new token
(--two-launch: check + write launch, then attention; --unfused: three
launches).  Inputs are resident in HBM before timing starts.  Default workload: 64 requests x 8192 tokens,
64 query / 8 KV heads, head_dim 128, page size 16, 40,000-page pool, one
stale expected tag (1% of requests, that request aborted and its bytes
excluded).

Prints one JSON line (rank 0).  Metric: KV-read GB/s of the whole step
(algorithmic bytes: sum over non-aborted requests of L * Hkv * D * 2 * bytes
per element) and steps/s.  Further sections of the line: the flushed batch
sweep, admission under a fixed byte budget (FP8 vs BF16 through the page
allocator), a whole decode step over a 61-layer stack (eager and HIP graph,
tracker on and off), the INT4- vs FP8-weight decode GEMM, the other
workloads (ragged batch, long context, latent cache) and the CPU oracle.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, 8.0 TB/s
BF16_MFMA_PEAK_TFLOPS = 2500.0 # MI355X dense bf16 matrix peak
FP8_MFMA_PEAK_TFLOPS = 5000.0  # MI355X dense fp8 matrix peak
METRIC = "decode-attn KV-read GB/s (% of HBM peak) + steps/s, FP8 vs BF16 KV cache"


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--workload", default="sweep_b64")
    p.add_argument("--splits", type=int, default=0, help="0 = library choice")
    p.add_argument("--batch", type=int, default=0,
                   help="requests of the main workload (0 = the workload's own; its page pool is kept)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-bf16", action="store_true")
    p.add_argument("--no-extra", action="store_true", help="skip the other workloads (GQA batch, long, latent)")
    p.add_argument("--no-sweep", action="store_true", help="skip the batch sweep B = 1, 8, 16, 32, 64")
    p.add_argument("--no-capacity", action="store_true",
                   help="skip the fixed-budget admission of 8192-token requests (FP8 vs BF16)")
    p.add_argument("--no-layers", action="store_true",
                   help="skip the whole-step runs over a layer stack (eager and HIP-graph replays)")
    p.add_argument("--layers", type=int, default=61, help="layers in the layer-stack step")
    p.add_argument("--layer-batches", default="1,8,64",
                   help="batch sizes of the layer-stack step (the latent cache runs those of them in {1, 64})")
    p.add_argument("--layers-only", action="store_true",
                   help="run only the layer-stack step (skips the headline workload's timing)")
    p.add_argument("--no-weights", action="store_true",
                   help="skip the weight-quantised decode GEMM runs (INT4 vs FP8 weights)")
    p.add_argument("--weights-only", action="store_true", help="run only the weight-quantised GEMM section")
    p.add_argument("--capacity-ref-batch", type=int, default=32,
                   help="the byte budget is what this many 8192-token requests take in the BF16 cache")
    p.add_argument("--flush-mib", type=int, default=512,
                   help="size of the write that evicts the 256 MB Infinity Cache before each flushed step")
    p.add_argument("--cpu-sample", type=int, default=8, help="requests in the CPU oracle sample")
    p.add_argument("--fp8-only-steps", action="store_true", help="time only the FP8 step (profiling runs)")
    p.add_argument("--unfused", action="store_true",
                   help="tag check, append and attention as three launches")
    p.add_argument("--two-launch", action="store_true",
                   help="kv_tag_check_append_* then the attention (default: kv_decode_step_* over one layer, "
                        "one launch: check, write and attention; BF16 latent: a check + write launch first)")
    p.add_argument("--graph", action="store_true",
                   help="time replays of a captured HIP graph of one step (default: eager launches)")
    p.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                   help="after timing, copy a MIB-MiB buffer 3 times (a known-size kernel for HBM counters)")
    return p.parse_args()


class DeviceCache:
    """One workload's cache on the device (FP8 or BF16), filled through the library's append."""

    def __init__(self, w, kv_dtype, host, torch, kv, fused=True, one_launch=True):
        self.w, self.kv_dtype, self.torch, self.kv = w, kv_dtype, torch, kv
        self.fused = fused
        # the library's whole step (kv_decode_step_* over one layer): one launch (plus the merge when split);
        # the BF16 latent cache keeps a check + write launch before it
        self.one_launch = fused and one_launch
        nk = w.num_pages * w.num_kv_heads * w.page_size * w.head_dim
        nv = w.num_pages * w.num_kv_heads * w.page_size * w.v_dim
        tdt = torch.uint8 if kv_dtype == "fp8" else torch.int16
        # pool contents before the fill do not matter for timing: zero them on the device
        self.kp = torch.zeros(nk, dtype=tdt, device="cuda")
        self.vp = None if w.latent else torch.zeros(nv, dtype=tdt, device="cuda")
        self.desc = kv.pool_desc(w.num_pages, w.page_size, w.num_kv_heads, w.head_dim, w.v_dim)
        self.pt, self.lens, self.q = host["dpt"], host["dlens"], host["dq"]
        self.tags, self.exp = host["dtags"], host["dexp"]
        self.max_ctx = host["max_ctx"]
        dv = None if w.latent else host["dv"]
        if kv_dtype == "fp8":
            self.k_scale = kv.calibrate_scale(host["dk_calib"])
            self.v_scale = self.k_scale if w.latent else kv.calibrate_scale(dv)
            kv.kv_append_fp8(self.desc, self.kp, self.vp, host["dk"], dv, host["dreq"], host["dpos"],
                             self.pt, k_scale=self.k_scale, v_scale=self.v_scale)
        else:
            self.k_scale = self.v_scale = 1.0
            kv.kv_append_bf16(self.desc, self.kp, self.vp, host["dk"], dv, host["dreq"], host["dpos"], self.pt)
        self.k_new, self.v_new = host["dk_new"], host["dv_new"]
        self.s_req, self.s_pos = host["ds_req"], host["ds_pos"]
        self.out = torch.empty((w.batch, w.num_q_heads, w.v_dim), dtype=torch.int16, device="cuda")
        self.flags = torch.zeros(w.batch, dtype=torch.int32, device="cuda")
        # latent: with no requested count the library picks per cache type (FP8 and BF16 work on different
        # head groups); the workspace is sized with the public bound, which covers both
        self.lat_splits = host["splits"] if w.latent else None
        if host["splits"]:
            self.splits = host["splits"]
        elif w.latent:
            self.splits = kv.paged_decode_attn_latent_auto_splits(w.batch, w.num_q_heads, self.max_ctx)
        else:
            self.splits = kv.paged_decode_attn_auto_splits(w.batch, w.num_kv_heads, self.max_ctx)
        n = kv.paged_decode_attn_workspace_bytes(w.batch, w.num_q_heads, w.v_dim, self.splits)
        self.ws = torch.empty(max(n // 4, 4), dtype=torch.float32, device="cuda")
        torch.cuda.synchronize()

    def check(self):
        self.kv.kv_tag_check(self.tags, self.pt, self.exp, self.lens, self.w.page_size, self.flags)

    def check_append(self):
        """The tag check and the write of one token per request as one launch."""
        if self.kv_dtype == "fp8":
            self.kv.kv_tag_check_append_fp8(self.desc, self.kp, self.vp, self.k_new, self.v_new, self.pt, self.lens,
                                            self.tags, self.exp, self.flags, k_scale=self.k_scale,
                                            v_scale=self.v_scale)
        else:
            self.kv.kv_tag_check_append_bf16(self.desc, self.kp, self.vp, self.k_new, self.v_new, self.pt,
                                             self.lens, self.tags, self.exp, self.flags)

    def append(self, tracker=True):
        f = self.flags if tracker else None
        if self.kv_dtype == "fp8":
            self.kv.kv_append_fp8(self.desc, self.kp, self.vp, self.k_new, self.v_new, self.s_req, self.s_pos,
                                  self.pt, f, k_scale=self.k_scale, v_scale=self.v_scale)
        else:
            self.kv.kv_append_bf16(self.desc, self.kp, self.vp, self.k_new, self.v_new, self.s_req, self.s_pos,
                                   self.pt, f)

    def attend(self, tracker=True):
        f = self.flags if tracker else None
        kv, w = self.kv, self.w
        if w.latent and self.kv_dtype == "fp8":
            kv.paged_decode_attn_latent_fp8(self.desc, self.q, self.kp, self.pt, self.lens, self.max_ctx, self.out, f,
                                            scale=self.k_scale, num_splits=self.lat_splits, workspace=self.ws)
        elif w.latent:
            kv.paged_decode_attn_latent_bf16(self.desc, self.q, self.kp, self.pt, self.lens, self.max_ctx, self.out,
                                             f, num_splits=self.lat_splits, workspace=self.ws)
        elif self.kv_dtype == "fp8":
            kv.paged_decode_attn_fp8(self.desc, self.q, self.kp, self.vp, self.pt, self.lens, self.max_ctx,
                                     self.out, f, k_scale=self.k_scale, v_scale=self.v_scale,
                                     num_splits=self.splits, workspace=self.ws)
        else:
            kv.paged_decode_attn_bf16(self.desc, self.q, self.kp, self.vp, self.pt, self.lens, self.max_ctx,
                                      self.out, f, num_splits=self.splits, workspace=self.ws)

    def lib_step(self, tracker=True):
        """kv_decode_step_* over this one layer: a single launch in which every block checks its request's
        page tags, the block(s) holding position L - 1 write the new token, and the attention runs (plus
        the merge when split); GQA and latent caches alike."""
        self.kv.decode_step(self.desc, self.kv_dtype, self.kp, self.vp, self.pt, self.lens, self.max_ctx, self.q,
                            self.k_new, self.v_new, None, None, self.out, page_tags=self.tags if tracker else None,
                            expected_tags=self.exp if tracker else None, abort_flags=self.flags if tracker else None,
                            k_scale=self.k_scale, v_scale=self.v_scale,
                            num_splits=self.lat_splits if self.w.latent else self.splits, workspace=self.ws)

    def step(self, tracker=True):
        if self.one_launch:
            self.lib_step(tracker)
            return
        if tracker and self.fused:
            self.check_append()
        else:
            if tracker:
                self.check()
            self.append(tracker)
        self.attend(tracker)

    def run(self, steps, warmup, tracker=True, graph=False):
        """Time `steps` back-to-back steps between two events on the launch stream (torch's current
        stream), eagerly or as replays of a captured graph of one step."""
        torch = self.torch
        for _ in range(warmup):
            self.step(tracker)
        torch.cuda.synchronize()
        if graph:
            g = torch.cuda.CUDAGraph()
            side = torch.cuda.Stream()
            side.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(side):
                self.step(tracker)
            torch.cuda.current_stream().wait_stream(side)
            with torch.cuda.graph(g):
                self.step(tracker)
            for _ in range(warmup):
                g.replay()
            torch.cuda.synchronize()
            fn = g.replay
        else:
            fn = lambda: self.step(tracker)  # noqa: E731
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        wall0 = time.perf_counter()
        t0.record()
        for _ in range(steps):
            fn()
        t1.record()
        torch.cuda.synchronize()
        wall = time.perf_counter() - wall0
        total_ms = t0.elapsed_time(t1)
        return dict(ms_per_step=total_ms / steps, wall_ms_per_step=1e3 * wall / steps)

    def run_flushed(self, steps, warmup, flush):
        """Per-step times with a cache-evicting write before every step, outside the event window:
        events before the step, after the check (+ append) and after the attention."""
        torch = self.torch
        for _ in range(warmup):
            flush.add_(1)
            self.step()
        torch.cuda.synchronize()
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
        for e in evs:
            flush.add_(1)
            e[0].record()
            if self.one_launch:  # the whole step is the one launch: it lands in the attention column
                e[1].record()
                self.lib_step()
                e[2].record()
                continue
            if self.fused:
                self.check_append()
            else:
                self.check()
                self.append()
            e[1].record()
            self.attend()
            e[2].record()
        torch.cuda.synchronize()
        per = np.array([[e[0].elapsed_time(e[1]), e[1].elapsed_time(e[2])] for e in evs])
        step = per.sum(axis=1)
        return dict(step_ms=float(np.median(step)), step_ms_p95=float(np.percentile(step, 95)),
                    attn_ms=float(np.median(per[:, 1])), attn_ms_p95=float(np.percentile(per[:, 1], 95)),
                    check_append_ms=float(np.median(per[:, 0])))

    def breakdown(self, steps, tracker=True):
        """Per-kernel durations: an event before and after each launch of every step."""
        torch = self.torch
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(steps)]
        torch.cuda.synchronize()
        for e in evs:
            e[0].record()
            if self.one_launch:  # one launch: check, write and attention are in the attention column
                e[1].record()
                e[2].record()
                self.lib_step(tracker)
                e[3].record()
                continue
            if tracker and self.fused:
                self.check_append()
            elif tracker:
                self.check()
            e[1].record()
            if not (tracker and self.fused):
                self.append(tracker)
            e[2].record()
            self.attend(tracker)
            e[3].record()
        torch.cuda.synchronize()
        per = np.array([[e[0].elapsed_time(e[1]), e[1].elapsed_time(e[2]), e[2].elapsed_time(e[3])] for e in evs])
        return dict(check_ms=float(np.median(per[:, 0])), append_ms=float(np.median(per[:, 1])),
                    attn_ms=float(np.median(per[:, 2])), attn_ms_mean=float(per[:, 2].mean()),
                    attn_ms_p95=float(np.percentile(per[:, 2], 95)),
                    step_ms_p95=float(np.percentile(per.sum(axis=1), 95)))


def capacity_admission(kv, w, kvd, budget_bytes, seed=0):
    """Admit requests of w.ctx_hi tokens through the library's page allocator until it reports too few free
    pages (KVFP8_ERR_NOSPACE), with the pool sized to a byte budget.

    A page costs its K and V elements plus three uint32 words: its tag, one page-table entry and one
    expected-tag entry; the FP8 cache also keeps its two float scales.  Before admission the free list is
    churned into a seeded random order (every page allocated once, then freed in a shuffled order), as in a
    pool that has been serving for a while.  Returns the pool size, the admitted page table and the tags."""
    S = w.page_size
    elt = 1 if kvd == "fp8" else 2
    page_bytes = S * w.num_kv_heads * (w.head_dim + w.v_dim) * elt + 3 * 4
    fixed = 2 * 4 if kvd == "fp8" else 0
    P = int((budget_bytes - fixed) // page_bytes)
    alloc = kv.PageAllocator(P)
    pages, _ = alloc.alloc(P)
    alloc.free(np.random.default_rng(seed).permutation(pages))
    need = -(-int(w.ctx_hi) // S)
    rows = []
    while True:
        try:
            p, _ = alloc.alloc(need)
        except kv.KvFp8Error as e:
            if e.status != kv.KVFP8_ERR_NOSPACE:
                raise
            break
        rows.append(p)
    table = np.stack(rows) if rows else np.zeros((0, need), dtype=np.int32)
    return dict(num_pages=P, page_bytes=page_bytes, admitted=len(rows), pages_left=alloc.free_count,
                token_capacity=P * S, page_table=table, tags=alloc.tags())


def measured_traffic(workload, splits):
    """HBM bytes per launch of the FP8 attention kernel from the committed counter runs, or None when the
    kernel's sources changed since those counters were taken (or they cover another launch shape)."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "attn_fp8_64x8192_traffic.json")
    if not os.path.exists(path):
        return None
    d = json.load(open(path))
    h = hashlib.sha256()
    for src in d["kernel_sources"]:
        h.update(open(os.path.join(ROOT, src), "rb").read())
    if h.hexdigest() != d["kernel_sources_sha256"] or d["workload"] != workload or d["splits"] != splits:
        return None
    return d["traffic_bytes"]


def cpu_baseline(w, n_req, min_seconds=10.0):
    """The oracle's step (tag check, e4m3 append of one token per request, fp64 attention) on a sample."""
    from concurrent.futures import ThreadPoolExecutor  # noqa: F401
    from threadpoolctl import threadpool_limits

    from kvsynth import workloads as wl
    from oracle import codec, paged, step

    ws = w.with_(batch=n_req, num_pages=int(wl.pages_needed(wl.ctx_lens(w.with_(batch=n_req)), w.page_size).sum()),
                 stale=False)
    lens = wl.ctx_lens(ws)
    pt, _ = wl.page_table(ws, lens)
    k, v = wl.all_kv(ws, lens)
    req, pos = wl.token_index(lens)
    ks, vs = codec.calibrate_scale(k), codec.calibrate_scale(v)
    kp, vp = wl.pool_init(ws, "k", 1), wl.pool_init(ws, "v", 1)
    paged.append_fp8(kp, vp, k, v, req, pos, pt, ks, vs)
    tags = wl.page_tags(ws)
    st = dict(dtype="fp8", k_pool=kp, v_pool=vp, page_table=pt, ctx_lens=lens, page_tags=tags,
              expected_tags=wl.expected_tags(ws, pt, lens, tags), num_kv_heads=ws.num_kv_heads,
              page_size=ws.page_size, head_dim=ws.head_dim, v_dim=ws.v_dim, k_scale=ks, v_scale=vs,
              sm_scale=1 / math.sqrt(ws.head_dim), latent=False)
    last = np.cumsum(lens) - 1
    workers = min(16, os.cpu_count() or 1, n_req)
    times = []
    with threadpool_limits(1):
        while len(times) < 3 or sum(times) < min_seconds:
            t = time.perf_counter()
            step.decode_step(st, wl.queries(ws), k[last], v[last], np.arange(n_req, dtype=np.int32),
                             (lens - 1).astype(np.int32), workers=workers)
            times.append(time.perf_counter() - t)
    dt = float(np.median(times))
    kv_bytes = int(lens.astype(np.int64).sum()) * ws.num_kv_heads * ws.head_dim * 2
    return {"value": kv_bytes / dt / 1e9, "unit": "GB/s", "cores": workers, "kind": "oracle",
            "sample": f"{n_req} of {w.batch} requests of {w.name} (same shapes, FP8 cache), one decode step "
                      f"(tag check + e4m3 append + fp64 attention), median of {len(times)} runs "
                      f"({sum(times):.1f} s of CPU time in all): {dt:.2f} s per step",
            "seconds": dt}


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on exactly one GPU; the decode path is single-GPU "
                                   "(requests or KV heads would shard across GPUs with no exchange)",
                          "n_gpus": args.gpus}))
        sys.exit(2)
    import torch

    import fp8_paged_kv_append_amd as kv
    from kvsynth import workloads as wl

    def dev(a):
        a = np.ascontiguousarray(a)
        if a.dtype == np.uint16:
            a = a.view(np.int16)
        elif a.dtype == np.uint32:
            a = a.view(np.int32)
        return torch.from_numpy(a).cuda()

    def prepare(w, splits, table=None):
        """Generate one workload's inputs on the host and move them to the device.  table = (page table,
        page tags) from the page allocator replaces the drawn ones."""
        t = time.perf_counter()
        lens = wl.ctx_lens(w)
        if table is None:
            pt, _ = wl.page_table(w, lens)
            tags = wl.page_tags(w)
        else:
            pt, tags = table
        stale = wl.stale_requests(w)
        exp = wl.expected_tags(w, pt, lens, tags, stale)
        k, v = wl.all_kv(w, lens)
        req, pos = wl.token_index(lens)
        q = wl.queries(w)
        last = np.cumsum(lens.astype(np.int64)) - 1
        host = dict(dpt=dev(pt), dlens=dev(lens), dq=dev(q), dtags=dev(tags), dexp=dev(exp), dk=dev(k),
                    dv=None if v is None else dev(v), dreq=dev(req), dpos=dev(pos), dk_new=dev(k[last]),
                    dv_new=None if v is None else dev(v[last]), ds_req=dev(np.arange(w.batch, dtype=np.int32)),
                    ds_pos=dev((lens - 1).astype(np.int32)), max_ctx=int(lens.max()), splits=splits)
        host["dk_calib"] = host["dk"]
        if w.outlier_frac > 0:               # the K scale comes from the outlier-free draw
            kc, _ = wl.all_kv(w, lens, outliers=False)
            host["dk_calib"] = dev(kc)
            del kc
        del k, v
        live = np.ones(w.batch, dtype=bool)
        live[stale] = False
        row = w.head_dim if w.latent else w.num_kv_heads * (w.head_dim + w.v_dim)
        elems = int(lens[live].astype(np.int64).sum()) * row
        flops = int(lens[live].astype(np.int64).sum()) * w.num_q_heads * (w.head_dim + w.v_dim) * 2
        log(f"{w.name}: inputs ready in {time.perf_counter() - t:.1f} s")
        return host, stale, elems, flops

    flush = torch.zeros((args.flush_mib << 20) // 4, dtype=torch.int32, device="cuda")

    def measure(w, kvd, host, stale, elems, steps, warmup, full=True, flushed=False):
        t = time.perf_counter()
        c = DeviceCache(w, kvd, host, torch, kv, fused=not args.unfused, one_launch=not args.two_launch)
        log(f"{w.name} {kvd}: cache filled in {time.perf_counter() - t:.1f} s, splits={c.splits}")
        elt = 1 if kvd == "fp8" else 2
        if flushed:
            r = c.run_flushed(steps, warmup, flush)
            r["kv_bytes"] = elems * elt
            r["gbs_attn"] = r["kv_bytes"] / (r["attn_ms"] * 1e-3) / 1e9
            r["gbs_step"] = r["kv_bytes"] / (r["step_ms"] * 1e-3) / 1e9
            r["splits"] = c.splits
            flags = c.flags.cpu().numpy().view(np.uint32)
            assert np.flatnonzero(flags).tolist() == stale.tolist(), "abort flags differ from the planted stale set"
            log(f"{w.name} {kvd} flushed: " + json.dumps({k_: (round(v_, 4) if isinstance(v_, float) else v_)
                                                          for k_, v_ in r.items()}))
            del c
            torch.cuda.empty_cache()
            return r
        r = c.run(steps, warmup, tracker=True, graph=args.graph)
        if full:
            r["other"] = c.run(steps, warmup, tracker=True, graph=not args.graph)
        r.update(c.breakdown(steps, tracker=True))
        flags = c.flags.cpu().numpy().view(np.uint32)
        assert np.flatnonzero(flags).tolist() == stale.tolist(), "abort flags differ from the planted stale set"
        if full and not args.fp8_only_steps:
            r["no_tracker"] = c.run(steps, warmup, tracker=False, graph=args.graph)
            r["flushed"] = c.run_flushed(steps, warmup, flush)
        r["kv_bytes"] = elems * elt
        r["gbs_step"] = r["kv_bytes"] / (r["ms_per_step"] * 1e-3) / 1e9
        r["gbs_attn"] = r["kv_bytes"] / (r["attn_ms_mean"] * 1e-3) / 1e9
        r["splits"] = c.splits
        log(f"{w.name} {kvd}: " + json.dumps({k_: (round(v_, 4) if isinstance(v_, float) else v_)
                                              for k_, v_ in r.items() if k_ not in ("no_tracker", "other")}))
        del c
        torch.cuda.empty_cache()
        return r

    def measure_layers(w, kvd, host, stale, n_layers, steps, warmup):
        """One decode step over n_layers layers (each layer's pool a copy of layer 0's), as one
        kv_decode_step_* call: eager, and replayed from captured HIP graphs, tracker on and off."""
        c = DeviceCache(w, kvd, host, torch, kv, fused=True)
        kps = torch.empty((n_layers, c.kp.numel()), dtype=c.kp.dtype, device="cuda")
        kps.copy_(c.kp.unsqueeze(0).expand(n_layers, -1))
        vps = None
        if c.vp is not None:
            vps = torch.empty((n_layers, c.vp.numel()), dtype=c.vp.dtype, device="cuda")
            vps.copy_(c.vp.unsqueeze(0).expand(n_layers, -1))
        c.kp = c.vp = None
        q = c.q.unsqueeze(0).expand(n_layers, *c.q.shape).contiguous()
        k_new = c.k_new.unsqueeze(0).expand(n_layers, *c.k_new.shape).contiguous()
        v_new = None if c.v_new is None else c.v_new.unsqueeze(0).expand(n_layers, *c.v_new.shape).contiguous()
        out = torch.empty((n_layers,) + tuple(c.out.shape), dtype=torch.int16, device="cuda")
        fp8 = kvd == "fp8"
        ks = [c.k_scale] * n_layers if fp8 else None
        vs = [c.v_scale] * n_layers if fp8 and not w.latent else None

        def one(tracker):
            kv.decode_step_layers(c.desc, kvd, kps, vps, c.pt, c.lens, c.max_ctx, q, k_new, v_new, out,
                                  page_tags=c.tags if tracker else None, expected_tags=c.exp if tracker else None,
                                  abort_flags=c.flags if tracker else None, k_scales=ks, v_scales=vs,
                                  workspace=c.ws)

        def timed(fn):
            for _ in range(warmup):
                fn()
            torch.cuda.synchronize()
            t0 = torch.cuda.Event(enable_timing=True)
            t1 = torch.cuda.Event(enable_timing=True)
            t0.record()
            for _ in range(steps):
                fn()
            t1.record()
            torch.cuda.synchronize()
            return 1e3 * t0.elapsed_time(t1) / steps

        res = {"eager_us": timed(lambda: one(True))}
        for tracker in (True, False):
            g = torch.cuda.CUDAGraph()
            side = torch.cuda.Stream()
            side.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(side):
                one(tracker)
            torch.cuda.current_stream().wait_stream(side)
            with torch.cuda.graph(g):
                one(tracker)
            res["graph_us" if tracker else "graph_no_tracker_us"] = timed(g.replay)
            del g
        flags = c.flags.cpu().numpy().view(np.uint32)
        assert np.flatnonzero(flags).tolist() == stale.tolist(), "abort flags differ from the planted stale set"
        r = {k_: round(v_, 2) for k_, v_ in res.items()}
        r["layers"] = n_layers
        r["per_layer_us"] = round(res["graph_us"] / n_layers, 2)
        r["steps_per_s"] = round(1e6 / res["graph_us"], 1)
        r["tokens_per_s"] = round((w.batch - len(stale)) * 1e6 / res["graph_us"], 1)
        r["check_overhead_pct"] = round(100 * (res["graph_us"] / res["graph_no_tracker_us"] - 1), 2)
        r["splits"] = c.splits
        log(f"{w.name} {kvd} x{n_layers} layers: " + json.dumps(r))
        del c, kps, vps, q, k_new, v_new, out
        torch.cuda.empty_cache()
        return r

    def measure_weights(reps=20):
        """The weight-quantised decode GEMM over a stack of 16 distinct 8192 x 8192 weight matrices
        (0.5 GB of INT4 codes / 1 GB of FP8 codes, so every pass streams from HBM), y = x W^T for
        M = 1..64 activation rows, INT4 (W4A16) and FP8 (W8A16) weights, the whole stack captured in
        one HIP graph and timed by replay."""
        from kvsynth import weights as wsyn
        sh = wsyn.SHAPES["stack_8k"]
        N, K, L = sh.n, sh.k, sh.layers
        gen = torch.Generator(device="cuda")
        out = {"workload": f"{L} weight matrices of {N} x {K} (bf16 N(0, 0.02^2) drawn on the device with a "
                           f"seeded generator, quantised by the library), y = x W^T per matrix",
               "bytes_per_matrix": {"int4": N * K // 2 + N * K // 128 * 2, "fp8": N * K + N * K // 128 * 2}}
        for bits in (4, 8):
            gen.manual_seed(sh.seed)
            packs, scs = [], []
            for _ in range(L):
                wf = (torch.randn(N, K, device="cuda", generator=gen) * 0.02).to(torch.bfloat16)
                pk = torch.empty(N * K // (2 if bits == 4 else 1), dtype=torch.uint8, device="cuda")
                sc = torch.empty(N * K // 128, dtype=torch.int16, device="cuda")
                (kv.w4_quantize_bf16 if bits == 4 else kv.w8_quantize_bf16)(wf, pk, sc)
                packs.append(pk)
                scs.append(sc)
                del wf
            torch.cuda.synchronize()
            f = kv.w4a16_gemm if bits == 4 else kv.w8a16_gemm
            res = {}
            for m in (1, 8, 16, 32, 64):
                x = (torch.randn(m, K, device="cuda", generator=gen)).to(torch.bfloat16)
                y = torch.empty(m, N, dtype=torch.bfloat16, device="cuda")
                sp = kv.wgemm_auto_splits(m, N, K)
                ws = torch.empty(max(kv.wgemm_workspace_bytes(m, N, K, sp), 16) // 4 + 4, dtype=torch.float32,
                                 device="cuda")

                def stack():
                    for li in range(L):
                        f(x, packs[li], scs[li], N, K, y, workspace=ws)

                stack()
                torch.cuda.synchronize()
                g = torch.cuda.CUDAGraph()
                side = torch.cuda.Stream()
                side.wait_stream(torch.cuda.current_stream())
                with torch.cuda.stream(side):
                    stack()
                torch.cuda.current_stream().wait_stream(side)
                with torch.cuda.graph(g):
                    stack()
                for _ in range(3):
                    g.replay()
                torch.cuda.synchronize()
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                e0.record()
                for _ in range(reps):
                    g.replay()
                e1.record()
                torch.cuda.synchronize()
                us = 1e3 * e0.elapsed_time(e1) / (reps * L)
                gbs = out["bytes_per_matrix"]["int4" if bits == 4 else "fp8"] / (us * 1e-6) / 1e9
                res[f"M{m}"] = {"us_per_gemm": round(us, 2), "weight_gbs": round(gbs, 1),
                                "pct_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 2),
                                "stack_passes_per_s": round(1e6 / (us * L), 1),
                                "tokens_per_s": round(m * 1e6 / (us * L), 1), "splits": sp}
                log(f"weights w{bits} M={m}: {res[f'M{m}']}")
                del g, x, y, ws
            out["int4" if bits == 4 else "fp8"] = res
            del packs, scs
            torch.cuda.empty_cache()
        out["int4_speedup"] = {mk: round(out["fp8"][mk]["us_per_gemm"] / out["int4"][mk]["us_per_gemm"], 3)
                               for mk in out["int4"]}
        out["note"] = ("tokens_per_s = M rows x passes over the stack per second (one token per request per "
                       "pass); weight_gbs counts codes + scales; graph replay of the whole stack")
        return out

    w = wl.WORKLOADS[args.workload]
    if args.batch:
        w = w.with_(name=f"{w.name}_b{args.batch}", batch=args.batch)
    results = {}
    if args.weights_only:
        print(json.dumps({"metric": "weight-quantised decode GEMM (INT4 vs FP8 weights), one GPU",
                          "weight_gemm": measure_weights()}), flush=True)
        return
    if args.layers_only:
        args.no_sweep = args.no_capacity = args.no_extra = args.no_cpu_baseline = True
        args.no_layers = False
    else:
        log(f"workload {w}")
        host, stale, kv_elems, flops = prepare(w, args.splits)
        for kvd in (["fp8"] if (args.no_bf16 or args.fp8_only_steps) else ["fp8", "bf16"]):
            results[kvd] = measure(w, kvd, host, stale, kv_elems, args.steps, args.warmup)
        del host
        torch.cuda.empty_cache()

    sweep = {}
    if not args.no_sweep and not args.fp8_only_steps:
        # B = 1 .. 64 at 8192 tokens, each step after a cache-evicting write: without it the smaller
        # points (16.8 MB of FP8 KV at B = 1) would be read from the 256 MB Infinity Cache
        for b in (1, 8, 16, 32, 64):
            wb = wl.WORKLOADS[f"sweep_b{b}"]
            hb, st_b, el_b, _ = prepare(wb, args.splits)
            e = {}
            for kvd in ("fp8", "bf16"):
                r = measure(wb, kvd, hb, st_b, el_b, args.steps, 3, flushed=True)
                e[kvd] = {"step_us": round(1e3 * r["step_ms"], 2), "step_us_p95": round(1e3 * r["step_ms_p95"], 2),
                          "steps_per_s": round(1e3 / r["step_ms"], 1), "attn_us": round(1e3 * r["attn_ms"], 2),
                          "attn_us_p95": round(1e3 * r["attn_ms_p95"], 2), "attn_gbs": round(r["gbs_attn"], 1),
                          "attn_pct_hbm_peak": round(100 * r["gbs_attn"] / HBM_PEAK_GBS, 2),
                          "splits": r["splits"]}
                if args.unfused or args.two_launch:
                    e[kvd]["check_append_us"] = round(1e3 * r["check_append_ms"], 2)
            e["fp8_speedup_step"] = round(e["bf16"]["step_us"] / e["fp8"]["step_us"], 3)
            e["stale_requests"] = len(st_b)
            sweep[f"B{b}"] = e
            del hb
            torch.cuda.empty_cache()

    capacity = {}
    if not args.no_capacity and not args.fp8_only_steps:
        # one byte budget, what the BF16 cache needs for capacity_ref_batch requests of 8192 tokens; each
        # cache admits requests through the page allocator until it runs out, then its step is timed at
        # that concurrency (flushed, like the sweep)
        wc0 = wl.WORKLOADS["sweep_b64"].with_(stale=False)
        need = -(-int(wc0.ctx_hi) // wc0.page_size)
        bf16_page = wc0.page_size * wc0.num_kv_heads * (wc0.head_dim + wc0.v_dim) * 2 + 3 * 4
        budget = args.capacity_ref_batch * need * bf16_page
        capacity = {"budget_bytes": budget,
                    "budget": f"BF16 K/V pages plus per-page tag, page-table and expected-tag words of "
                              f"{args.capacity_ref_batch} requests x {wc0.ctx_hi} tokens",
                    "admission": "requests of 8192 tokens admitted through kv_page_alloc until KVFP8_ERR_NOSPACE, "
                                 "free list churned into a seeded random order first"}
        for kvd in ("fp8", "bf16"):
            adm = capacity_admission(kv, wc0, kvd, budget)
            wc = wc0.with_(name=f"capacity_{kvd}", batch=adm["admitted"], num_pages=adm["num_pages"])
            hc, st_c, el_c, _ = prepare(wc, args.splits, table=(adm["page_table"], adm["tags"]))
            r = measure(wc, kvd, hc, st_c, el_c, args.steps, 3, flushed=True)
            capacity[kvd] = {"num_pages": adm["num_pages"], "token_capacity": adm["token_capacity"],
                             "admitted_requests": adm["admitted"], "pages_left": adm["pages_left"],
                             "step_us": round(1e3 * r["step_ms"], 2), "attn_us": round(1e3 * r["attn_ms"], 2),
                             "attn_gbs": round(r["gbs_attn"], 1),
                             "tokens_per_s": round(adm["admitted"] / (r["step_ms"] * 1e-3), 1),
                             "splits": r["splits"]}
            del hc
            torch.cuda.empty_cache()
        capacity["fp8_over_bf16"] = {
            "admitted": round(capacity["fp8"]["admitted_requests"] / capacity["bf16"]["admitted_requests"], 3),
            "tokens_per_s": round(capacity["fp8"]["tokens_per_s"] / capacity["bf16"]["tokens_per_s"], 3)}
        capacity["note"] = ("tokens_per_s = admitted requests / flushed step time: one new token per request "
                            "per step of one attention layer")

    layer_runs = {}
    if not args.no_layers and not args.fp8_only_steps:
        # the attention part of a whole decode step: args.layers layers sharing one page table and tag set
        # (kv_decode_step_*: one check, then each layer's write + attention), timed eagerly (one library
        # call per step) and as replays of a captured HIP graph, with the tracker on and off
        n_l = args.layers
        lb = [int(x) for x in args.layer_batches.split(",") if x]
        for wname, batches in (("sweep_b64", lb), ("latent", [b for b in lb if b in (1, 64)])):
            for b in batches:
                base = wl.WORKLOADS[wname]
                # no stale tags here: with the tracker on an aborted request would skip its work, which is
                # not the check's cost
                wb = base.with_(name=f"{wname}_layers_b{b}", batch=b,
                                num_pages=b * (-(-int(base.ctx_hi) // base.page_size)), stale=False)
                hb, st_b, el_b, _ = prepare(wb, 0)
                e = {}
                for kvd in ("fp8", "bf16"):
                    r = measure_layers(wb, kvd, hb, st_b, n_l, max(10, args.steps // 2), 3)
                    r["kv_gb_per_s"] = round(el_b * (1 if kvd == "fp8" else 2) * n_l / (r["graph_us"] * 1e-6) / 1e9, 1)
                    e[kvd] = r
                e["fp8_speedup_graph"] = round(e["bf16"]["graph_us"] / e["fp8"]["graph_us"], 3)
                e["stale_requests"] = len(st_b)
                layer_runs[f"{wname}_B{b}"] = e
                del hb
                torch.cuda.empty_cache()

    weight_runs = None
    if not args.no_weights and not args.fp8_only_steps and not args.layers_only:
        weight_runs = measure_weights()

    extra = {}
    if not args.no_extra and not args.fp8_only_steps:
        for name in ("gqa_batch", "long", "latent"):
            we = wl.WORKLOADS[name]
            he, st_e, el_e, fl_e = prepare(we, we.num_splits)
            ex = {"workload": f"{we.batch} requests, context {we.ctx_lo}-{we.ctx_hi}, {we.num_q_heads} query / "
                              f"{we.num_kv_heads} KV heads, score dim {we.head_dim}, value dim {we.v_dim}, "
                              f"page {we.page_size}" + (", K outliers x20" if we.outlier_frac else "")}
            for kvd in ("fp8", "bf16"):
                r = measure(we, kvd, he, st_e, el_e, max(10, args.steps // 2), 3, full=False)
                e = {"ms_per_step": round(r["ms_per_step"], 5), "step_gbs": round(r["gbs_step"], 1),
                     "attn_ms": round(r["attn_ms_mean"], 5), "attn_gbs": round(r["gbs_attn"], 1),
                     "attn_pct_hbm_peak": round(100 * r["gbs_attn"] / HBM_PEAK_GBS, 2), "splits": r["splits"]}
                if we.latent:
                    e["splits"] = f"library choice per cache type (at most {r['splits']})" if not we.num_splits else \
                        r["splits"]
                    tf = fl_e / (r["attn_ms_mean"] * 1e-3) / 1e12
                    e["attn_tflops"] = round(tf, 1)
                    # FP8 cache: QK (576 of every 1088 flops per cached element and head) runs on FP8
                    # MFMAs, PV on bf16 ones, so the peak is that mix's: both parts at their own rate
                    if kvd == "fp8":
                        qk = we.head_dim / (we.head_dim + we.v_dim)
                        peak = 1.0 / (qk / FP8_MFMA_PEAK_TFLOPS + (1.0 - qk) / BF16_MFMA_PEAK_TFLOPS)
                        peak_note = "QK on FP8 MFMAs (5.0 PFLOP/s), PV on bf16 MFMAs (2.5 PFLOP/s)"
                    else:
                        peak = BF16_MFMA_PEAK_TFLOPS
                        peak_note = "QK and PV on bf16 MFMAs (2.5 PFLOP/s)"
                    e["mfma_roofline"] = {"bound": "mfma", "achieved": round(tf, 1), "peak": round(peak, 1),
                                          "unit": "TFLOP/s", "frac": round(tf / peak, 4), "flops_per_launch": fl_e,
                                          "peak_is": peak_note}
                ex[kvd] = e
            extra[name] = ex
            del he
            torch.cuda.empty_cache()

    if args.layers_only:
        print(json.dumps({"metric": "decode steps/s over a layer stack (one GPU)", "n_gpus": 1, "steps": args.steps,
                          "layer_stack_step": layer_runs}), flush=True)
        return
    f8 = results["fp8"]
    if args.unfused or args.two_launch:
        step_desc = (("tag check + append(1 token/request)" if args.unfused else
                      "fused tag check + append(1 token/request)") + " + attention (+ merge when split)")
        kernel_desc = "paged_decode_attn_fp8 (split kernel, plus the merge kernel when splits > 1)"
        breakdown = (({"tag_check": round(f8["check_ms"], 5), "append": round(f8["append_ms"], 5)}
                      if args.unfused else {"tag_check_append": round(f8["check_ms"], 5)}) |
                     {"attention": round(f8["attn_ms"], 5), "step_p95": round(f8["step_ms_p95"], 5),
                      "note": "events around each launch of eager steps"})
    else:
        step_desc = ("one launch (kv_decode_step_fp8 over one layer): every block checks its request's page tags, "
                     "the block holding position L-1 writes the new token (1 token/request), attention "
                     "(+ merge when split)")
        kernel_desc = ("attn_gqa_split_kernel<fp8> with the tag check and the token write in the same launch "
                       "(plus the merge kernel when splits > 1)")
        breakdown = {"one_launch_step": round(f8["attn_ms"], 5), "step_p95": round(f8["step_ms_p95"], 5),
                     "note": "events around the step's launch, eager steps"}
    line = {
        "metric": METRIC,
        "value": round(f8["gbs_step"], 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(f8["ms_per_step"], 5),
        "steps_per_s": round(1e3 / f8["ms_per_step"], 1),
        "pct_hbm_peak": round(100 * f8["gbs_step"] / HBM_PEAK_GBS, 2),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "kv_cache": "fp8_e4m3",
        "data": "synthetic",
        "config": {"workload": f"{w.name}: {w.batch} requests x {w.ctx_hi} tokens, {w.num_q_heads} query / "
                               f"{w.num_kv_heads} KV heads, head_dim {w.head_dim}, page {w.page_size}, "
                               f"{w.num_pages}-page pool, FP8 e4m3 cache, 1% stale tags",
                   "batch": w.batch, "ctx": int(w.ctx_hi), "num_q_heads": w.num_q_heads,
                   "num_kv_heads": w.num_kv_heads, "head_dim": w.head_dim, "page_size": w.page_size,
                   "splits": f8["splits"],
                   "step": step_desc},
        "roofline": {"bound": "hbm", "achieved": round(f8["gbs_attn"], 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(f8["gbs_attn"] / HBM_PEAK_GBS, 4),
                     "traffic": measured_traffic(w.name, f8["splits"]),
                     "algorithmic_bytes": f8["kv_bytes"],
                     "kernel": kernel_desc,
                     "attn_ms_mean": round(f8["attn_ms_mean"], 5), "attn_ms_p95": round(f8["attn_ms_p95"], 5)},
        "step_breakdown_ms": breakdown,
        "timing": ("steps replayed from a captured HIP graph of one step" if args.graph else
                   "eager back-to-back steps") + ", between two events on the launch stream",
        ("eager_ms_per_step" if args.graph else "graph_ms_per_step"): round(f8["other"]["ms_per_step"], 5),
    }
    if "flushed" in f8:
        fl = f8["flushed"]
        line["flushed_step"] = {"step_us": round(1e3 * fl["step_ms"], 2), "step_us_p95": round(1e3 * fl["step_ms_p95"], 2),
                                "attn_us": round(1e3 * fl["attn_ms"], 2),
                                "note": f"median over steps each preceded by a {args.flush_mib} MiB write"}
    if sweep:
        line["batch_sweep_flushed"] = sweep
    if capacity:
        line["capacity_fixed_budget"] = capacity
    if weight_runs:
        line["weight_gemm"] = weight_runs
    if layer_runs:
        line["layer_stack_step"] = layer_runs | {
            "note": f"one decode step over {args.layers} layers sharing one page table and tag set "
                    "(kv_decode_step_*: GQA, one launch per layer that writes the layer's token, layer 0's also running "
                    "the tag check; latent, a check + write launch (the check in layer 0 only) and the attention); graph_us = replay of a captured HIP graph of the whole step, eager_us = one "
                    "library call per step; tokens_per_s = non-aborted requests x steps/s"}
    if "no_tracker" in f8:
        nt = f8["no_tracker"]
        line["tracker_off"] = {"ms_per_step": round(nt["ms_per_step"], 5),
                               "check_overhead_pct": round(100 * (f8["ms_per_step"] / nt["ms_per_step"] - 1), 2)}
    if "bf16" in results:
        b = results["bf16"]
        line["bf16_twin"] = {"value": round(b["gbs_step"], 1), "unit": "GB/s", "ms_per_step": round(b["ms_per_step"], 5),
                             "attn_gbs": round(b["gbs_attn"], 1), "attn_ms_mean": round(b["attn_ms_mean"], 5),
                             "fp8_speedup_step": round(b["ms_per_step"] / f8["ms_per_step"], 3)}
    if extra:
        line["other_workloads"] = extra
    if args.copy_calibration:
        n = args.copy_calibration << 20
        src = torch.ones(n // 4, dtype=torch.int32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        line["copy_calibration_bytes"] = n
    if not args.no_cpu_baseline:
        log(f"cpu baseline: oracle on {args.cpu_sample} requests")
        cb = cpu_baseline(w, args.cpu_sample)
        line["cpu_baseline"] = {k_: (round(v_, 4) if isinstance(v_, float) else v_) for k_, v_ in cb.items()
                                if k_ != "seconds"}
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
