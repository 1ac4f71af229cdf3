#!/usr/bin/env python3
"""Decode-step benchmark on one MI355X: FP8 (e4m3) vs BF16 paged KV cache.

A step is one pass of the whole hot path for one attention layer over one batch: the batched page-tag
check, the append of every request's new token (quantised to e4m3 for the FP8 cache) and paged decode
attention (split kernel + log-sum-exp merge when the context is split).  The headline step is the
library's kv_decode_step_* over that one layer in its default form, the pages' design: the tag check as
its own batched launch (fused with the token write: kv_tag_check_append_*), then the attention reading
the flags it left.  The one-launch form (the check inside the attention blocks) is reported next to it.

Inputs are resident in HBM before timing starts.  Timed loops rotate through several disjoint page sets
of one pool (at least 768 MB of KV in all, two at the least), so no step reads what the previous one left
in the 256 MB Infinity Cache.  Default workload: 64 requests x 8192 tokens, 64 query / 8 KV heads,
head_dim 128, page size 16, one stale expected tag (1 % of requests, that request aborted and its bytes
excluded).

Prints one JSON line.  Metric: KV-read GB/s of the whole step (algorithmic bytes: sum over non-aborted
requests of L * Hkv * (D + Dv) * bytes per element) and steps/s.  Further sections: the attention kernel
against the HBM roofline and against measured read-only kernels (attainable rate), the batch sweep with the
tag check's overhead (interleaved on/off repeats, 95 % confidence interval), admission under a fixed byte
budget, a step over a 61-layer stack (HIP graph), the INT4- vs FP8-weight decode GEMM, the other workloads
(ragged batch, long context, latent cache) and the CPU oracle.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import platform
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, 8.0 TB/s
BF16_MFMA_PEAK_TFLOPS = 2500.0 # MI355X dense bf16 matrix peak
FP8_MFMA_PEAK_TFLOPS = 5000.0  # MI355X dense fp8 matrix peak
METRIC = "decode-attn KV-read GB/s (% of HBM peak) + steps/s, FP8 vs BF16 KV cache"
ROTATE_BYTES = 768 << 20       # KV bytes the rotated page sets of a timing loop hold at least


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
                   help="requests of the main workload (0 = the workload's own)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-bf16", action="store_true")
    p.add_argument("--no-extra", action="store_true", help="skip the other workloads (GQA batch, long, latent)")
    p.add_argument("--no-sweep", action="store_true", help="skip the batch sweep B = 1, 8, 16, 32, 64")
    p.add_argument("--no-capacity", action="store_true",
                   help="skip the fixed-budget admission of 8192-token requests (FP8 vs BF16)")
    p.add_argument("--no-layers", action="store_true", help="skip the whole-step runs over a layer stack")
    p.add_argument("--layers", type=int, default=61, help="layers in the layer-stack step")
    p.add_argument("--layer-batches", default="1,8,64",
                   help="batch sizes of the layer-stack step (the latent cache runs those of them in {1, 64})")
    p.add_argument("--layers-only", action="store_true", help="run only the layer-stack step")
    p.add_argument("--no-weights", action="store_true", help="skip the weight-quantised decode GEMM runs")
    p.add_argument("--weights-only", action="store_true", help="run only the weight-quantised GEMM section")
    p.add_argument("--capacity-ref-batch", type=int, default=32,
                   help="the byte budget is what this many 8192-token requests take in the BF16 cache")
    p.add_argument("--cpu-sample", type=int, default=16, help="requests in the CPU oracle sample")
    p.add_argument("--ci-repeats", type=int, default=12,
                   help="interleaved tracker on/off pairs behind each overhead confidence interval")
    p.add_argument("--fp8-only-steps", action="store_true",
                   help="time only the FP8 headline (profiling runs: the step, then attention and check alone)")
    p.add_argument("--mode", choices=("separate", "fused"), default="separate",
                   help="step form of the headline (separate: the library's default)")
    p.add_argument("--warm-seconds", type=float, default=1.0,
                   help="back-to-back steps before the headline is timed, so that clocks leave their idle states")
    p.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                   help="after timing, copy a MIB-MiB buffer 3 times (a known-size kernel for HBM counters)")
    return p.parse_args()


def copies_for(touched_bytes):
    return max(2, -(-ROTATE_BYTES // max(1, touched_bytes)))


def t95(df):
    """Two-sided 95 % quantile of Student's t with df degrees of freedom."""
    from scipy import stats
    return float(stats.t.ppf(0.975, df))


class Workset:
    """One workload's inputs on the device, with `copies` page tables over disjoint page sets of one pool
    (or, given table = (page table, tags) from the page allocator, that one table)."""

    def __init__(self, w, splits, copies, dev, table=None):
        from kvsynth import workloads as wl
        t = time.perf_counter()
        self.w, self.splits = w, splits
        lens = wl.ctx_lens(w)
        if table is None:
            pts, P = wl.rotation_tables(w, lens, copies)
            tags = wl.page_tags(w.with_(num_pages=P))
        else:
            pts, tags = table[0][None], table[1]
            P, copies = w.num_pages, 1
        self.copies, self.num_pages = copies, P
        stale = wl.stale_requests(w)
        exps = np.stack([wl.expected_tags(w, pts[c], lens, tags, stale) for c in range(copies)])
        k, v = wl.all_kv(w, lens)
        req, pos = wl.token_index(lens)
        last = np.cumsum(lens.astype(np.int64)) - 1
        self.lens, self.stale = lens, stale
        self.dpt = dev(pts)                # [copies][B][stride]
        self.dexp = dev(exps)
        self.dtags, self.dlens, self.dq = dev(tags), dev(lens), dev(wl.queries(w))
        self.dk, self.dv = dev(k), (None if v is None else dev(v))
        self.dreq, self.dpos = dev(req), dev(pos)
        self.dk_new, self.dv_new = dev(k[last]), (None if v is None else dev(v[last]))
        self.dk_calib = self.dk
        if w.outlier_frac > 0:             # the K scale comes from the outlier-free draw
            kc, _ = wl.all_kv(w, lens, outliers=False)
            self.dk_calib = dev(kc)
            del kc
        del k, v
        self.max_ctx = int(lens.max())
        live = np.ones(w.batch, dtype=bool)
        live[stale] = False
        row = w.head_dim if w.latent else w.num_kv_heads * (w.head_dim + w.v_dim)
        self.kv_elems = int(lens[live].astype(np.int64).sum()) * row
        self.flops = int(lens[live].astype(np.int64).sum()) * w.num_q_heads * (w.head_dim + w.v_dim) * 2
        need = wl.pages_needed(lens, w.page_size)
        # the (page, kv head) blocks one step reads, per page set, for the read-rate calibration
        self.block_ids = []
        for c in range(copies):
            ids = [pts[c, r, :need[r]] for r in range(w.batch) if live[r]]
            ids = np.concatenate(ids).astype(np.int64) if ids else np.zeros(0, np.int64)
            H = w.num_kv_heads
            self.block_ids.append(dev((ids[:, None] * H + np.arange(H)[None, :]).ravel().astype(np.int32)))
        log(f"{w.name}: inputs ready in {time.perf_counter() - t:.1f} s ({copies} page sets, {P} pages)")


class Cache:
    """One cache type (FP8 or BF16) over a Workset, every page set filled through the library's append.
    pool_clones > 1 keeps that many copies of the whole pool (one page table) instead."""

    def __init__(self, ws, kvd, torch, kv, pool_clones=1):
        self.ws, self.kvd, self.torch, self.kv = ws, kvd, torch, kv
        w = ws.w
        self.fp8 = kvd == "fp8"
        tdt = torch.uint8 if self.fp8 else torch.int16
        P = ws.num_pages
        nk = P * w.num_kv_heads * w.page_size * w.head_dim
        nv = P * w.num_kv_heads * w.page_size * w.v_dim
        # K and V pools in one allocation (V right after K), so that one read-rate launch covers both
        kvmem = torch.zeros(nk + (0 if w.latent else nv), dtype=tdt, device="cuda")
        kp = kvmem[:nk]
        vp = None if w.latent else kvmem[nk:]
        self.kvmem = kvmem
        self.desc = kv.pool_desc(P, w.page_size, w.num_kv_heads, w.head_dim, w.v_dim)
        dv = None if w.latent else ws.dv
        if self.fp8:
            self.k_scale = kv.calibrate_scale(ws.dk_calib)
            self.v_scale = self.k_scale if w.latent else kv.calibrate_scale(dv)
        else:
            self.k_scale = self.v_scale = 1.0
        for c in range(ws.copies):
            if self.fp8:
                kv.kv_append_fp8(self.desc, kp, vp, ws.dk, dv, ws.dreq, ws.dpos, ws.dpt[c], k_scale=self.k_scale,
                                 v_scale=self.v_scale)
            else:
                kv.kv_append_bf16(self.desc, kp, vp, ws.dk, dv, ws.dreq, ws.dpos, ws.dpt[c])
        self.kps, self.vps = [kp], [vp]
        for _ in range(pool_clones - 1):
            mem = kvmem.clone()
            self.kps.append(mem[:nk])
            self.vps.append(None if vp is None else mem[nk:])
        self.n = max(ws.copies, pool_clones)
        self.flags = torch.zeros((self.n, w.batch), dtype=torch.int32, device="cuda")
        self.out = torch.empty((w.batch, w.num_q_heads, w.v_dim), dtype=torch.int16, device="cuda")
        if ws.splits:
            self.splits = ws.splits
        elif w.latent:
            self.splits = kv.paged_decode_attn_latent_auto_splits(w.batch, w.num_q_heads, ws.max_ctx)
        else:
            self.splits = kv.paged_decode_attn_auto_splits(w.batch, w.num_kv_heads, ws.max_ctx)
        # latent: with no requested count the library picks per cache type; the workspace is sized with
        # the public bound, which covers both
        self.req_splits = ws.splits
        nb = kv.paged_decode_attn_workspace_bytes(w.batch, w.num_q_heads, w.v_dim, self.splits)
        self.wsp = torch.zeros(max(nb // 4, 4), dtype=torch.float32, device="cuda")  # zeroed once
        torch.cuda.synchronize()

    def _c(self, i):
        i %= self.n
        return (self.kps[i % len(self.kps)], self.vps[i % len(self.vps)], self.ws.dpt[i % self.ws.copies],
                self.ws.dexp[i % self.ws.copies], self.flags[i])

    def check_append(self, i):
        kp, vp, pt, exp, fl = self._c(i)
        ws = self.ws
        if self.fp8:
            self.kv.kv_tag_check_append_fp8(self.desc, kp, vp, ws.dk_new, ws.dv_new, pt, ws.dlens, ws.dtags, exp, fl,
                                            k_scale=self.k_scale, v_scale=self.v_scale)
        else:
            self.kv.kv_tag_check_append_bf16(self.desc, kp, vp, ws.dk_new, ws.dv_new, pt, ws.dlens, ws.dtags, exp,
                                             fl)

    def attend(self, i, tracker=True):
        kp, vp, pt, _, fl = self._c(i)
        f = fl if tracker else None
        kv, ws, w = self.kv, self.ws, self.ws.w
        if w.latent and self.fp8:
            kv.paged_decode_attn_latent_fp8(self.desc, ws.dq, kp, pt, ws.dlens, ws.max_ctx, self.out, f,
                                            scale=self.k_scale, num_splits=self.req_splits, workspace=self.wsp)
        elif w.latent:
            kv.paged_decode_attn_latent_bf16(self.desc, ws.dq, kp, pt, ws.dlens, ws.max_ctx, self.out, f,
                                             num_splits=self.req_splits, workspace=self.wsp)
        elif self.fp8:
            kv.paged_decode_attn_fp8(self.desc, ws.dq, kp, vp, pt, ws.dlens, ws.max_ctx, self.out, f,
                                     k_scale=self.k_scale, v_scale=self.v_scale, num_splits=self.req_splits,
                                     workspace=self.wsp)
        else:
            kv.paged_decode_attn_bf16(self.desc, ws.dq, kp, vp, pt, ws.dlens, ws.max_ctx, self.out, f,
                                      num_splits=self.req_splits, workspace=self.wsp)

    def step(self, i, mode="separate"):
        """kv_decode_step_* over this one layer.  separate: the check + write launch, then the attention
        (the library's default); fused: the check inside the attention launch; off: no tracker (one
        attention launch whose block holding position L - 1 writes the token)."""
        kp, vp, pt, exp, fl = self._c(i)
        ws = self.ws
        on = mode != "off"
        self.kv.decode_step(self.desc, self.kvd, kp, vp, pt, ws.dlens, ws.max_ctx, ws.dq, ws.dk_new, ws.dv_new,
                            None, None, self.out, page_tags=ws.dtags if on else None,
                            expected_tags=exp if on else None, abort_flags=fl if on else None,
                            k_scale=self.k_scale, v_scale=self.v_scale, num_splits=self.req_splits,
                            workspace=self.wsp, fused_check=mode == "fused")

    def flags_ok(self):
        fl = self.flags.cpu().numpy().view(np.uint32)
        for c in range(self.n):
            assert np.flatnonzero(fl[c]).tolist() == self.ws.stale.tolist(), "flags differ from the planted set"


class Timer:
    def __init__(self, torch, steps, warmup):
        self.torch, self.steps, self.warmup = torch, steps, warmup

    def back_to_back(self, fn, steps=None):
        """ms per call of `steps` back-to-back calls fn(0), fn(1), ... between two events on the launch stream."""
        torch = self.torch
        steps = steps or self.steps
        for i in range(self.warmup):
            fn(i)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(steps):
            fn(i)
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps

    def warm(self, fn, seconds=1.0):
        """Run fn back to back for about `seconds`, so that clocks have left their idle states."""
        t0 = time.perf_counter()
        i = 0
        while time.perf_counter() - t0 < seconds:
            for _ in range(50):
                fn(i)
                i += 1
            self.torch.cuda.synchronize()

    def per_call(self, fn):
        """ms of each of `steps` calls (an event before and after every call)."""
        torch = self.torch
        for i in range(self.warmup):
            fn(i)
        torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(self.steps)]
        for i, (a, b) in enumerate(ev):
            a.record()
            fn(i)
            b.record()
        torch.cuda.synchronize()
        return np.array([a.elapsed_time(b) for a, b in ev])

    def overhead(self, on, off, repeats, n=None):
        """Tracker overhead: `repeats` interleaved pairs of back-to-back blocks (n calls with the check,
        n without, the order alternating between pairs); per pair the ratio of block times.  Returns the
        mean overhead in percent, its 95 % confidence interval (Student's t over the pairs) and the calls."""
        n = n or max(10, self.steps // 2)
        r = []
        for k in range(repeats):
            if k % 2 == 0:
                a = self.back_to_back(on, n)
                b = self.back_to_back(off, n)
            else:
                b = self.back_to_back(off, n)
                a = self.back_to_back(on, n)
            r.append(100.0 * (a / b - 1.0))
        r = np.array(r)
        half = t95(len(r) - 1) * r.std(ddof=1) / math.sqrt(len(r))
        return {"overhead_pct": round(float(r.mean()), 3), "ci95_pct": [round(float(r.mean() - half), 3),
                                                                         round(float(r.mean() + half), 3)],
                "pairs": int(repeats), "calls_per_block": int(n), "calls_in_all": int(2 * repeats * n)}

    def graph(self, fn, copies):
        """ms per call of replays of one captured HIP graph holding `copies` calls fn(0..copies-1)."""
        torch = self.torch
        for i in range(copies):
            fn(i)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for i in range(copies):
                fn(i)
        torch.cuda.current_stream().wait_stream(side)
        with torch.cuda.graph(g):
            for i in range(copies):
                fn(i)
        reps = max(2, self.steps // copies)
        ms = self.back_to_back(lambda i: g.replay(), reps)
        del g
        return ms / copies


def attainable(torch, kv, ws, cache, timer):
    """Read-only kernels over the same bytes as the attention: a sequential stream of the step's KV byte
    count, and the (page, kv head) blocks of K and V one step reads, in the order of the page table (both
    rotated through the page sets).  GB/s of each."""
    w = ws.w
    nbytes = ws.kv_elems * (1 if cache.fp8 else 2)
    sink = torch.zeros(kv.READ_SINK_WORDS, dtype=torch.int32, device="cuda")
    bufs = [torch.empty(nbytes // 4 + 4, dtype=torch.int32, device="cuda").fill_(i + 1) for i in range(2)]
    t_stream = min(timer.back_to_back(lambda i: kv.kv_read_stream(bufs[i % 2], sink, nbytes=nbytes))
                   for _ in range(3))
    del bufs
    blk = w.page_size * w.head_dim * (1 if cache.fp8 else 2)
    # the K blocks' ids, then the V blocks' (the V pool follows the K pool in memory): one launch
    v_off = cache.kps[0].numel() * cache.kps[0].element_size() // blk
    ids_kv = [torch.cat([ids, ids + v_off]) if cache.vps[0] is not None else ids for ids in ws.block_ids]

    def blocks(i):
        kv.kv_read_blocks(cache.kvmem, blk, ids_kv[i % ws.copies], sink)

    t_blocks = min(timer.back_to_back(blocks) for _ in range(3))
    stream_gbs = nbytes / (t_stream * 1e-3) / 1e9
    blocks_gbs = nbytes / (t_blocks * 1e-3) / 1e9
    return {"stream_gbs": round(stream_gbs, 1), "page_blocks_gbs": round(blocks_gbs, 1),
            "attainable_gbs": round(max(stream_gbs, blocks_gbs), 1),
            "bytes": nbytes, "block_bytes": blk,
            "note": "kv_read_stream over the step's KV byte count (contiguous), and kv_read_blocks over the "
                    "same (page, kv head) blocks of K and V the attention reads, in one launch; the best of "
                    "three back-to-back runs of each; attainable_gbs = the faster of the two, the read rate "
                    "pct_attainable is taken against"}


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


def stored_traffic(workload, mode):
    """HBM bytes per launch of the FP8 attention kernel as two committed counter runs measured them
    (rocprofv3 --pmc FETCH_SIZE, then WRITE_SIZE), or None when the kernel's sources changed since or the
    figure is of another step form."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "attn_fp8_64x8192_traffic.json")
    if not os.path.exists(path):
        return None
    d = json.load(open(path))
    h = hashlib.sha256()
    for src in d["kernel_sources"]:
        h.update(open(os.path.join(ROOT, src), "rb").read())
    if h.hexdigest() != d["kernel_sources_sha256"] or d["workload"] != workload or d.get("mode") != mode:
        return None
    return d


def copy_calibration(torch, mib):
    """Three device copies of mib MiB: a kernel of known traffic that scales the HBM counters."""
    if not mib:
        return 0
    n = mib << 20
    src = torch.ones(n // 4, dtype=torch.int32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    return n


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or "unknown"


def cpu_baseline(w, n_req, min_seconds=10.0):
    """The oracle's step (tag check, e4m3 append of one token per request, fp64 attention) on a sample of
    the workload's requests, over a thread pool with BLAS threads 1 per worker."""
    from threadpoolctl import threadpool_limits

    from kvsynth import workloads as wl
    from oracle import codec, paged, step

    n_req = min(n_req, w.batch)
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
    # a GPU machine gives one GPU a share of at most 16 CPU threads, whatever os.cpu_count() shows there
    host_cpus = os.cpu_count() or 1
    try:
        usable = len(os.sched_getaffinity(0))
    except AttributeError:
        usable = host_cpus
    workers = max(1, min(16, usable))
    times = []
    with threadpool_limits(1):
        while len(times) < 3 or sum(times) < min_seconds:
            t = time.perf_counter()
            step.decode_step(st, wl.queries(ws), k[last], v[last], np.arange(n_req, dtype=np.int32),
                             (lens - 1).astype(np.int32), workers=workers)
            times.append(time.perf_counter() - t)
    dt = float(np.median(times))
    kv_bytes = int(lens.astype(np.int64).sum()) * ws.num_kv_heads * (ws.head_dim + ws.v_dim)
    return {"value": round(kv_bytes / dt / 1e9, 4), "unit": "GB/s", "cores": workers, "kind": "oracle",
            "sample": f"{n_req} of {w.batch} requests of {w.name} (same shapes, FP8 cache), one decode step "
                      f"(tag check + e4m3 append + fp64 attention), median of {len(times)} runs "
                      f"({sum(times):.1f} s in all): {dt:.2f} s per step",
            "host_logical_cpus": host_cpus, "usable_cpus": usable, "cpu_model": cpu_model(),
            "threads": f"ThreadPoolExecutor({workers}) over requests, BLAS threads 1 per worker"}


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

    timer = Timer(torch, args.steps, args.warmup)

    def touched(w):
        lens = wl.ctx_lens(w)
        row = w.head_dim if w.latent else w.num_kv_heads * (w.head_dim + w.v_dim)
        return int(lens.astype(np.int64).sum()) * row  # FP8 bytes; BF16 twice as many

    def headline(w, kvd, ws, full=True):
        c = Cache(ws, kvd, torch, kv)
        elt = 1 if kvd == "fp8" else 2
        r = {"kv_bytes": ws.kv_elems * elt, "splits": c.splits, "page_sets": c.n}
        timer.warm(lambda i: c.step(i, args.mode), args.warm_seconds)
        r["step_ms"] = timer.back_to_back(lambda i: c.step(i, args.mode))
        # the attention launch alone (reading the flags the steps left): the best of three back-to-back
        # blocks, a kernel time inside the step's
        r["attn_ms"] = min(timer.back_to_back(lambda i: c.attend(i)) for _ in range(3))
        r["check_append_ms"] = min(timer.back_to_back(c.check_append) for _ in range(3))
        per = timer.per_call(lambda i: c.step(i, args.mode))
        r["step_ms_median_events"] = float(np.median(per))
        r["step_ms_p95_events"] = float(np.percentile(per, 95))
        c.flags_ok()
        if full:
            other = "fused" if args.mode == "separate" else "separate"
            r["other_ms"] = timer.back_to_back(lambda i: c.step(i, other))
            r["no_tracker_ms"] = timer.back_to_back(lambda i: c.step(i, "off"))
            r["overhead"] = timer.overhead(lambda i: c.step(i, args.mode), lambda i: c.step(i, "off"),
                                           args.ci_repeats)
            r["graph_ms"] = timer.graph(lambda i: c.step(i, args.mode), c.n)
            if kvd == "fp8":
                r["attainable"] = attainable(torch, kv, ws, c, timer)
        c.flags_ok()
        log(f"{w.name} {kvd}: " + json.dumps({k_: (round(v_, 5) if isinstance(v_, float) else v_)
                                              for k_, v_ in r.items()}))
        del c
        torch.cuda.empty_cache()
        return r

    def sweep_point(w, kvd, ws):
        c = Cache(ws, kvd, torch, kv)
        elt = 1 if kvd == "fp8" else 2
        kv_bytes = ws.kv_elems * elt
        per = timer.per_call(lambda i: c.step(i))
        step_b2b = timer.back_to_back(lambda i: c.step(i))
        attn = timer.back_to_back(lambda i: c.attend(i))
        fused = timer.back_to_back(lambda i: c.step(i, "fused"))
        ov = timer.overhead(lambda i: c.step(i), lambda i: c.step(i, "off"), args.ci_repeats)
        c.flags_ok()
        e = {"step_us": round(1e3 * step_b2b, 2), "step_us_median_events": round(1e3 * float(np.median(per)), 2),
             "step_us_p95_events": round(1e3 * float(np.percentile(per, 95)), 2),
             "steps_per_s": round(1e3 / step_b2b, 1), "step_gbs": round(kv_bytes / (step_b2b * 1e-3) / 1e9, 1),
             "attn_us": round(1e3 * attn, 2), "attn_gbs": round(kv_bytes / (attn * 1e-3) / 1e9, 1),
             "attn_pct_hbm_peak": round(100 * kv_bytes / (attn * 1e-3) / 1e9 / HBM_PEAK_GBS, 2),
             "fused_one_launch_step_us": round(1e3 * fused, 2), "tracker": ov, "splits": c.splits,
             "page_sets": c.n}
        log(f"{w.name} {kvd}: {json.dumps(e)}")
        del c
        torch.cuda.empty_cache()
        return e

    def measure_layers(w, kvd, n_layers, steps, warmup):
        """One decode step over n_layers layers (each layer's pool a copy of layer 0's, so every layer's
        bytes are distinct), as one kv_decode_step_* call replayed from captured HIP graphs: tracker on
        (separate check launch, and fused), tracker off, and the overhead with its confidence interval."""
        ws = Workset(w, 0, 1, dev)
        c = Cache(ws, kvd, torch, kv)
        kp0, vp0 = c.kps[0], c.vps[0]
        kps = torch.empty((n_layers, kp0.numel()), dtype=kp0.dtype, device="cuda")
        kps.copy_(kp0.unsqueeze(0).expand(n_layers, -1))
        vps = None
        if vp0 is not None:
            vps = torch.empty((n_layers, vp0.numel()), dtype=vp0.dtype, device="cuda")
            vps.copy_(vp0.unsqueeze(0).expand(n_layers, -1))
        c.kps = c.vps = None
        del kp0, vp0
        q = ws.dq.unsqueeze(0).expand(n_layers, *ws.dq.shape).contiguous()
        k_new = ws.dk_new.unsqueeze(0).expand(n_layers, *ws.dk_new.shape).contiguous()
        v_new = None if ws.dv_new is None else ws.dv_new.unsqueeze(0).expand(n_layers, *ws.dv_new.shape).contiguous()
        out = torch.empty((n_layers,) + tuple(c.out.shape), dtype=torch.int16, device="cuda")
        fp8 = kvd == "fp8"
        ks = [c.k_scale] * n_layers if fp8 else None
        vs = [c.v_scale] * n_layers if fp8 and not w.latent else None
        flags = c.flags[0]

        def one(mode):
            on = mode != "off"
            kv.decode_step_layers(c.desc, kvd, kps, vps, ws.dpt[0], ws.dlens, ws.max_ctx, q, k_new, v_new, out,
                                  page_tags=ws.dtags if on else None, expected_tags=ws.dexp[0] if on else None,
                                  abort_flags=flags if on else None, k_scales=ks, v_scales=vs, workspace=c.wsp,
                                  fused_check=mode == "fused")

        lt = Timer(torch, steps, warmup)
        graphs = {}
        for mode in ("separate", "fused", "off"):
            g = torch.cuda.CUDAGraph()
            side = torch.cuda.Stream()
            side.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(side):
                one(mode)
            torch.cuda.current_stream().wait_stream(side)
            with torch.cuda.graph(g):
                one(mode)
            graphs[mode] = g
        res = {"eager_us": 1e3 * lt.back_to_back(lambda i: one("separate"))}
        for mode, key in (("separate", "graph_us"), ("fused", "graph_fused_us"), ("off", "graph_no_tracker_us")):
            res[key] = 1e3 * lt.back_to_back(lambda i, g=graphs[mode]: g.replay())
        ov = lt.overhead(lambda i: graphs["separate"].replay(), lambda i: graphs["off"].replay(), args.ci_repeats,
                         n=max(3, steps // 4))
        del graphs
        fl = flags.cpu().numpy().view(np.uint32)
        assert np.flatnonzero(fl).tolist() == ws.stale.tolist(), "flags differ from the planted stale set"
        r = {k_: round(v_, 2) for k_, v_ in res.items()}
        r["layers"] = n_layers
        r["per_layer_us"] = round(res["graph_us"] / n_layers, 2)
        r["steps_per_s"] = round(1e6 / res["graph_us"], 1)
        r["tokens_per_s"] = round((w.batch - len(ws.stale)) * 1e6 / res["graph_us"], 1)
        r["tracker"] = ov
        r["splits"] = c.splits
        r["kv_gb_per_s"] = round(ws.kv_elems * (1 if fp8 else 2) * n_layers / (res["graph_us"] * 1e-6) / 1e9, 1)
        log(f"{w.name} {kvd} x{n_layers} layers: " + json.dumps(r))
        del c, kps, vps, q, k_new, v_new, out, ws
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
                wsb = torch.zeros(max(kv.wgemm_workspace_bytes(m, N, K, sp), 16) // 4 + 4, dtype=torch.float32,
                                  device="cuda")

                def stack(i):
                    for li in range(L):
                        f(x, packs[li], scs[li], N, K, y, workspace=wsb)

                wt = Timer(torch, reps, 3)
                us = 1e3 * wt.graph(stack, 1) / L
                gbs = out["bytes_per_matrix"]["int4" if bits == 4 else "fp8"] / (us * 1e-6) / 1e9
                res[f"M{m}"] = {"us_per_gemm": round(us, 2), "weight_gbs": round(gbs, 1),
                                "pct_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 2),
                                "stack_passes_per_s": round(1e6 / (us * L), 1),
                                "tokens_per_s": round(m * 1e6 / (us * L), 1), "splits": sp}
                log(f"weights w{bits} M={m}: {res[f'M{m}']}")
                del x, y, wsb
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
    if args.weights_only:
        print(json.dumps({"metric": "weight-quantised decode GEMM (INT4 vs FP8 weights), one GPU",
                          "weight_gemm": measure_weights()}), flush=True)
        return
    if args.layers_only:
        args.no_sweep = args.no_capacity = args.no_extra = args.no_cpu_baseline = args.no_weights = True

    results = {}
    if not args.layers_only:
        log(f"workload {w}")
        ws = Workset(w, args.splits, copies_for(touched(w)), dev)
        for kvd in (["fp8"] if (args.no_bf16 or args.fp8_only_steps) else ["fp8", "bf16"]):
            results[kvd] = headline(w, kvd, ws, full=not args.fp8_only_steps)
        del ws
        torch.cuda.empty_cache()
        if args.fp8_only_steps:
            f8 = results["fp8"]
            copy_calibration(torch, args.copy_calibration)
            print(json.dumps({"metric": METRIC, "mode": args.mode, "steps": args.steps,
                              "ms_per_step": round(f8["step_ms"], 5), "attn_ms": round(f8["attn_ms"], 5),
                              "check_append_ms": round(f8["check_append_ms"], 5),
                              "value": round(f8["kv_bytes"] / (f8["step_ms"] * 1e-3) / 1e9, 1)}), flush=True)
            return

    sweep = {}
    if not args.no_sweep:
        for b in (1, 8, 16, 32, 64):
            wb = wl.WORKLOADS[f"sweep_b{b}"]
            wsb = Workset(wb, args.splits, copies_for(touched(wb)), dev)
            e = {kvd: sweep_point(wb, kvd, wsb) for kvd in ("fp8", "bf16")}
            e["fp8_speedup_step"] = round(e["bf16"]["step_us"] / e["fp8"]["step_us"], 3)
            e["stale_requests"] = len(wsb.stale)
            sweep[f"B{b}"] = e
            del wsb
            torch.cuda.empty_cache()

    capacity = {}
    if not args.no_capacity:
        # one byte budget, what the BF16 cache needs for capacity_ref_batch requests of 8192 tokens; each
        # cache admits requests through the page allocator until it runs out, then its step is timed at
        # that concurrency, rotating between two copies of the admitted pool
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
            wsc = Workset(wc, args.splits, 1, dev, table=(adm["page_table"], adm["tags"]))
            c = Cache(wsc, kvd, torch, kv, pool_clones=2)
            step = timer.back_to_back(lambda i: c.step(i))
            c.flags_ok()
            capacity[kvd] = {"num_pages": adm["num_pages"], "token_capacity": adm["token_capacity"],
                             "admitted_requests": adm["admitted"], "pages_left": adm["pages_left"],
                             "step_us": round(1e3 * step, 2),
                             "tokens_per_s": round(adm["admitted"] / (step * 1e-3), 1), "splits": c.splits}
            del c, wsc
            torch.cuda.empty_cache()
        capacity["fp8_over_bf16"] = {
            "admitted": round(capacity["fp8"]["admitted_requests"] / capacity["bf16"]["admitted_requests"], 3),
            "tokens_per_s": round(capacity["fp8"]["tokens_per_s"] / capacity["bf16"]["tokens_per_s"], 3)}
        capacity["note"] = ("tokens_per_s = admitted requests / step time (one new token per request per step of "
                            "one attention layer), steps rotating between two copies of the admitted pool")

    layer_runs = {}
    if not args.no_layers:
        n_l = args.layers
        lb = [int(x) for x in args.layer_batches.split(",") if x]
        for wname, batches in (("sweep_b64", lb), ("latent", [b for b in lb if b in (1, 64)])):
            for b in batches:
                base = wl.WORKLOADS[wname]
                # no stale tags here: with the tracker on an aborted request would skip its work, which is
                # not the check's cost
                wb = base.with_(name=f"{wname}_layers_b{b}", batch=b,
                                num_pages=b * (-(-int(base.ctx_hi) // base.page_size)), stale=False)
                e = {kvd: measure_layers(wb, kvd, n_l, max(10, args.steps // 2), 3) for kvd in ("fp8", "bf16")}
                e["fp8_speedup_graph"] = round(e["bf16"]["graph_us"] / e["fp8"]["graph_us"], 3)
                layer_runs[f"{wname}_B{b}"] = e

    weight_runs = None
    if not args.no_weights:
        weight_runs = measure_weights()

    extra = {}
    if not args.no_extra:
        for name in ("gqa_batch", "long", "latent"):
            we = wl.WORKLOADS[name]
            wse = Workset(we, we.num_splits, copies_for(touched(we)), dev)
            ex = {"workload": f"{we.batch} requests, context {we.ctx_lo}-{we.ctx_hi}, {we.num_q_heads} query / "
                              f"{we.num_kv_heads} KV heads, score dim {we.head_dim}, value dim {we.v_dim}, "
                              f"page {we.page_size}" + (", K outliers x20" if we.outlier_frac else ""),
                  "page_sets": wse.copies}
            for kvd in ("fp8", "bf16"):
                c = Cache(wse, kvd, torch, kv)
                elt = 1 if kvd == "fp8" else 2
                kvb = wse.kv_elems * elt
                step = timer.back_to_back(lambda i: c.step(i))
                attn = timer.back_to_back(lambda i: c.attend(i))
                fused = timer.back_to_back(lambda i: c.step(i, "fused"))
                c.flags_ok()
                e = {"ms_per_step": round(step, 5), "step_gbs": round(kvb / (step * 1e-3) / 1e9, 1),
                     "attn_ms": round(attn, 5), "attn_gbs": round(kvb / (attn * 1e-3) / 1e9, 1),
                     "attn_pct_hbm_peak": round(100 * kvb / (attn * 1e-3) / 1e9 / HBM_PEAK_GBS, 2),
                     "fused_one_launch_ms": round(fused, 5), "splits": c.splits}
                if we.latent:
                    e["splits"] = f"library choice per cache type (at most {c.splits})" if not we.num_splits else \
                        c.splits
                    tf = wse.flops / (attn * 1e-3) / 1e12
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
                                          "unit": "TFLOP/s", "frac": round(tf / peak, 4),
                                          "frac_of_bf16_peak": round(tf / BF16_MFMA_PEAK_TFLOPS, 4),
                                          "flops_per_launch": wse.flops, "peak_is": peak_note}
                log(f"{name} {kvd}: {json.dumps(e)}")
                ex[kvd] = e
                del c
                torch.cuda.empty_cache()
            extra[name] = ex
            del wse
            torch.cuda.empty_cache()

    if args.layers_only:
        print(json.dumps({"metric": "decode steps/s over a layer stack (one GPU)", "n_gpus": 1, "steps": args.steps,
                          "layer_stack_step": layer_runs}), flush=True)
        return

    f8 = results["fp8"]
    kvb = f8["kv_bytes"]
    gbs = kvb / (f8["step_ms"] * 1e-3) / 1e9
    attn_gbs = kvb / (f8["attn_ms"] * 1e-3) / 1e9
    att = f8["attainable"]
    traffic = stored_traffic(w.name, args.mode)
    line = {
        "metric": METRIC,
        "value": round(gbs, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(f8["step_ms"], 5),
        "steps_per_s": round(1e3 / f8["step_ms"], 1),
        "pct_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 2),
        "pct_attainable": round(100 * gbs / att["attainable_gbs"], 2),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "kv_cache": "fp8_e4m3",
        "data": "synthetic",
        "config": {"workload": f"{w.name}: {w.batch} requests x {w.ctx_hi} tokens, {w.num_q_heads} query / "
                               f"{w.num_kv_heads} KV heads, head_dim {w.head_dim}, page {w.page_size}, "
                               f"FP8 e4m3 cache, 1% stale tags; steps rotate through {f8['page_sets']} "
                               f"disjoint page sets of one pool",
                   "batch": w.batch, "ctx": int(w.ctx_hi), "num_q_heads": w.num_q_heads,
                   "num_kv_heads": w.num_kv_heads, "head_dim": w.head_dim, "page_size": w.page_size,
                   "splits": f8["splits"],
                   "step": ("kv_decode_step_fp8 over one layer: the tag check as its own batched launch, fused with "
                            "the write of 1 token/request (kv_tag_check_append_fp8), then the attention (+ merge "
                            "when split) reading its flags") if args.mode == "separate" else
                           "kv_decode_step_fp8 over one layer with KVFP8_STEP_FUSED_CHECK (one launch)"},
        "roofline": {"bound": "hbm", "achieved": round(attn_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(attn_gbs / HBM_PEAK_GBS, 4),
                     "traffic": None if traffic is None else traffic["traffic_bytes"],
                     "traffic_source": (None if traffic is None else
                                        "stored counter figure (two rocprofv3 --pmc runs of this launch shape on "
                                        "the current kernel sources): " + traffic["summary"]),
                     "algorithmic_bytes": kvb,
                     "kernel": "attn_gqa_split_kernel<fp8> (paged_decode_attn_fp8 reading the check's flags)",
                     "attn_ms": round(f8["attn_ms"], 5),
                     "timing": "back-to-back attention launches between two events on the launch stream, rotating "
                               "page sets, the best of three blocks (a kernel time within the step's)",
                     "pct_attainable": round(100 * attn_gbs / att["attainable_gbs"], 2)},
        "attainable_read": att,
        "step_breakdown_ms": {"check_append": round(f8["check_append_ms"], 5), "attention": round(f8["attn_ms"], 5),
                              "step": round(f8["step_ms"], 5),
                              "step_median_events": round(f8["step_ms_median_events"], 5),
                              "step_p95_events": round(f8["step_ms_p95_events"], 5),
                              "note": "each part timed back to back on its own; events around every step for "
                                      "the median and p95"},
        ("fused_one_launch_step" if args.mode == "separate" else "separate_check_step"): {
            "ms_per_step": round(f8["other_ms"], 5), "value": round(kvb / (f8["other_ms"] * 1e-3) / 1e9, 1)},
        "tracker_off": {"ms_per_step": round(f8["no_tracker_ms"], 5), "check": f8["overhead"]},
        "graph_ms_per_step": round(f8["graph_ms"], 5),
        "timing": "eager back-to-back steps between two events on the launch stream",
    }
    if "bf16" in results:
        b = results["bf16"]
        line["bf16_twin"] = {"value": round(b["kv_bytes"] / (b["step_ms"] * 1e-3) / 1e9, 1), "unit": "GB/s",
                             "ms_per_step": round(b["step_ms"], 5), "attn_ms": round(b["attn_ms"], 5),
                             "attn_gbs": round(b["kv_bytes"] / (b["attn_ms"] * 1e-3) / 1e9, 1),
                             "other_form_ms": round(b["other_ms"], 5), "tracker": b["overhead"],
                             "fp8_speedup_step": round(b["step_ms"] / f8["step_ms"], 3)}
    if sweep:
        line["batch_sweep"] = sweep
    if capacity:
        line["capacity_fixed_budget"] = capacity
    if weight_runs:
        line["weight_gemm"] = weight_runs
    if layer_runs:
        line["layer_stack_step"] = layer_runs | {
            "note": f"one decode step over {args.layers} layers sharing one page table and tag set "
                    "(kv_decode_step_*: layer 0's check + write launch, then its attention; every later layer one "
                    "attention launch that writes the layer's token); graph_us = replay of a captured HIP graph of "
                    "the whole step, graph_fused_us with the check inside layer 0's attention launch, eager_us = "
                    "one library call per step; tracker = overhead of the check (interleaved graph replays with "
                    "and without it, 95 % CI); tokens_per_s = non-aborted requests x steps/s"}
    if extra:
        line["other_workloads"] = extra
    if args.copy_calibration:
        line["copy_calibration_bytes"] = copy_calibration(torch, args.copy_calibration)
    if not args.no_cpu_baseline:
        log(f"cpu baseline: oracle on {args.cpu_sample} requests")
        line["cpu_baseline"] = cpu_baseline(w, args.cpu_sample)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
