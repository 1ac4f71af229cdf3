"""Seeded synthetic workloads for paged decode attention over an FP8/BF16 KV cache.

This module only draws random numbers and arranges them into the shapes the
decode path consumes: context lengths, page tables, page tags, expected tags
(with planted stale entries), bf16 queries and per-request bf16 K/V rows, and
the random bytes a page pool starts with.  It holds none of the method's
arithmetic (no quantisation, no scale, no attention); both the CPU oracle and
the GPU path read their inputs from here and from nowhere else.

The workload shapes follow the decode setting the Cloudflare blog post
"Smaller, faster, safer: running Kimi and GLM at scale" describes in its
section "Quantized KV cache" (per-token K and V kept in physical cache pages,
one decode token per request, concurrency 1..64) and the integrity-check
section of the agentlenshq summary of that post ("KV Cache 完整性检查": each
physical page carries a tag, each request has an expected (page, tag) list).
The pages do not give model shapes; the five shapes below are the synthetic
stand-ins for the pages' Kimi K2.6 decode measurements.

Every array comes from numpy.random.Generator(PCG64(seed_sequence)); the seed
sequence names the workload, the request and the tensor, so any single
request can be regenerated on its own (the oracle checks sampled requests of
the large workloads that way).  bf16 values are N(0,1) float32 draws rounded
to bfloat16 by torch's conversion (round to nearest even).
"""
from __future__ import annotations

import dataclasses
import os
from concurrent.futures import ThreadPoolExecutor
from typing import Optional

import numpy as np

# tensor ids inside a request's seed sequence
_T_K, _T_V, _T_LAT, _T_OUTLIER, _T_Q = 1, 2, 3, 4, 5
# stream ids for workload-level draws
_S_CTX, _S_PAGES, _S_TAGS, _S_STALE, _S_POOL_K, _S_POOL_V = 11, 12, 13, 14, 15, 16


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int            # score dimension (576 for the latent cache)
    v_dim: int               # value dimension (512 for the latent cache)
    page_size: int
    num_pages: int           # physical pages in the pool
    ctx_lo: int              # context lengths: uniform integers in [ctx_lo, ctx_hi]
    ctx_hi: int
    seed: int
    latent: bool = False
    num_splits: int = 0      # 0 = let the library choose
    outlier_frac: float = 0.0
    outlier_mult: float = 20.0
    stale: bool = False      # plant stale expected tags in ~1% of requests

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    def with_(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


def _workloads() -> dict:
    w = {}
    w["tiny"] = Workload("tiny", batch=1, num_q_heads=8, num_kv_heads=1, head_dim=128, v_dim=128,
                         page_size=16, num_pages=16, ctx_lo=256, ctx_hi=256, seed=0)
    w["gqa_batch"] = Workload("gqa_batch", batch=32, num_q_heads=64, num_kv_heads=8, head_dim=128,
                              v_dim=128, page_size=16, num_pages=40000, ctx_lo=1024, ctx_hi=8192, seed=1)
    for b in (1, 8, 16, 32, 64):
        w[f"sweep_b{b}"] = Workload(f"sweep_b{b}", batch=b, num_q_heads=64, num_kv_heads=8, head_dim=128,
                                    v_dim=128, page_size=16, num_pages=40000, ctx_lo=8192, ctx_hi=8192,
                                    seed=2, stale=True)
    w["long"] = Workload("long", batch=4, num_q_heads=64, num_kv_heads=8, head_dim=128, v_dim=128,
                         page_size=64, num_pages=16384, ctx_lo=131072, ctx_hi=131072, seed=3,
                         num_splits=32, outlier_frac=0.001, outlier_mult=20.0)
    w["latent"] = Workload("latent", batch=64, num_q_heads=128, num_kv_heads=1, head_dim=576, v_dim=512,
                           page_size=64, num_pages=8192, ctx_lo=4096, ctx_hi=4096, seed=4, latent=True)
    return w


WORKLOADS = _workloads()


def _rng(*ids) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([int(i) for i in ids])))


def to_bf16_bits(x_f32: np.ndarray) -> np.ndarray:
    """Round float32 draws to bfloat16 with torch's conversion; return the raw uint16 bits."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x_f32, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to float32 (exact: a bf16 is the top half of a float32)."""
    return (b.astype(np.uint32) << 16).view(np.float32)


# ----------------------------------------------------------------------------- metadata

def ctx_lens(w: Workload) -> np.ndarray:
    """Context length of every request, counting the token appended this step."""
    if w.ctx_lo == w.ctx_hi:
        return np.full(w.batch, w.ctx_lo, dtype=np.int32)
    return _rng(w.seed, _S_CTX, w.batch).integers(w.ctx_lo, w.ctx_hi, size=w.batch,
                                                    endpoint=True).astype(np.int32)


def pages_needed(lens: np.ndarray, page_size: int) -> np.ndarray:
    return (np.asarray(lens, dtype=np.int64) + page_size - 1) // page_size


def page_table(w: Workload, lens: np.ndarray, stride: Optional[int] = None):
    """Physical pages for every request, drawn without replacement from the pool.

    Entry i of row r holds the page of tokens [i*S, (i+1)*S).  Entries past the
    pages a request uses hold -1, which is not a valid page: a reader that
    touched them would be caught.  Returns (table int32[B][stride], stride).
    """
    need = pages_needed(lens, w.page_size)
    total = int(need.sum())
    if total > w.num_pages:
        raise ValueError(f"{w.name}: {total} pages needed, pool has {w.num_pages}")
    if stride is None:
        stride = int(max(int(need.max()) if len(need) else 1, 1))
    perm = _rng(w.seed, _S_PAGES, w.batch).permutation(w.num_pages)[:total].astype(np.int32)
    pt = np.full((w.batch, stride), -1, dtype=np.int32)
    off = 0
    for r in range(w.batch):
        n = int(need[r])
        pt[r, :n] = perm[off:off + n]
        off += n
    return pt, stride


def page_tags(w: Workload) -> np.ndarray:
    """Current uint32 tag of every physical page (a generation counter's value)."""
    return _rng(w.seed, _S_TAGS, w.batch).integers(0, 2**32, size=w.num_pages, dtype=np.uint32)


def stale_requests(w: Workload) -> np.ndarray:
    """Requests that get one stale expected tag: max(1, round(1% of B)) when B >= 8, none below."""
    if not w.stale or w.batch < 8:
        return np.zeros(0, dtype=np.int64)
    n = max(1, int(round(0.01 * w.batch)))
    return np.sort(_rng(w.seed, _S_STALE, w.batch).choice(w.batch, size=n, replace=False))


def expected_tags(w: Workload, pt: np.ndarray, lens: np.ndarray, tags: np.ndarray,
                  stale: Optional[np.ndarray] = None) -> np.ndarray:
    """The (page, tag) list a request expects: the page's tag at allocation time.

    For each stale request one random used entry holds tag-1 (mod 2**32), as a
    page that was reallocated after the request recorded it would.  Unused
    entries hold 0 and are never read.
    """
    if stale is None:
        stale = stale_requests(w)
    need = pages_needed(lens, w.page_size)
    exp = np.zeros(pt.shape, dtype=np.uint32)
    for r in range(pt.shape[0]):
        n = int(need[r])
        exp[r, :n] = tags[pt[r, :n]]
    rng = _rng(w.seed, _S_STALE, w.batch, 1)
    for r in stale:
        i = int(rng.integers(0, int(need[r])))
        exp[r, i] = np.uint32((int(exp[r, i]) - 1) % 2**32)
    return exp


# ----------------------------------------------------------------------------- values

def queries(w: Workload) -> np.ndarray:
    """bf16 bits [B][Hq][head_dim]."""
    x = _rng(w.seed, _T_Q, w.batch).standard_normal((w.batch, w.num_q_heads, w.head_dim),
                                                    dtype=np.float32)
    return to_bf16_bits(x)


def request_k(w: Workload, r: int, length: int, outliers: bool = True) -> np.ndarray:
    """bf16 bits [L][Hkv][head_dim] of request r's keys (the latent vector when w.latent).

    With w.outlier_frac > 0 and outliers=True, a seeded i.i.d. fraction of the
    elements is multiplied by w.outlier_mult (in float32, then rounded to bf16);
    outliers=False returns the outlier-free draw.
    """
    tid = _T_LAT if w.latent else _T_K
    x = _rng(w.seed, tid, r).standard_normal((length, w.num_kv_heads, w.head_dim), dtype=np.float32)
    b = to_bf16_bits(x)
    if outliers and w.outlier_frac > 0:
        m = _rng(w.seed, _T_OUTLIER, r).random((length, w.num_kv_heads, w.head_dim)) < w.outlier_frac
        big = to_bf16_bits(bf16_bits_to_f32(b[m]) * np.float32(w.outlier_mult))
        b[m] = big
    return b


def request_v(w: Workload, r: int, length: int) -> np.ndarray:
    """bf16 bits [L][Hkv][v_dim] of request r's values (GQA workloads only)."""
    if w.latent:
        raise ValueError("the latent cache has no separate values")
    x = _rng(w.seed, _T_V, r).standard_normal((length, w.num_kv_heads, w.v_dim), dtype=np.float32)
    return to_bf16_bits(x)


def all_kv(w: Workload, lens: np.ndarray, outliers: bool = True, threads: Optional[int] = None):
    """Every request's K (and V), concatenated in request order: ([sum L][Hkv][D], [sum L][Hkv][Dv] or None).

    Requests are generated independently (each has its own stream), so a
    thread pool fills them in parallel with the same result as a serial loop.
    """
    lens = np.asarray(lens, dtype=np.int64)
    total = int(lens.sum())
    offs = np.concatenate([[0], np.cumsum(lens)])
    k = np.empty((total, w.num_kv_heads, w.head_dim), dtype=np.uint16)
    v = None if w.latent else np.empty((total, w.num_kv_heads, w.v_dim), dtype=np.uint16)

    def fill(r):
        a, b = int(offs[r]), int(offs[r + 1])
        k[a:b] = request_k(w, r, b - a, outliers=outliers)
        if v is not None:
            v[a:b] = request_v(w, r, b - a)

    n = threads or min(16, os.cpu_count() or 1)
    if n <= 1 or len(lens) <= 1:
        for r in range(len(lens)):
            fill(r)
    else:
        with ThreadPoolExecutor(n) as ex:
            list(ex.map(fill, range(len(lens))))
    return k, v


def token_index(lens: np.ndarray):
    """(request id int32[N], position int32[N]) of every token, in request order."""
    lens = np.asarray(lens, dtype=np.int64)
    req = np.repeat(np.arange(len(lens), dtype=np.int32), lens)
    offs = np.concatenate([[0], np.cumsum(lens)[:-1]])
    pos = (np.arange(int(lens.sum()), dtype=np.int64) - np.repeat(offs, lens)).astype(np.int32)
    return req, pos


def pool_bytes(w: Workload, which: str, elt_bytes: int, num_pages: Optional[int] = None) -> np.ndarray:
    """Random initial contents of a page pool (uint8, flat): pages never written keep these bytes."""
    p = w.num_pages if num_pages is None else num_pages
    if which == "k":
        n = p * w.num_kv_heads * w.page_size * w.head_dim * elt_bytes
        sid = _S_POOL_K
    else:
        n = p * w.num_kv_heads * w.page_size * w.v_dim * elt_bytes
        sid = _S_POOL_V
    return np.frombuffer(_rng(w.seed, sid, elt_bytes).bytes(n), dtype=np.uint8).copy()


def pool_init(w: Workload, which: str, elt_bytes: int, num_pages: Optional[int] = None) -> np.ndarray:
    """The same random bytes as pool_bytes, viewed as a pool in logical order [P][Hkv][S][D]
    (uint8 elements for elt_bytes 1, uint16 for 2)."""
    p = w.num_pages if num_pages is None else num_pages
    d = w.head_dim if which == "k" else w.v_dim
    flat = pool_bytes(w, which, elt_bytes, p)
    return flat.view(np.uint8 if elt_bytes == 1 else np.uint16).reshape(p, w.num_kv_heads, w.page_size, d)


def rotation_tables(w: Workload, lens: np.ndarray, copies: int):
    """`copies` page tables over disjoint page sets of one pool, for timing loops that rotate through
    them so that consecutive steps read different memory.  The pool has max(w.num_pages, copies x the
    pages one batch needs) pages; its pages are drawn without replacement across all copies.  Returns
    (tables int32 [copies][B][stride], num_pages)."""
    need = int(pages_needed(lens, w.page_size).sum())
    P = max(w.num_pages, copies * need)
    wb = w.with_(batch=w.batch * copies, num_pages=P)
    pt, stride = page_table(wb, np.tile(np.asarray(lens, dtype=np.int32), copies))
    return pt.reshape(copies, w.batch, stride), P
