"""Paged KV cache: pool layout, append (quantise + scatter), gather, tag check (oracle).

Pages and tags follow the integrity-check description of the Cloudflare post
as the agentlenshq summary gives it (section "KV Cache 完整性检查") and the
xujun.org note (section "一个不能出错的共享缓存"): the cache lives in physical
pages, each request lists its pages, each physical page carries a tag that
changes when the page is reallocated, the server records which pages and tags
each request expects, and a batched check before decode reads the cache
aborts any request whose list no longer matches.

Readings where the pages are silent:

* Page table: int32 [B][stride]; entry i of request r is the physical page
  of its tokens [i*S, (i+1)*S).  Entries at or past ceil(L_r / S) are never
  read or checked.
* Pool layout (element = one e4m3 byte or one bf16; E = 16 bytes of elements).
  Every (page, head) block is contiguous.
    V: [P][Hkv][Dv][S]  element (page, head, d, slot) -- each (page, head)
                        block of V is stored transposed (slot fastest).
    K: [P][Hkv][S/16][16][D] with the 16-token sub-page block reordered in
       16-byte chunks: token t = 4s + i of the sub-page (s, i in 0..3) and
       byte chunk c of its row (c = q*NI + k, NI = D*bytes/64, q in 0..3)
       sit at chunk position ((s*NI + k)*4 + q)*4 + i.  Each group of four
       tokens thus holds, for each k, four 64-byte runs (one per q) of four
       16-byte chunks (one per token).  S must be a multiple of 16 and a
       K row a multiple of 64 bytes.
  Latent cache (one vector per token shared by all query heads; a pool
  written with no V pool):
    C: [P][Hkv][S][Dl] row-major (Hkv = 1), element (page, head, slot, d);
       the tokens of a page are consecutive rows.
* Flags, rewritten on every check (not sticky), uint32 per request:
    bit0 (1) a used entry's page tag differs from the expected tag;
    bit1 (2) a used entry's page id is outside [0, P), or the context needs
             more pages than the page-table row holds.
  A request with L <= 0 uses no pages and gets flag 0.
* Append skips every token of a flagged request; a token whose page is not
  in the pool or whose position is outside its page-table row is skipped.
"""
from __future__ import annotations

import numpy as np

from . import codec

FLAG_TAG_MISMATCH = 1
FLAG_BAD_PAGE = 2


def k_offset(page, head, slot, d, num_kv_heads, page_size, head_dim, elt_bytes):
    """Flat element offset of K element (page, head, slot, d) in the chunk-reordered block."""
    E = 16 // elt_bytes                      # elements per 16-byte chunk
    NI = head_dim * elt_bytes // 64          # chunks per 64-byte slice of a row
    slot = np.asarray(slot, dtype=np.int64)
    d = np.asarray(d, dtype=np.int64)
    u, t = slot // 16, slot % 16
    s, i = t // 4, t % 4
    c = d // E
    q, k = c // NI, c % NI
    chunk = ((s * NI + k) * 4 + q) * 4 + i
    block = (np.int64(page) * num_kv_heads + head) * page_size * head_dim
    return block + u * 16 * head_dim + chunk * E + d % E


def c_offset(page, head, slot, d, num_kv_heads, page_size, dim):
    """Flat element offset of latent element (page, head, slot, d): row-major rows of `dim` elements."""
    slot = np.asarray(slot, dtype=np.int64)
    d = np.asarray(d, dtype=np.int64)
    return ((np.int64(page) * num_kv_heads + head) * page_size + slot) * dim + d


def v_offset(page, head, slot, d, num_kv_heads, page_size, v_dim):
    """Flat element offset of V element (page, head, slot, d) in the transposed block."""
    return ((np.int64(page) * num_kv_heads + head) * v_dim + d) * page_size + slot


def tag_check(page_tags, page_table, expected, ctx_lens, page_size):
    """Batched (page, tag) validation: uint32 flags per request."""
    page_tags = np.asarray(page_tags, dtype=np.uint32)
    P = page_tags.shape[0]
    B, stride = page_table.shape
    flags = np.zeros(B, dtype=np.uint32)
    for r in range(B):
        L = int(ctx_lens[r])
        if L <= 0:
            continue
        n = (L + page_size - 1) // page_size
        f = 0
        if n > stride:
            f |= FLAG_BAD_PAGE
            n = stride
        ids = page_table[r, :n].astype(np.int64)
        bad = (ids < 0) | (ids >= P)
        if bad.any():
            f |= FLAG_BAD_PAGE
        ok = ~bad
        if (page_tags[ids[ok]] != expected[r, :n][ok]).any():
            f |= FLAG_TAG_MISMATCH
        flags[r] = f
    return flags


def _token_targets(tok_req, tok_pos, page_table, num_pages, page_size, flags):
    """(token index, page, slot) of every token the append writes."""
    tok_req = np.asarray(tok_req, dtype=np.int64)
    tok_pos = np.asarray(tok_pos, dtype=np.int64)
    B, stride = page_table.shape
    keep = (tok_req >= 0) & (tok_req < B) & (tok_pos >= 0) & (tok_pos < stride * page_size)
    if flags is not None:
        fl = np.asarray(flags)
        keep &= np.where(keep, fl[np.clip(tok_req, 0, max(B - 1, 0))] == 0, False)
    idx = np.nonzero(keep)[0]
    page = page_table[tok_req[idx], tok_pos[idx] // page_size].astype(np.int64)
    ok = (page >= 0) & (page < num_pages)
    idx, page = idx[ok], page[ok]
    slot = tok_pos[idx] % page_size
    return idx, page, slot


def append(k_pool, v_pool, k_new, v_new, tok_req, tok_pos, page_table, num_kv_heads, page_size,
           flags=None, chunk=4096):
    """Write already-encoded rows into the pools (in place).

    k_pool/v_pool: flat element arrays laid out as in the module docstring
    (v_pool None for the latent cache).  k_new [N][Hkv][D], v_new [N][Hkv][Dv]
    hold the elements to store (e4m3 codes or bf16 bits).  The scatter is a
    plain indexed assignment, token rows in order (later tokens win if two
    land on one slot), done `chunk` tokens at a time to bound memory.
    """
    N, H, D = k_new.shape
    assert H == num_kv_heads
    elt = k_pool.dtype.itemsize
    num_pages = k_pool.size // (H * page_size * D)
    idx, page, slot = _token_targets(tok_req, tok_pos, page_table, num_pages, page_size, flags)
    h = np.arange(H, dtype=np.int64)[None, :, None]
    d = np.arange(D, dtype=np.int64)[None, None, :]
    for a in range(0, idx.size, chunk):
        i, p, s = idx[a:a + chunk], page[a:a + chunk, None, None], slot[a:a + chunk, None, None]
        if v_pool is None:
            k_pool[c_offset(p, h, s, d, H, page_size, D)] = k_new[i]
        else:
            k_pool[k_offset(p, h, s, d, H, page_size, D, elt)] = k_new[i]
        if v_pool is not None:
            Dv = v_new.shape[2]
            dv = np.arange(Dv, dtype=np.int64)[None, None, :]
            v_pool[v_offset(p, h, s, dv, H, page_size, Dv)] = v_new[i]
    return k_pool, v_pool


def append_fp8(k_pool, v_pool, k_bf16, v_bf16, tok_req, tok_pos, page_table, num_kv_heads, page_size,
               k_scale, v_scale, flags=None):
    """FP8 write path: quantise each new row to e4m3 with its tensor's scale, then scatter."""
    kq = codec.quantize_e4m3(k_bf16, k_scale)
    vq = None if v_bf16 is None else codec.quantize_e4m3(v_bf16, v_scale)
    return append(k_pool, v_pool, kq, vq, tok_req, tok_pos, page_table, num_kv_heads, page_size, flags)


def gather(k_pool, v_pool, page_table, r, length, num_kv_heads, page_size, head_dim, v_dim):
    """Request r's first `length` rows read back through its page table.

    Returns (k [L][Hkv][D], v [L][Hkv][Dv] or None), in the pool's element type.
    """
    t = np.arange(length, dtype=np.int64)
    page = page_table[r, t // page_size].astype(np.int64)
    slot = t % page_size
    h = np.arange(num_kv_heads, dtype=np.int64)
    d = np.arange(head_dim, dtype=np.int64)
    if v_pool is None:
        ko = c_offset(page[:, None, None], h[None, :, None], slot[:, None, None], d[None, None, :],
                      num_kv_heads, page_size, head_dim)
    else:
        ko = k_offset(page[:, None, None], h[None, :, None], slot[:, None, None], d[None, None, :],
                      num_kv_heads, page_size, head_dim, k_pool.dtype.itemsize)
    k = k_pool[ko]
    v = None
    if v_pool is not None:
        dv = np.arange(v_dim, dtype=np.int64)
        vo = v_offset(page[:, None, None], h[None, :, None], slot[:, None, None], dv[None, None, :],
                      num_kv_heads, page_size, v_dim)
        v = v_pool[vo]
    return k, v


class PageAllocator:
    """Free list over P pages with the integrity check's page tags (agentlenshq summary, section
    "KV Cache 完整性检查"; xujun.org note, section "一个不能出错的共享缓存": a page's tag changes when
    the page is reallocated, so an old holder's (page, tag) pair no longer matches).

    Readings where the pages are silent: the tag is a uint32 generation counter that goes up by one
    (mod 2**32) each time the page is handed out and is left alone on free; the free list is a stack
    (last freed, first handed out) that starts as 0, 1, 2, ...; a request that cannot be met takes
    nothing ("nospace"); a free that names a page out of range, not in use, or twice frees nothing.
    """

    NOSPACE = "nospace"
    INVALID = "invalid"

    def __init__(self, num_pages, initial_tags=None):
        self.tags = (np.zeros(num_pages, dtype=np.uint32) if initial_tags is None
                     else np.array(initial_tags, dtype=np.uint32))
        self.free_list = list(range(num_pages - 1, -1, -1))   # last element = next handed out
        self.in_use = [False] * num_pages

    @property
    def free_count(self):
        return len(self.free_list)

    def alloc(self, n):
        if n > len(self.free_list):
            return self.NOSPACE
        pages = []
        for _ in range(n):
            p = self.free_list.pop()
            self.in_use[p] = True
            self.tags[p] = np.uint32((int(self.tags[p]) + 1) % 2 ** 32)
            pages.append(p)
        return np.array(pages, dtype=np.int32), self.tags[pages].copy()

    def free(self, pages):
        pages = [int(p) for p in pages]
        if len(set(pages)) != len(pages) or any(p < 0 or p >= len(self.in_use) or not self.in_use[p] for p in pages):
            return self.INVALID
        for p in pages:
            self.in_use[p] = False
            self.free_list.append(p)
        return None


def kv_bytes(requests, tokens, layers, kv_heads, head_dim, bytes_per_element):
    """KV-cache size as the zdabc.icu article writes it (section "显存为什么会成为长上下文推理的瓶颈"):
    requests x tokens x layers x KV heads x head_dim x 2 (K and V) x bytes per element."""
    return requests * tokens * layers * kv_heads * head_dim * 2 * bytes_per_element
