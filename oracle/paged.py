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
* Pools hold the cache in its logical order, as numpy arrays
    K, V    [P][Hkv][S][D]  element (page, kv head, slot, d);
    latent  [P][1][S][Dl]   one vector per token shared by all query heads (no V pool).
  Token t of request r, kv head g, lives at pool[page_table[r][t // S]][g][t % S][:].  Where the
  library keeps these elements in memory is its own business; the tests compare through a mapping
  of their own and the oracle never sees it.
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


def append(k_pool, v_pool, k_new, v_new, tok_req, tok_pos, page_table, flags=None):
    """Write already-encoded rows into the pools (in place).

    k_pool/v_pool: logical pools [P][Hkv][S][D] / [P][Hkv][S][Dv] (v_pool None for the latent cache).
    k_new [N][Hkv][D], v_new [N][Hkv][Dv] hold the elements to store (e4m3 codes or bf16 bits).  Token n
    goes to pool[page_table[tok_req[n]][tok_pos[n] // S]][:][tok_pos[n] % S][:], one token after the
    other in order (a later token wins if two land on one slot).
    """
    P, H, S, _ = k_pool.shape
    assert k_new.shape[1] == H
    idx, page, slot = _token_targets(tok_req, tok_pos, page_table, P, S, flags)
    for n, p, s in zip(idx.tolist(), page.tolist(), slot.tolist()):
        k_pool[p, :, s, :] = k_new[n]
        if v_pool is not None:
            v_pool[p, :, s, :] = v_new[n]
    return k_pool, v_pool


def append_fp8(k_pool, v_pool, k_bf16, v_bf16, tok_req, tok_pos, page_table, k_scale, v_scale, flags=None):
    """FP8 write path: quantise each new row to e4m3 with its tensor's scale, then scatter."""
    kq = codec.quantize_e4m3(k_bf16, k_scale)
    vq = None if v_bf16 is None else codec.quantize_e4m3(v_bf16, v_scale)
    return append(k_pool, v_pool, kq, vq, tok_req, tok_pos, page_table, flags)


def gather(k_pool, v_pool, page_table, r, length):
    """Request r's first `length` tokens read back through its page table.

    Returns (k [L][Hkv][D], v [L][Hkv][Dv] or None), in the pool's element type.
    """
    S = k_pool.shape[2]
    t = np.arange(length, dtype=np.int64)
    page = page_table[r, t // S].astype(np.int64)
    slot = t % S
    k = k_pool[page, :, slot, :]
    v = None if v_pool is None else v_pool[page, :, slot, :]
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
