"""MI355X (gfx950) paged decode attention over an FP8 e4m3 or BF16 KV cache.

Thin Python binding over libkvfp8.so (C ABI in include/kvfp8.h).  Every
function here only checks and marshals torch tensors (device, dtype,
contiguity) and passes raw pointers plus the current HIP stream; all work
runs in the library's HIP kernels.  There is no CPU fallback: if the library
is missing, calls raise.

bf16 tensors may be passed as torch.bfloat16 or as 16-bit integer views;
e4m3 pools as torch.uint8 (or torch.float8_e4m3fn).
"""
from __future__ import annotations

from typing import Optional

import torch

from . import _lib
from ._lib import (FLAG_BAD_PAGE, FLAG_TAG_MISMATCH, KVFP8_ERR_NOSPACE, READ_SINK_WORDS, LayerStack,  # noqa: F401
                   PoolDesc)

__all__ = ["KvFp8Error", "PoolDesc", "pool_desc", "kv_absmax_bf16", "kv_scale_from_absmax", "calibrate_scale",
           "kv_append_fp8", "kv_append_bf16", "kv_tag_check", "kv_tag_check_append_fp8",
           "kv_tag_check_append_bf16", "paged_decode_attn_workspace_bytes",
           "paged_decode_attn_auto_splits", "paged_decode_attn_fp8", "paged_decode_attn_bf16", "paged_decode_attn_fp8_noalloc",
           "paged_decode_attn_latent_auto_splits", "paged_decode_attn_latent_fp8",
           "paged_decode_attn_latent_bf16", "kv_gather_fp8", "kv_gather_bf16", "decode_step", "decode_step_layers", "PageAllocator",
           "w4_quantize_bf16", "w8_quantize_bf16", "wgemm_auto_splits", "wgemm_workspace_bytes", "w4a16_gemm",
           "w8a16_gemm", "kv_read_stream", "kv_read_blocks", "READ_SINK_WORDS",
           "lib"]


class KvFp8Error(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {_lib.STATUS.get(status, status)} ({lib().kvfp8_status_string(status).decode()})")


def lib():
    return _lib.load()


def _check(status: int, where: str):
    if status != _lib.KVFP8_OK:
        raise KvFp8Error(status, where)


_BF16 = (torch.bfloat16, torch.int16, torch.uint16) if hasattr(torch, "uint16") else (torch.bfloat16, torch.int16)
_U8 = (torch.uint8, torch.float8_e4m3fn)
_I32 = (torch.int32,)
_U32 = (torch.int32, torch.uint32) if hasattr(torch, "uint32") else (torch.int32,)


def _ptr(t: Optional[torch.Tensor], dtypes, name: str, allow_none=False):
    if t is None:
        if allow_none:
            return None
        raise ValueError(f"{name} is required")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if t.dtype not in dtypes:
        raise TypeError(f"{name}: dtype {t.dtype} not in {dtypes}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


def _stream(stream=None):
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def pool_desc(num_pages, page_size, num_kv_heads, head_dim, v_dim=None) -> PoolDesc:
    return PoolDesc(int(num_pages), int(page_size), int(num_kv_heads), int(head_dim),
                    int(head_dim if v_dim is None else v_dim))


# ----------------------------------------------------------------------------- scale

def kv_absmax_bf16(x: torch.Tensor, absmax_bits: torch.Tensor, stream=None):
    """Max-accumulate max|x| (float32 bits) into absmax_bits[0] (a device int32/uint32 tensor)."""
    _check(lib().kv_absmax_bf16(_ptr(x, _BF16, "x"), x.numel(), _ptr(absmax_bits, _U32, "absmax_bits"),
                                _stream(stream)), "kv_absmax_bf16")


def kv_scale_from_absmax(absmax_bits: int) -> float:
    return float(lib().kv_scale_from_absmax(int(absmax_bits) & 0xFFFFFFFF))


def calibrate_scale(*tensors: torch.Tensor) -> float:
    """Per-tensor scale fl32(max|x| / 448) over one or more bf16 device tensors (synchronises once)."""
    acc = torch.zeros(1, dtype=torch.int32, device=tensors[0].device)
    for t in tensors:
        kv_absmax_bf16(t, acc)
    return kv_scale_from_absmax(int(acc.item()))


# ----------------------------------------------------------------------------- write path

def kv_append_fp8(desc: PoolDesc, k_pool, v_pool, k_new, v_new, tok_req, tok_pos, page_table,
                  abort_flags=None, *, k_scale: float, v_scale: float = 1.0, stream=None):
    B, stride = page_table.shape
    _check(lib().kv_append_fp8(
        desc, _ptr(k_pool, _U8, "k_pool"), _ptr(v_pool, _U8, "v_pool", True), _ptr(k_new, _BF16, "k_new"),
        _ptr(v_new, _BF16, "v_new", True), _ptr(tok_req, _I32, "tok_req"), _ptr(tok_pos, _I32, "tok_pos"),
        tok_req.numel(), _ptr(page_table, _I32, "page_table"), B, stride,
        _ptr(abort_flags, _U32, "abort_flags", True), float(k_scale), float(v_scale), _stream(stream)),
        "kv_append_fp8")


def kv_append_bf16(desc: PoolDesc, k_pool, v_pool, k_new, v_new, tok_req, tok_pos, page_table,
                   abort_flags=None, *, stream=None):
    B, stride = page_table.shape
    _check(lib().kv_append_bf16(
        desc, _ptr(k_pool, _BF16, "k_pool"), _ptr(v_pool, _BF16, "v_pool", True), _ptr(k_new, _BF16, "k_new"),
        _ptr(v_new, _BF16, "v_new", True), _ptr(tok_req, _I32, "tok_req"), _ptr(tok_pos, _I32, "tok_pos"),
        tok_req.numel(), _ptr(page_table, _I32, "page_table"), B, stride,
        _ptr(abort_flags, _U32, "abort_flags", True), _stream(stream)), "kv_append_bf16")


# ----------------------------------------------------------------------------- integrity check

def kv_tag_check(page_tags, page_table, expected_tags, ctx_lens, page_size: int, abort_flags, stream=None):
    B, stride = page_table.shape
    _check(lib().kv_tag_check(
        _ptr(page_tags, _U32, "page_tags"), page_tags.numel(), _ptr(page_table, _I32, "page_table"),
        _ptr(expected_tags, _U32, "expected_tags"), stride, _ptr(ctx_lens, _I32, "ctx_lens"), B, int(page_size),
        _ptr(abort_flags, _U32, "abort_flags"), _stream(stream)), "kv_tag_check")


def kv_tag_check_append_fp8(desc: PoolDesc, k_pool, v_pool, k_new, v_new, page_table, ctx_lens, page_tags,
                            expected_tags, abort_flags, *, k_scale: float, v_scale: float = 1.0, stream=None):
    """One launch: tag check, then each clean request's token r written at position ctx_lens[r] - 1."""
    B, stride = page_table.shape
    _check(lib().kv_tag_check_append_fp8(
        desc, _ptr(k_pool, _U8, "k_pool"), _ptr(v_pool, _U8, "v_pool", True), _ptr(k_new, _BF16, "k_new"),
        _ptr(v_new, _BF16, "v_new", True), _ptr(page_table, _I32, "page_table"), stride,
        _ptr(ctx_lens, _I32, "ctx_lens"), B, _ptr(page_tags, _U32, "page_tags"),
        _ptr(expected_tags, _U32, "expected_tags"), _ptr(abort_flags, _U32, "abort_flags"), float(k_scale),
        float(v_scale), _stream(stream)), "kv_tag_check_append_fp8")


def kv_tag_check_append_bf16(desc: PoolDesc, k_pool, v_pool, k_new, v_new, page_table, ctx_lens, page_tags,
                             expected_tags, abort_flags, *, stream=None):
    B, stride = page_table.shape
    _check(lib().kv_tag_check_append_bf16(
        desc, _ptr(k_pool, _BF16, "k_pool"), _ptr(v_pool, _BF16, "v_pool", True), _ptr(k_new, _BF16, "k_new"),
        _ptr(v_new, _BF16, "v_new", True), _ptr(page_table, _I32, "page_table"), stride,
        _ptr(ctx_lens, _I32, "ctx_lens"), B, _ptr(page_tags, _U32, "page_tags"),
        _ptr(expected_tags, _U32, "expected_tags"), _ptr(abort_flags, _U32, "abort_flags"), _stream(stream)),
        "kv_tag_check_append_bf16")


# ----------------------------------------------------------------------------- attention

def paged_decode_attn_workspace_bytes(batch, num_q_heads, v_dim, num_splits) -> int:
    return int(lib().paged_decode_attn_workspace_bytes(int(batch), int(num_q_heads), int(v_dim), int(num_splits)))


def paged_decode_attn_auto_splits(batch, num_kv_heads, max_ctx_len) -> int:
    return int(lib().paged_decode_attn_auto_splits(int(batch), int(num_kv_heads), int(max_ctx_len)))


def decode_step_layers(desc: PoolDesc, kv_dtype: str, k_pools, v_pools, page_table, ctx_lens, max_ctx_len: int,
                       q, k_new, v_new, out, *, page_tags=None, expected_tags=None, abort_flags=None,
                       k_scales=None, v_scales=None, sm_scale: float = 0.0, num_splits: int = 0,
                       workspace=None, stream=None, fused_check: bool = False):
    """One decode step over a stack of layers sharing the page table, tags and flags (kv_decode_step_*):
    the tag check once, as its own launch with layer 0's write (fused_check: inside layer 0's attention
    launch instead), then each layer's write and attention in stream order.  sm_scale 0 lets the
    library use 1/sqrt(score dim).

    k_pools/v_pools: [layers][pool elements] (v_pools None: the latent cache, v_new None too);
    q [layers][B][Hq][D]; k_new/v_new [layers][B][Hkv][D|Dv]; out [layers][B][Hq][Dv];
    k_scales/v_scales: per-layer floats (FP8).  page_tags None = no-op tracker."""
    import numpy as np
    if kv_dtype not in ("fp8", "bf16"):
        raise ValueError(f"kv_dtype {kv_dtype!r}")
    fp8 = kv_dtype == "fp8"
    pool_t = _U8 if fp8 else _BF16
    n_layers, B, Hq, D = q.shape
    latent = v_pools is None
    for name, t in (("k_pools", k_pools), ("v_pools", v_pools), ("k_new", k_new), ("v_new", v_new), ("out", out)):
        if t is not None and t.shape[0] != n_layers:
            raise ValueError(f"{name}: {t.shape[0]} layers, q has {n_layers}")
    Hkv, Dk, Dv = desc.num_kv_heads, desc.head_dim, desc.v_dim
    if D != Dk or k_new.numel() != n_layers * B * Hkv * Dk or out.numel() != n_layers * B * Hq * Dv or (
            not latent and (v_new is None or v_new.numel() != n_layers * B * Hkv * Dv)):
        raise ValueError("q, k_new, v_new and out must be [layers][B][heads][dim] stacks of the descriptor's shape")
    if page_table.shape[0] != B or ctx_lens.numel() != B:
        raise ValueError("page_table and ctx_lens need one row per request")
    slots = desc.num_pages * desc.page_size * desc.num_kv_heads
    if k_pools.numel() != n_layers * slots * desc.head_dim or (
            not latent and v_pools.numel() != n_layers * slots * desc.v_dim):
        raise ValueError("each layer's pool must hold exactly the pool the descriptor describes")
    ks = vs = None
    if fp8:
        if k_scales is None or (not latent and v_scales is None):
            raise ValueError("the FP8 cache needs per-layer scales")
        ks = np.ascontiguousarray(np.asarray(k_scales, dtype=np.float32).reshape(-1))
        vs = None if latent else np.ascontiguousarray(np.asarray(v_scales, dtype=np.float32).reshape(-1))
        if ks.size != n_layers or (vs is not None and vs.size != n_layers):
            raise ValueError("one K (and V) scale per layer")
    stack = LayerStack(n_layers, _ptr(k_pools, pool_t, "k_pools"), _ptr(v_pools, pool_t, "v_pools", True),
                       _ptr(q, _BF16, "q"), _ptr(k_new, _BF16, "k_new"), _ptr(v_new, _BF16, "v_new", True),
                       None if ks is None else ks.ctypes.data, None if vs is None else vs.ctypes.data,
                       _ptr(out, _BF16, "out"), _lib.STEP_FUSED_CHECK if fused_check else 0)
    ws, wsb = _ws(workspace)
    f = lib().kv_decode_step_fp8 if fp8 else lib().kv_decode_step_bf16
    _check(f(desc, stack, Hq, _ptr(page_table, _I32, "page_table"), page_table.shape[1],
             _ptr(ctx_lens, _I32, "ctx_lens"), B, int(max_ctx_len), _ptr(page_tags, _U32, "page_tags", True),
             _ptr(expected_tags, _U32, "expected_tags", True), _ptr(abort_flags, _U32, "abort_flags", True),
             float(sm_scale), int(num_splits), ws, wsb, _stream(stream)), f"kv_decode_step_{kv_dtype}")


def _ws(workspace):
    if workspace is None:
        return None, 0
    if not workspace.is_cuda or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous device tensor")
    return workspace.data_ptr(), workspace.numel() * workspace.element_size()


def paged_decode_attn_fp8(desc: PoolDesc, q, k_pool, v_pool, page_table, ctx_lens, max_ctx_len: int, out,
                          abort_flags=None, *, k_scale: float, v_scale: float, sm_scale: float = 0.0,
                          num_splits: int = 0, workspace=None, stream=None):
    B, Hq, D = q.shape
    ws, wsb = _ws(workspace)
    _check(lib().paged_decode_attn_fp8(
        desc, _ptr(q, _BF16, "q"), Hq, _ptr(k_pool, _U8, "k_pool"), _ptr(v_pool, _U8, "v_pool"),
        _ptr(page_table, _I32, "page_table"), page_table.shape[1], _ptr(ctx_lens, _I32, "ctx_lens"), B,
        int(max_ctx_len), _ptr(abort_flags, _U32, "abort_flags", True), float(k_scale), float(v_scale),
        float(sm_scale), int(num_splits), ws, wsb, _ptr(out, _BF16, "out"), _stream(stream)),
        "paged_decode_attn_fp8")


def paged_decode_attn_fp8_noalloc(desc: PoolDesc, q, k_pool, v_pool, page_table, ctx_lens, max_ctx_len: int, out,
                                  abort_flags=None, *, k_scale: float, v_scale: float, sm_scale: float = 0.0,
                                  num_splits: int = 0, stream=None):
    """paged_decode_attn_fp8 with the split partials in the library's own device scratch (no workspace)."""
    B, Hq, D = q.shape
    _check(lib().paged_decode_attn_fp8_noalloc(
        desc, _ptr(q, _BF16, "q"), Hq, _ptr(k_pool, _U8, "k_pool"), _ptr(v_pool, _U8, "v_pool"),
        _ptr(page_table, _I32, "page_table"), page_table.shape[1], _ptr(ctx_lens, _I32, "ctx_lens"), B,
        int(max_ctx_len), _ptr(abort_flags, _U32, "abort_flags", True), float(k_scale), float(v_scale),
        float(sm_scale), int(num_splits), _ptr(out, _BF16, "out"), _stream(stream)),
        "paged_decode_attn_fp8_noalloc")


def paged_decode_attn_bf16(desc: PoolDesc, q, k_pool, v_pool, page_table, ctx_lens, max_ctx_len: int, out,
                           abort_flags=None, *, sm_scale: float = 0.0, num_splits: int = 0,
                           workspace=None, stream=None):
    B, Hq, D = q.shape
    ws, wsb = _ws(workspace)
    _check(lib().paged_decode_attn_bf16(
        desc, _ptr(q, _BF16, "q"), Hq, _ptr(k_pool, _BF16, "k_pool"), _ptr(v_pool, _BF16, "v_pool"),
        _ptr(page_table, _I32, "page_table"), page_table.shape[1], _ptr(ctx_lens, _I32, "ctx_lens"), B,
        int(max_ctx_len), _ptr(abort_flags, _U32, "abort_flags", True), float(sm_scale), int(num_splits), ws, wsb,
        _ptr(out, _BF16, "out"), _stream(stream)), "paged_decode_attn_bf16")


def paged_decode_attn_latent_auto_splits(batch, num_q_heads, max_ctx_len) -> int:
    return int(lib().paged_decode_attn_latent_auto_splits(int(batch), int(num_q_heads), int(max_ctx_len)))


def paged_decode_attn_latent_fp8(desc: PoolDesc, q, pool, page_table, ctx_lens, max_ctx_len: int, out,
                                 abort_flags=None, *, scale: float, sm_scale: float = 0.0,
                                 num_splits: int = 0, workspace=None, stream=None):
    B, Hq, D = q.shape
    ws, wsb = _ws(workspace)
    _check(lib().paged_decode_attn_latent_fp8(
        desc, _ptr(q, _BF16, "q"), Hq, _ptr(pool, _U8, "pool"), _ptr(page_table, _I32, "page_table"),
        page_table.shape[1], _ptr(ctx_lens, _I32, "ctx_lens"), B, int(max_ctx_len),
        _ptr(abort_flags, _U32, "abort_flags", True), float(scale), float(sm_scale), int(num_splits), ws, wsb,
        _ptr(out, _BF16, "out"), _stream(stream)), "paged_decode_attn_latent_fp8")


def paged_decode_attn_latent_bf16(desc: PoolDesc, q, pool, page_table, ctx_lens, max_ctx_len: int, out,
                                  abort_flags=None, *, sm_scale: float = 0.0, num_splits: int = 0,
                                  workspace=None, stream=None):
    B, Hq, D = q.shape
    ws, wsb = _ws(workspace)
    _check(lib().paged_decode_attn_latent_bf16(
        desc, _ptr(q, _BF16, "q"), Hq, _ptr(pool, _BF16, "pool"), _ptr(page_table, _I32, "page_table"),
        page_table.shape[1], _ptr(ctx_lens, _I32, "ctx_lens"), B, int(max_ctx_len),
        _ptr(abort_flags, _U32, "abort_flags", True), float(sm_scale), int(num_splits), ws, wsb,
        _ptr(out, _BF16, "out"), _stream(stream)), "paged_decode_attn_latent_bf16")


# ----------------------------------------------------------------------------- weight-quantised GEMM

def _wq_check(w_or_x, n, k, packed, scales, bits):
    need = lib().w4_packed_bytes(n, k) if bits == 4 else lib().w8_packed_bytes(n, k)
    if need == 0:
        raise ValueError(f"unsupported weight shape {n} x {k} (N a multiple of 16, K of 256)")
    if packed.numel() * packed.element_size() != need:
        raise ValueError(f"packed codes: {packed.numel() * packed.element_size()} bytes, the layout needs {need}")
    if scales.numel() != lib().wq_scales_count(n, k):
        raise ValueError("scales: one bf16 per output channel and group of 128 input channels")


def w4_quantize_bf16(w, packed, scales, stream=None):
    """bf16 weights w [N][K] -> INT4 codes (packed, uint8 [N*K/2]) and bf16 group scales [N/16][K/128][16]."""
    n, k = w.shape
    _wq_check(w, n, k, packed, scales, 4)
    _check(lib().w4_quantize_bf16(_ptr(w, _BF16, "w"), n, k, _ptr(packed, _U8, "packed"),
                                  _ptr(scales, _BF16, "scales"), _stream(stream)), "w4_quantize_bf16")


def w8_quantize_bf16(w, packed, scales, stream=None):
    """bf16 weights w [N][K] -> e4m3 codes (packed, uint8 [N*K]) and bf16 group scales [N/16][K/128][16]."""
    n, k = w.shape
    _wq_check(w, n, k, packed, scales, 8)
    _check(lib().w8_quantize_bf16(_ptr(w, _BF16, "w"), n, k, _ptr(packed, _U8, "packed"),
                                  _ptr(scales, _BF16, "scales"), _stream(stream)), "w8_quantize_bf16")


def wgemm_auto_splits(m, n, k) -> int:
    return int(lib().wgemm_auto_splits(int(m), int(n), int(k)))


def wgemm_workspace_bytes(m, n, k, num_splits) -> int:
    return int(lib().wgemm_workspace_bytes(int(m), int(n), int(k), int(num_splits)))


def _wgemm(bits, x, w_packed, scales, n, k, y, num_splits, workspace, stream):
    m = x.shape[0]
    if x.shape != (m, k) or y.shape != (m, n):
        raise ValueError(f"x must be [M][{k}] and y [M][{n}]")
    _wq_check(x, n, k, w_packed, scales, bits)
    ws, wsb = _ws(workspace)
    f = lib().w4a16_gemm if bits == 4 else lib().w8a16_gemm
    _check(f(_ptr(x, _BF16, "x"), m, _ptr(w_packed, _U8, "w_packed"), _ptr(scales, _BF16, "scales"), int(n),
             int(k), int(num_splits), ws, wsb, _ptr(y, _BF16, "y"), _stream(stream)), f"w{bits}a16_gemm")


def w4a16_gemm(x, w_packed, scales, n, k, y, *, num_splits: int = 0, workspace=None, stream=None):
    """y [M][N] (bf16) = x [M][K] (bf16) times the INT4 weights (packed by w4_quantize_bf16), transposed.
    With several splits, `workspace` (wgemm_workspace_bytes) must have been zeroed once before its first use."""
    _wgemm(4, x, w_packed, scales, n, k, y, num_splits, workspace, stream)


def w8a16_gemm(x, w_packed, scales, n, k, y, *, num_splits: int = 0, workspace=None, stream=None):
    """y [M][N] (bf16) = x [M][K] (bf16) times the FP8 weights (packed by w8_quantize_bf16), transposed."""
    _wgemm(8, x, w_packed, scales, n, k, y, num_splits, workspace, stream)


# ----------------------------------------------------------------------------- read-rate calibration

def kv_read_stream(src, sink, nbytes=None, stream=None):
    """Read nbytes (default: all) of a device tensor; sink: int32/uint32 [READ_SINK_WORDS] checksum words."""
    n = src.numel() * src.element_size() if nbytes is None else int(nbytes)
    if not src.is_cuda or not src.is_contiguous():
        raise ValueError("src must be a contiguous device tensor")
    _check(lib().kv_read_stream(src.data_ptr(), n, _ptr(sink, _U32, "sink"), _stream(stream)), "kv_read_stream")


def kv_read_blocks(base, block_bytes, ids, sink, stream=None):
    """Read the block_bytes-byte blocks ids[k] of a device tensor (ids int32 on the device)."""
    if not base.is_cuda or not base.is_contiguous():
        raise ValueError("base must be a contiguous device tensor")
    nb = base.numel() * base.element_size() // int(block_bytes)
    _check(lib().kv_read_blocks(base.data_ptr(), nb, int(block_bytes), _ptr(ids, _I32, "ids"), ids.numel(),
                                _ptr(sink, _U32, "sink"), _stream(stream)), "kv_read_blocks")


# ----------------------------------------------------------------------------- read back (tests)

def kv_gather_fp8(desc: PoolDesc, k_pool, v_pool, tok_req, tok_pos, page_table, k_out, v_out=None, stream=None):
    B, stride = page_table.shape
    _check(lib().kv_gather_fp8(
        desc, _ptr(k_pool, _U8, "k_pool"), _ptr(v_pool, _U8, "v_pool", True), _ptr(tok_req, _I32, "tok_req"),
        _ptr(tok_pos, _I32, "tok_pos"), tok_req.numel(), _ptr(page_table, _I32, "page_table"), B, stride,
        _ptr(k_out, _U8, "k_out"), _ptr(v_out, _U8, "v_out", True), _stream(stream)), "kv_gather_fp8")


def kv_gather_bf16(desc: PoolDesc, k_pool, v_pool, tok_req, tok_pos, page_table, k_out, v_out=None, stream=None):
    B, stride = page_table.shape
    _check(lib().kv_gather_bf16(
        desc, _ptr(k_pool, _BF16, "k_pool"), _ptr(v_pool, _BF16, "v_pool", True), _ptr(tok_req, _I32, "tok_req"),
        _ptr(tok_pos, _I32, "tok_pos"), tok_req.numel(), _ptr(page_table, _I32, "page_table"), B, stride,
        _ptr(k_out, _BF16, "k_out"), _ptr(v_out, _BF16, "v_out", True), _stream(stream)), "kv_gather_bf16")


# ----------------------------------------------------------------------------- page allocator

class PageAllocator:
    """The library's host-side page allocator (kv_page_alloc_*): a free list over a pool's pages whose
    tags change each time a page is handed to a new owner.  The state lives in a numpy buffer owned here."""

    def __init__(self, num_pages: int, initial_tags=None):
        import numpy as np
        n = lib().kv_page_alloc_state_bytes(num_pages)
        if n == 0:
            raise KvFp8Error(-2, "kv_page_alloc_state_bytes")
        self.num_pages = num_pages
        self._state = np.zeros((n + 3) // 4, dtype=np.uint32)
        tags = None if initial_tags is None else np.ascontiguousarray(initial_tags, dtype=np.uint32)
        if tags is not None and tags.shape != (num_pages,):
            raise ValueError("initial_tags must have one entry per page")
        _check(lib().kv_page_alloc_init(self._state.ctypes.data, self._state.nbytes, num_pages,
                                        None if tags is None else tags.ctypes.data), "kv_page_alloc_init")
        self._keep = tags

    @property
    def free_count(self) -> int:
        return int(lib().kv_page_alloc_free_count(self._state.ctypes.data))

    def alloc(self, n: int):
        """n pages (int32) and their new tags (uint32); raises KvFp8Error(KVFP8_ERR_NOSPACE) if short."""
        import numpy as np
        pages = np.empty(n, dtype=np.int32)
        tags = np.empty(n, dtype=np.uint32)
        _check(lib().kv_page_alloc(self._state.ctypes.data, n, pages.ctypes.data, tags.ctypes.data), "kv_page_alloc")
        return pages, tags

    def free(self, pages):
        import numpy as np
        pages = np.ascontiguousarray(pages, dtype=np.int32)
        _check(lib().kv_page_free(self._state.ctypes.data, pages.ctypes.data, pages.size), "kv_page_free")

    def tags(self):
        """The current tag of every page (host uint32 [P]), for upload to the device tag array."""
        import numpy as np
        out = np.empty(self.num_pages, dtype=np.uint32)
        _check(lib().kv_page_alloc_tags(self._state.ctypes.data, out.ctypes.data), "kv_page_alloc_tags")
        return out


# ----------------------------------------------------------------------------- one decode step

def decode_step(desc: PoolDesc, kv_dtype: str, k_pool, v_pool, page_table, ctx_lens, max_ctx_len: int, q,
                k_new, v_new, tok_req, tok_pos, out, *, page_tags=None, expected_tags=None, abort_flags=None,
                k_scale: float = 1.0, v_scale: float = 1.0, sm_scale: float = 0.0, num_splits: int = 0,
                workspace=None, stream=None, fused_check: bool = False):
    """One attention layer's decode step, in stream order: tag check -> append -> attention.

    With page_tags/expected_tags given, the batched check writes abort_flags
    first and the write and the attention honour them; with page_tags None
    (the no-op tracker) no check runs and abort_flags is passed through
    (None = no flags).  tok_req/tok_pos None means one new token per
    request, at position ctx_lens[r] - 1: the step is then kv_decode_step_*
    over this one layer: the check + write launch, then the attention (with
    no tracker, one attention launch whose block holding position L - 1
    writes the token); fused_check puts the check in the attention launch
    (one launch for the GQA and FP8 latent caches).  Otherwise three
    launches: kv_tag_check, kv_append_*, the attention.
    """
    if kv_dtype not in ("fp8", "bf16"):
        raise ValueError(f"kv_dtype {kv_dtype!r}")
    if page_tags is not None and (expected_tags is None or abort_flags is None):
        raise ValueError("the tag check needs expected_tags and an abort_flags buffer")
    if (tok_req is None) != (tok_pos is None):
        raise ValueError("tok_req and tok_pos are given together or not at all")
    if tok_req is None:
        fp8 = kv_dtype == "fp8"
        latent = v_pool is None
        decode_step_layers(desc, kv_dtype, k_pool.reshape(1, -1), None if latent else v_pool.reshape(1, -1),
                           page_table, ctx_lens, max_ctx_len, q.unsqueeze(0), k_new.unsqueeze(0),
                           None if latent else v_new.unsqueeze(0), out.unsqueeze(0), page_tags=page_tags,
                           expected_tags=expected_tags, abort_flags=abort_flags,
                           k_scales=[k_scale] if fp8 else None,
                           v_scales=[v_scale] if fp8 and not latent else None, sm_scale=sm_scale,
                           num_splits=num_splits, workspace=workspace, stream=stream, fused_check=fused_check)
        return
    if page_tags is not None:
        kv_tag_check(page_tags, page_table, expected_tags, ctx_lens, desc.page_size, abort_flags, stream=stream)
    if kv_dtype == "fp8":
        kv_append_fp8(desc, k_pool, v_pool, k_new, v_new, tok_req, tok_pos, page_table, abort_flags,
                      k_scale=k_scale, v_scale=v_scale, stream=stream)
        paged_decode_attn_fp8(desc, q, k_pool, v_pool, page_table, ctx_lens, max_ctx_len, out, abort_flags,
                              k_scale=k_scale, v_scale=v_scale, sm_scale=sm_scale, num_splits=num_splits,
                              workspace=workspace, stream=stream)
    else:
        kv_append_bf16(desc, k_pool, v_pool, k_new, v_new, tok_req, tok_pos, page_table, abort_flags,
                       stream=stream)
        paged_decode_attn_bf16(desc, q, k_pool, v_pool, page_table, ctx_lens, max_ctx_len, out, abort_flags,
                               sm_scale=sm_scale, num_splits=num_splits, workspace=workspace, stream=stream)
