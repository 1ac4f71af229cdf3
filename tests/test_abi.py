"""The C ABI on the CPU: the header is plain C, the library loads and exports every declared entry
point, and host-side argument checks return their status codes before touching any device."""
import ctypes as C
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kvfp8.h")
HEADERS = [os.path.join(ROOT, "include", h) for h in sorted(os.listdir(os.path.join(ROOT, "include")))
           if h.endswith(".h")]


def _declared():
    src = "\n".join(open(h).read() for h in HEADERS)
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\*?\s*([a-z_][a-z0-9_]*)\s*\(", src, flags=re.M)
    return sorted(set(names))


def test_header_declares_the_entry_points():
    names = _declared()
    for n in ["kv_append_fp8", "kv_append_bf16", "kv_tag_check", "paged_decode_attn_fp8", "paged_decode_attn_bf16",
              "paged_decode_attn_workspace_bytes", "kv_gather_fp8", "kv_gather_bf16", "kv_absmax_bf16",
              "kv_scale_from_absmax", "kvfp8_abi_version", "kvfp8_status_string"]:
        assert n in names, n


def test_header_compiles_as_c_and_cxx():
    for h in HEADERS:
        for lang, std in (("c", "-std=c11"), ("c++", "-std=c++17")):
            r = subprocess.run(["gcc", "-x", lang, std, "-Wall", "-Werror", "-fsyntax-only", h],
                               capture_output=True, text=True)
            assert r.returncode == 0, (h, r.stderr)


@pytest.fixture(scope="module")
def lib():
    from fp8_paged_kv_append_amd import _lib
    return _lib.load()


def test_library_exports_every_declared_symbol(lib):
    from fp8_paged_kv_append_amd import _lib
    for n in _declared():
        assert hasattr(lib, n), n
        assert n in _lib.PROTOTYPES, n


def test_version_and_status_strings(lib):
    assert lib.kvfp8_abi_version() == 2
    for s in range(-8, 1):
        assert lib.kvfp8_status_string(s).decode() not in ("", "unknown status")
    assert lib.kvfp8_status_string(5) == b"unknown status"


def test_scale_from_absmax_is_fp32_division(lib):
    import numpy as np
    for a in [3.0, 4.5, 1e-3, 17.25, 3.3e38]:
        bits = int(np.float32(a).view(np.uint32))
        assert lib.kv_scale_from_absmax(bits) == float(np.float32(a) / np.float32(448))


def test_host_validation_codes(lib):
    from fp8_paged_kv_append_amd import _lib
    d = _lib.PoolDesc(16, 16, 1, 128, 128)
    A = 4096                      # a fake, 16-byte aligned "device" address; never dereferenced
    # null descriptor / pointers
    assert lib.kv_append_fp8(None, A, A, A, A, A, A, 1, A, 1, 1, None, 1.0, 1.0, None) == -1
    assert lib.kv_append_fp8(d, None, A, A, A, A, A, 1, A, 1, 1, None, 1.0, 1.0, None) == -1
    assert lib.kv_append_fp8(d, A, None, A, A, A, A, 1, A, 1, 1, None, 1.0, 1.0, None) == -1   # v_pool w/o v_new
    # shapes and values
    assert lib.kv_append_fp8(d, A, A, A, A, A, A, -1, A, 1, 1, None, 1.0, 1.0, None) == -2
    assert lib.kv_append_fp8(d, A, A, A, A, A, A, 0, A, 1, 1, None, 1.0, 1.0, None) == 0      # nothing to do
    assert lib.kv_append_fp8(d, A, A, A, A, A, A, 1, A, 1, 1, None, 0.0, 1.0, None) == -7
    assert lib.kv_append_fp8(d, A, A, A, A, A, A, 1, A, 1, 1, None, float("nan"), 1.0, None) == -7
    assert lib.kv_append_fp8(d, A + 2, A, A, A, A, A, 1, A, 1, 1, None, 1.0, 1.0, None) == -5
    bad = _lib.PoolDesc(16, 24, 1, 128, 128)                        # page size not a multiple of 16
    assert lib.kv_append_bf16(bad, A, A, A, A, A, A, 1, A, 1, 1, None, None) == -3
    # tag check
    assert lib.kv_tag_check(A, 4, A, A, 0, A, 1, 16, A, None) == -2
    assert lib.kv_tag_check(A, 4, A, None, 1, A, 1, 16, A, None) == -1
    assert lib.kv_tag_check(A, 4, A, A, 1, A, 0, 16, A, None) == 0
    # fused check + write
    g = lib.kv_tag_check_append_fp8
    assert g(d, A, A, A, A, A, 16, A, 0, A, A, A, 1., 1., None) == 0                           # empty batch
    assert g(d, A, A, A, A, A, 0, A, 1, A, A, A, 1., 1., None) == -2
    assert g(d, A, A, A, A, A, 16, A, 1, A, None, A, 1., 1., None) == -1                       # no expected tags
    assert g(d, A, None, A, A, A, 16, A, 1, A, A, A, 1., 1., None) == -1                       # v_new w/o v_pool
    assert g(d, A, A, A, A, A, 16, A, 1, A, A, A, 1., 0., None) == -7
    wide = _lib.PoolDesc(16, 16, 64, 128, 128)                      # 64 x 128 > 4096 elements per row
    assert lib.kv_tag_check_append_bf16(wide, A, A, A, A, A, 16, A, 1, A, A, A, None) == -3
    # attention
    f = lib.paged_decode_attn_fp8
    assert f(d, A, 8, A, A, A, 16, A, 0, 256, None, 1., 1., 1., 0, None, 0, A, None) == 0     # empty batch
    assert f(d, A, 8, A, A, A, 16, A, 1, 256, None, 1., 1., 1., 0, None, 0, None, None) == -1
    assert f(d, A, 8, A, A, A, 15, A, 1, 256, None, 1., 1., 1., 0, None, 0, A, None) == -2     # 15*16 < 256
    assert f(d, A, 32, A, A, A, 16, A, 1, 256, None, 1., 1., 1., 0, None, 0, A, None) == -3    # group 32 > 16
    assert f(d, A, 8, A, A, A, 16, A, 1, 256, None, 1., -1., 1., 0, None, 0, A, None) == -7
    assert f(d, A, 8, A, A, A, 16, A, 1, 256, None, 1., 1., -1., 0, None, 0, A, None) == -7     # sm_scale < 0
    assert f(d, A, 8, A, A, A, 16, A, 1, 256, None, 1., 1., float("inf"), 0, None, 0, A, None) == -7
    assert f(d, A, 8, A, A, A, 16, A, 1, 256, None, 1., 1., 1., 5, None, 0, A, None) == -2     # 5 splits > 4 tiles
    assert f(d, A, 8, A, A, A, 16, A, 1, 256, None, 1., 1., 1., 2, None, 0, A, None) == -1     # no workspace
    assert f(d, A, 8, A, A, A, 16, A, 1, 256, None, 1., 1., 1., 2, A, 64, A, None) == -4       # too small
    # the allocation-free form: partials beyond its scratch are refused before anything else happens
    na = lib.paged_decode_attn_fp8_noalloc
    d8 = _lib.PoolDesc(16, 16, 8, 128, 128)
    assert 64 * 64 * 4 * 129 * 4 > _lib.NOALLOC_SCRATCH_BYTES >= 64 * 64 * 2 * 129 * 4
    assert na(d8, A, 64, A, A, A, 16, A, 64, 256, None, 1., 1., 1., 4, A, None) == -4
    assert na(d8, A, 64, A, A, A, 16, A, 64, 256, None, 1., 1., 1., 5, A, None) == -2       # 5 splits > 4 tiles
    assert na(d8, A, 64, A, A, A, 16, A, 0, 256, None, 1., 1., 1., 0, A, None) == 0        # empty batch
    assert na(d8, None, 64, A, A, A, 16, A, 1, 256, None, 1., 1., 1., 0, A, None) == -1
    d64 = _lib.PoolDesc(16, 16, 1, 64, 64)
    assert f(d64, A, 8, A, A, A, 16, A, 1, 256, None, 1., 1., 1., 0, None, 0, A, None) == -3
    # one step over a layer stack: every layer checked before anything is enqueued
    step = lib.kv_decode_step_fp8
    sc = (C.c_float * 3)(1., 1., 1.)
    bad = (C.c_float * 3)(1., 0., 1.)                               # layer 1's K scale is invalid
    Ls = _lib.LayerStack(3, A, A, A, A, A, C.cast(sc, C.c_void_p), C.cast(sc, C.c_void_p), A)
    args = (8, A, 16, A, 1, 256, A, A, A, 1., 0, A, 1 << 20, None)
    assert step(d, None, *args) == -1
    assert step(d, _lib.LayerStack(3, A, A, A, A, A, C.cast(sc, C.c_void_p), C.cast(sc, C.c_void_p), A, 2),
                *args) == -7                                        # an option bit the library does not know
    assert step(d, _lib.LayerStack(0, A, A, A, A, A, C.cast(sc, C.c_void_p), C.cast(sc, C.c_void_p), A), *args) == -2
    assert step(d, _lib.LayerStack(3, A, A, A, A, A, None, None, A), *args) == -1     # FP8 needs the scales
    assert step(d, _lib.LayerStack(3, A, A, A, A, A, C.cast(bad, C.c_void_p), C.cast(sc, C.c_void_p), A),
                *args) == -7
    assert step(d, _lib.LayerStack(3, A, A, A, A, A + 8, C.cast(sc, C.c_void_p), C.cast(sc, C.c_void_p), A),
                *args) == -5                                        # layer 0's v_new misaligned
    assert step(d, _lib.LayerStack(3, A, None, A, A, A, C.cast(sc, C.c_void_p), None, A), *args) == -1
    assert step(d, Ls, 8, A, 16, A, 1, 256, A, None, A, 1., 0, A, 1 << 20, None) == -1   # tags w/o expected
    assert step(d, Ls, 32, A, 16, A, 1, 256, A, A, A, 1., 0, A, 1 << 20, None) == -3    # group 32 > 16
    assert step(d, Ls, 8, A, 16, A, 0, 256, A, A, A, 1., 0, A, 1 << 20, None) == 0      # empty batch
    assert lib.kv_decode_step_bf16(d, _lib.LayerStack(2, A, A, A, A, A, None, None, A), 8, A, 15, A, 1, 256,
                                   None, None, None, 1., 0, A, 1 << 20, None) == -2     # 15*16 < 256
    # weight-quantised GEMM
    assert lib.w4_packed_bytes(64, 256) == 64 * 128 and lib.w8_packed_bytes(64, 256) == 64 * 256
    assert lib.w4_packed_bytes(24, 256) == 0 and lib.w8_packed_bytes(64, 384) == 0
    assert lib.wq_scales_count(64, 512) == 64 * 4
    assert lib.w4_quantize_bf16(A, 64, 200, A, A, None) == -2
    assert lib.w4_quantize_bf16(None, 64, 256, A, A, None) == -1
    assert lib.w8_quantize_bf16(A, 64, 256, A, A + 1, None) == -5
    gm = lib.w4a16_gemm
    assert gm(A, 0, A, A, 64, 256, 0, None, 0, A, None) == -2                 # M = 0
    assert gm(A, 65, A, A, 64, 256, 0, None, 0, A, None) == -2                # M > 64
    assert gm(A, 4, A, A, 64, 256, 2, None, 0, A, None) == -2                 # 2 splits > 1 chunk
    assert gm(A, 4, A, A, 64, 512, 2, None, 0, A, None) == -1                 # no workspace
    assert gm(A, 4, A, A, 64, 512, 2, A, 64, A, None) == -4                   # too small
    assert lib.w8a16_gemm(A + 8, 4, A, A, 64, 256, 0, None, 0, A, None) == -5
    # M > 16 keeps a split's scales in LDS: at most 64 groups (8192 inputs) per split
    assert gm(A, 32, A, A, 64, 16384, 1, None, 0, A, None) == -3
    assert 2 <= lib.wgemm_auto_splits(32, 64, 16384)                           # the library's own choice fits
    assert lib.w4_packed_bytes(65536, 65536) == 65536 * 65536 // 2
    assert lib.wgemm_workspace_bytes(4, 64, 512, 1) == 0
    # counters (padded to 256 B), then 1 KiB of partials per split, 16-channel tile (N rounded up to 128) and
    # 16-row tile
    assert lib.wgemm_workspace_bytes(4, 64, 512, 2) == 512 + 2 * 8 * 1024
    assert lib.wgemm_workspace_bytes(1, 8192, 8192, 4) == 65536 + 4 * 512 * 1024
    assert lib.wgemm_workspace_bytes(33, 8192, 8192, 4) == 65536 + 4 * 512 * 3 * 1024
    assert 1 <= lib.wgemm_auto_splits(1, 8192, 8192) <= 32
    # read-rate calibration
    assert lib.kv_read_stream(A, 0, A, None) == 0
    assert lib.kv_read_stream(None, 64, A, None) == -1
    assert lib.kv_read_stream(A, 62, A, None) == -2                           # not a multiple of 4 bytes
    assert lib.kv_read_stream(A + 4, 64, A, None) == -5
    assert lib.kv_read_blocks(A, 16, 2048, A, 0, A, None) == 0
    assert lib.kv_read_blocks(A, 16, 2008, A, 4, A, None) == -2              # block not a multiple of 16 bytes
    assert lib.kv_read_blocks(A, 16, 2048, None, 4, A, None) == -1
    assert lib.kv_read_blocks(A + 8, 16, 2048, A, 4, A, None) == -5
    assert lib.paged_decode_attn_workspace_bytes(64, 64, 128, 1) == 0
    # split counters (one per request and query head, padded to 256 B), then partials and lse
    assert lib.paged_decode_attn_workspace_bytes(64, 64, 128, 2) == 64 * 64 * 128 + 64 * 64 * 2 * 129 * 4
    assert lib.paged_decode_attn_workspace_bytes(1, 8, 512, 4) == 1024 + 8 * 4 * 513 * 4
