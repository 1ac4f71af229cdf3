"""ctypes loader for libkvfp8.so and the C prototypes of include/kvfp8.h."""
from __future__ import annotations

import ctypes as C
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
# KVFP8_LIB names another build of the library (the host-sanitizer test loads one that way)
LIB_PATH = os.environ.get("KVFP8_LIB") or os.path.join(_HERE, "libkvfp8.so")

KVFP8_OK = 0
STATUS = {0: "KVFP8_OK", -1: "KVFP8_ERR_NULL", -2: "KVFP8_ERR_SHAPE", -3: "KVFP8_ERR_UNSUPPORTED",
          -4: "KVFP8_ERR_WORKSPACE", -5: "KVFP8_ERR_ALIGN", -6: "KVFP8_ERR_HIP", -7: "KVFP8_ERR_VALUE",
          -8: "KVFP8_ERR_NOSPACE"}
KVFP8_ERR_NOSPACE = -8
FLAG_TAG_MISMATCH = 1
FLAG_BAD_PAGE = 2
READ_SINK_WORDS = 2048
NOALLOC_SCRATCH_BYTES = 8 << 20


class PoolDesc(C.Structure):
    _fields_ = [("num_pages", C.c_int32), ("page_size", C.c_int32), ("num_kv_heads", C.c_int32),
                ("head_dim", C.c_int32), ("v_dim", C.c_int32)]


class LayerStack(C.Structure):
    _fields_ = [("num_layers", C.c_int32), ("k_pools", C.c_void_p), ("v_pools", C.c_void_p), ("q", C.c_void_p),
                ("k_new", C.c_void_p), ("v_new", C.c_void_p), ("k_scales", C.c_void_p), ("v_scales", C.c_void_p),
                ("out", C.c_void_p), ("options", C.c_uint32)]
STEP_FUSED_CHECK = 1


_p = C.c_void_p
_i32 = C.c_int32
_i64 = C.c_int64
_f32 = C.c_float
_u32 = C.c_uint32
_sz = C.c_size_t
_desc = C.POINTER(PoolDesc)

PROTOTYPES = {
    "kvfp8_abi_version": (C.c_int, []),
    "kvfp8_status_string": (C.c_char_p, [C.c_int]),
    "kv_absmax_bf16": (C.c_int, [_p, _i64, _p, _p]),
    "kv_scale_from_absmax": (_f32, [_u32]),
    "kv_append_fp8": (C.c_int, [_desc, _p, _p, _p, _p, _p, _p, _i32, _p, _i32, _i32, _p, _f32, _f32, _p]),
    "kv_append_bf16": (C.c_int, [_desc, _p, _p, _p, _p, _p, _p, _i32, _p, _i32, _i32, _p, _p]),
    "kv_tag_check": (C.c_int, [_p, _i32, _p, _p, _i32, _p, _i32, _i32, _p, _p]),
    "kv_tag_check_append_fp8": (C.c_int, [_desc, _p, _p, _p, _p, _p, _i32, _p, _i32, _p, _p, _p, _f32, _f32, _p]),
    "kv_tag_check_append_bf16": (C.c_int, [_desc, _p, _p, _p, _p, _p, _i32, _p, _i32, _p, _p, _p, _p]),
    "kv_decode_step_fp8": (C.c_int, [_desc, C.POINTER(LayerStack), _i32, _p, _i32, _p, _i32, _i32, _p, _p, _p,
                                     _f32, _i32, _p, _sz, _p]),
    "kv_decode_step_bf16": (C.c_int, [_desc, C.POINTER(LayerStack), _i32, _p, _i32, _p, _i32, _i32, _p, _p, _p,
                                      _f32, _i32, _p, _sz, _p]),
    "paged_decode_attn_workspace_bytes": (_sz, [_i32, _i32, _i32, _i32]),
    "paged_decode_attn_auto_splits": (_i32, [_i32, _i32, _i32]),
    "paged_decode_attn_fp8": (C.c_int, [_desc, _p, _i32, _p, _p, _p, _i32, _p, _i32, _i32, _p, _f32, _f32,
                                        _f32, _i32, _p, _sz, _p, _p]),
    "paged_decode_attn_bf16": (C.c_int, [_desc, _p, _i32, _p, _p, _p, _i32, _p, _i32, _i32, _p, _f32, _i32,
                                         _p, _sz, _p, _p]),
    "paged_decode_attn_fp8_noalloc": (C.c_int, [_desc, _p, _i32, _p, _p, _p, _i32, _p, _i32, _i32, _p, _f32, _f32,
                                                _f32, _i32, _p, _p]),
    "paged_decode_attn_latent_auto_splits": (_i32, [_i32, _i32, _i32]),
    "paged_decode_attn_latent_fp8": (C.c_int, [_desc, _p, _i32, _p, _p, _i32, _p, _i32, _i32, _p, _f32, _f32, _i32,
                                               _p, _sz, _p, _p]),
    "paged_decode_attn_latent_bf16": (C.c_int, [_desc, _p, _i32, _p, _p, _i32, _p, _i32, _i32, _p, _f32, _i32, _p,
                                                _sz, _p, _p]),
    "kv_page_alloc_state_bytes": (_sz, [_i32]),
    "kv_page_alloc_init": (C.c_int, [_p, _sz, _i32, _p]),
    "kv_page_alloc_free_count": (_i32, [_p]),
    "kv_page_alloc": (C.c_int, [_p, _i32, _p, _p]),
    "kv_page_free": (C.c_int, [_p, _p, _i32]),
    "kv_page_alloc_tags": (C.c_int, [_p, _p]),
    "w4_packed_bytes": (_sz, [_i32, _i32]),
    "w8_packed_bytes": (_sz, [_i32, _i32]),
    "wq_scales_count": (_sz, [_i32, _i32]),
    "w4_quantize_bf16": (C.c_int, [_p, _i32, _i32, _p, _p, _p]),
    "w8_quantize_bf16": (C.c_int, [_p, _i32, _i32, _p, _p, _p]),
    "wgemm_auto_splits": (_i32, [_i32, _i32, _i32]),
    "wgemm_workspace_bytes": (_sz, [_i32, _i32, _i32, _i32]),
    "w4a16_gemm": (C.c_int, [_p, _i32, _p, _p, _i32, _i32, _i32, _p, _sz, _p, _p]),
    "w8a16_gemm": (C.c_int, [_p, _i32, _p, _p, _i32, _i32, _i32, _p, _sz, _p, _p]),
    "kv_read_stream": (C.c_int, [_p, _sz, _p, _p]),
    "kv_read_blocks": (C.c_int, [_p, _i64, _i64, _p, _i64, _p, _p]),
    "kv_gather_fp8": (C.c_int, [_desc, _p, _p, _p, _p, _i32, _p, _i32, _i32, _p, _p, _p]),
    "kv_gather_bf16": (C.c_int, [_desc, _p, _p, _p, _p, _i32, _p, _i32, _i32, _p, _p, _p]),
}

_lib = None


def load(path: str = LIB_PATH) -> C.CDLL:
    """Load the HIP library once; raise if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m fp8_paged_kv_append_amd.build` "
                           "(the decode path has no fallback)")
    lib = C.CDLL(path)
    for name, (res, args) in PROTOTYPES.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    _lib = lib
    return lib
