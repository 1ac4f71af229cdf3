"""GPU parity of the latent (MLA-style) cache: 576-wide shared vector per token, values = first 512 dims.

Bar as for GQA: every (request, head) row within max|o - ref| / max|ref| <= 1e-2 of the fp64 oracle;
aborted or invalid requests give zero rows; the pool bytes written by the append equal the oracle's.
"""
import numpy as np
import pytest
import torch

import fp8_paged_kv_append_amd as kv
from kvsynth import workloads as wl
from oracle import attention, codec
from tests.gpu_util import ATTN_TOL, Case, attn_error, dev, host, note

pytestmark = pytest.mark.gpu


def _latent_attend(c, flags=None, num_splits=0, max_ctx=None):
    w = c.w
    mc = c.max_ctx if max_ctx is None else max_ctx
    out = c.out_tensor()
    splits = num_splits or kv.paged_decode_attn_latent_auto_splits(w.batch, w.num_q_heads, mc)
    ws = c.workspace(splits)
    if c.kv_dtype == "fp8":
        kv.paged_decode_attn_latent_fp8(c.desc, c.dq, c.dkp, c.dpt, c.dlens, mc, out, flags, scale=c.d_k_scale,
                                        sm_scale=c.sm_scale, num_splits=num_splits, workspace=ws)
    else:
        kv.paged_decode_attn_latent_bf16(c.desc, c.dq, c.dkp, c.dpt, c.dlens, mc, out, flags,
                                         sm_scale=c.sm_scale, num_splits=num_splits, workspace=ws)
    torch.cuda.synchronize()
    return host(out, np.uint16)


def _check(c, got, flags=None):
    ref = c.oracle_attend(flags=flags)
    err = attn_error(got, ref)
    note(f"  latent {c.kv_dtype} Hq={c.w.num_q_heads}: max row error {err:.3e}")
    assert err <= ATTN_TOL
    return err


@pytest.mark.parametrize("kv_dtype", ["fp8", "bf16"])
@pytest.mark.parametrize("hq", [128, 16, 80])
def test_latent_ragged(kv_dtype, hq):
    w = wl.WORKLOADS["latent"].with_(batch=5, num_q_heads=hq, num_pages=120, ctx_lo=1, ctx_hi=700)
    lens = np.array([1, 31, 33, 64, 700], dtype=np.int32)
    note(f"latent ragged {kv_dtype} Hq={hq}")
    c = Case(w, kv_dtype, lens=lens)
    c.fill_device()
    torch.cuda.synchronize()
    et = np.uint8 if kv_dtype == "fp8" else np.uint16
    assert np.array_equal(c.device_k(), c.okp)
    outs = []
    for splits in (0, 1, 2, 5):
        got = _latent_attend(c, num_splits=splits)
        _check(c, got)
        outs.append(codec.f64_from_bf16(got))
    for o in outs[1:]:
        assert np.max(attention.row_rel_error(o, outs[0])) <= 2.0 ** -7


@pytest.mark.parametrize("kv_dtype", ["fp8", "bf16"])
def test_latent_short_last_splits(kv_dtype):
    """Two splits of 35 tiles (1,120 tokens: the 128-head kernel, not the wave-pair one), the requests' second
    split holding 1 to 6 tiles and the first a whole one: the tile-copy ring copies nothing past a split's
    last tile and waits only for copies it issued.  Then the library's split count (the wave-pair kernel for
    FP8, splits of at most 1,024 tokens) over the same requests."""
    lens = np.array([1121, 1152, 1184, 1216, 1248, 1280, 1312, 2240], dtype=np.int32)
    w = wl.WORKLOADS["latent"].with_(batch=len(lens), num_pages=250, ctx_lo=1121, ctx_hi=2240)
    note(f"latent short last splits {kv_dtype}")
    c = Case(w, kv_dtype, lens=lens)
    c.fill_device()
    outs = []
    for splits in (2, 0):
        got = _latent_attend(c, num_splits=splits)
        _check(c, got)
        outs.append(codec.f64_from_bf16(got))
    assert np.max(attention.row_rel_error(outs[1], outs[0])) <= 2.0 ** -7


@pytest.mark.parametrize("kv_dtype", ["fp8", "bf16"])
def test_latent_page16_and_abort(kv_dtype):
    w = wl.WORKLOADS["latent"].with_(batch=4, num_q_heads=64, page_size=16, num_pages=200, ctx_lo=100, ctx_hi=800)
    note(f"latent page16/abort {kv_dtype}")
    c = Case(w, kv_dtype)
    c.fill_device()
    base = _latent_attend(c)
    _check(c, base)
    fl = np.array([0, 2, 0, 1], dtype=np.uint32)
    got = _latent_attend(c, flags=dev(fl), num_splits=3)
    assert not got[1].any() and not got[3].any()
    _check(c, got, flags=fl)
    # a bad page id with the tracker off zeroes that request only
    pt = c.pt.copy()
    pt[2, 1] = w.num_pages + 3
    c.dpt = dev(pt)
    got = _latent_attend(c, num_splits=2)
    assert not got[2].any() and got[0].any()


@pytest.mark.parametrize("batch,kv_dtype", [(64, "fp8"), (64, "bf16"), (16, "fp8"), (16, "bf16")])
def test_latent_full_size_sampled(batch, kv_dtype):
    """B requests x 4096 tokens, 128 heads, page 64, 8192-page pool, in the library's default split: at
    64 requests the 128-head kernel, at 16 the FP8 cache's wave-pair kernel (8 splits of 512 tokens)."""
    w = wl.WORKLOADS["latent"].with_(batch=batch)
    note(f"latent full size B={batch} {kv_dtype}")
    c = Case(w, kv_dtype, oracle_fill=False)
    assert c.d_k_scale == float(c.o_k_scale)
    c.fill_device()
    got = _latent_attend(c)
    for r in sorted({0, batch // 2 - 1, batch - 1}):
        ref = c.oracle_request(r)
        err = float(np.max(attention.row_rel_error(codec.f64_from_bf16(got[r]), ref)))
        note(f"  request {r}: row error {err:.3e}")
        assert err <= ATTN_TOL


@pytest.mark.parametrize("kv_dtype", ["fp8", "bf16"])
def test_latent_query_dynamic_range(kv_dtype):
    """Queries whose heads span 1e-3..1e3 in scale, with elements far below their head's max (beyond the
    2^9 range that two e4m3 terms hold exactly in the FP8 path) and one all-zero head: rows still within
    tolerance of the oracle, and the zero head gives the plain mean of the values."""
    w = wl.WORKLOADS["latent"].with_(batch=3, num_q_heads=32, num_pages=60, ctx_lo=40, ctx_hi=300)
    note(f"latent q dynamic range {kv_dtype}")
    c = Case(w, kv_dtype)
    c.fill_device()
    rng = np.random.default_rng(11)
    qf = wl.bf16_bits_to_f32(c.q).astype(np.float32)                      # [B][Hq][576]
    head_scale = (10.0 ** rng.uniform(-3, 3, size=(1, w.num_q_heads, 1))).astype(np.float32)
    tiny = rng.random(qf.shape) < 0.05                                     # 5% of elements ~1e-5 of the rest
    qf = np.where(tiny, qf * 1e-5, qf) * head_scale
    qf[:, 7, :] = 0.0
    c.q = wl.to_bf16_bits(qf)
    c.dq = dev(c.q)
    got = _latent_attend(c)
    _check(c, got)
    # head 7 has zero scores: uniform weights, the output is the mean of the dequantised value rows
    for r in range(w.batch):
        ref = c.oracle_request(r)[7]
        assert np.max(attention.row_rel_error(codec.f64_from_bf16(got[r, 7])[None], ref[None])) <= ATTN_TOL


@pytest.mark.parametrize("kv_dtype", ["fp8", "bf16"])
def test_latent_128_head_kernel_many_splits(kv_dtype):
    """6 and 12 splits of more than 1,024 tokens each, so the 128-head kernel runs (not the wave-pair one)
    and the merge takes groups of 8 and 16 splits: fp16 partials for the FP8 cache, fp32 for BF16.  The
    second request is shorter, so its last splits are empty.  Rows within tolerance of the oracle, and the
    split counts agree with each other."""
    w = wl.WORKLOADS["latent"].with_(batch=2, num_pages=400, ctx_lo=9000, ctx_hi=14000)
    lens = np.array([14000, 9000], dtype=np.int32)
    note(f"latent 128-head kernel, 6 and 12 splits {kv_dtype}")
    c = Case(w, kv_dtype, lens=lens)
    c.fill_device()
    outs = []
    for splits in (6, 12):
        got = _latent_attend(c, num_splits=splits)
        _check(c, got)
        outs.append(codec.f64_from_bf16(got))
    assert np.max(attention.row_rel_error(outs[1], outs[0])) <= 2.0 ** -7


@pytest.mark.parametrize("kv_dtype", ["fp8", "bf16"])
def test_latent_one_request_many_splits(kv_dtype):
    """One request of 4096 tokens over 128 heads at the library's split count (32: the wave-pair kernel with
    fp16 partials for the FP8 cache, the 128-head kernel with fp32 partials for BF16) and at 20: the merge
    takes all of a row's splits in one group of 32.  Rows within tolerance of the oracle, and the two split
    counts agree."""
    w = wl.WORKLOADS["latent"].with_(batch=1, num_pages=80, ctx_lo=4096, ctx_hi=4096)
    note(f"latent one request, 32 and 20 splits {kv_dtype}")
    c = Case(w, kv_dtype)
    c.fill_device()
    assert kv.paged_decode_attn_latent_auto_splits(1, w.num_q_heads, c.max_ctx) == 32
    outs = []
    for splits in (0, 20):
        got = _latent_attend(c, num_splits=splits)
        _check(c, got)
        outs.append(codec.f64_from_bf16(got))
    assert np.max(attention.row_rel_error(outs[1], outs[0])) <= 2.0 ** -7
