"""GPU parity, attention tier: device decode attention vs the fp64 oracle.

Bar: every (request, head) row within max|o - ref| / max|ref| <= 1e-2 (bf16
output), the tolerance the work is held to; aborted or invalid requests give
all-zero rows; physical page placement does not change a single output bit.
"""
import numpy as np
import pytest
import torch

import fp8_paged_kv_append_amd as kv
from kvsynth import workloads as wl
from oracle import attention, codec, paged
from tests.gpu_util import ATTN_TOL, Case, attn_error, dev, host, note

pytestmark = pytest.mark.gpu

DTYPES = ["fp8", "bf16"]


def _check(c, got, flags=None, requests=None):
    ref = c.oracle_attend(flags=flags, requests=requests)
    err = attn_error(got, ref)
    note(f"  {c.w.name} {c.kv_dtype}: max row error {err:.3e}")
    assert err <= ATTN_TOL
    return err


@pytest.mark.parametrize("kv_dtype", DTYPES)
def test_tiny_full(kv_dtype):
    """1 request x 256 tokens, 8 query / 1 KV head, pages in shuffled physical order."""
    note(f"tiny {kv_dtype}")
    c = Case(wl.WORKLOADS["tiny"], kv_dtype)
    c.fill_device()
    for splits in (0, 1, 2, 4):
        got = c.attend(num_splits=splits)
        _check(c, got)


@pytest.mark.parametrize("kv_dtype", DTYPES)
def test_gqa_ragged_lengths(kv_dtype):
    """64/8 heads, page 16, lengths spanning several tiles with ragged tails, pages from a shared pool."""
    w = wl.WORKLOADS["gqa_batch"].with_(batch=6, num_pages=1200, ctx_lo=1, ctx_hi=1500)
    lens = np.array([1, 15, 16, 17, 65, 1500], dtype=np.int32)
    note(f"gqa ragged {kv_dtype}")
    c = Case(w, kv_dtype, lens=lens)
    c.fill_device()
    outs = []
    for splits in (0, 1, 2, 3, 7, 24):
        got = c.attend(num_splits=splits)
        _check(c, got)
        outs.append(codec.f64_from_bf16(got))
    # every split count gives the same answer up to fp32 rounding (within 2 bf16 ulps of the row max)
    for o in outs[1:]:
        assert np.max(attention.row_rel_error(o, outs[0])) <= 2.0 ** -7


@pytest.mark.parametrize("kv_dtype", DTYPES)
def test_values_beyond_fp16_range_with_splits(kv_dtype, monkeypatch):
    """Values up to ~2e7 in magnitude, far beyond fp16's largest finite 65504 (each drawn value times 2^22,
    exact in bf16): the split partials and their merge, inside the launch up to 16 splits and by a merge launch
    beyond, keep every row within the bar.  The FP8 cache's partials are fp16 in units of the e4m3 codes,
    which stay within 448 whatever the scale; partials of the scaled values themselves would overflow."""
    draw_v = wl.request_v

    def big_v(w, r, length):
        f = (draw_v(w, r, length).astype(np.uint32) << 16).view(np.float32) * np.float32(2.0 ** 22)
        return (f.view(np.uint32) >> 16).astype(np.uint16)

    monkeypatch.setattr(wl, "request_v", big_v)
    w = wl.WORKLOADS["gqa_batch"].with_(batch=3, num_pages=400, ctx_lo=1, ctx_hi=2000)
    note(f"values beyond fp16 range {kv_dtype}")
    c = Case(w, kv_dtype, lens=np.array([2000, 1100, 333], dtype=np.int32))
    assert np.abs(codec.f64_from_bf16(c.v)).max() > 65504.0
    c.fill_device()
    for splits in (1, 4, 16, 20):
        got = c.attend(num_splits=splits)
        assert np.abs(codec.f64_from_bf16(got)).max() > 65504.0
        _check(c, got)


@pytest.mark.parametrize("kv_dtype", DTYPES)
def test_wave_tile_counts(kv_dtype):
    """Every count of 64-token tiles per wave from 0 to 7, odd and even (each wave of a block takes every
    fourth tile: its two-tile ring has a tail of two or three and issues nothing past its last tile), in one
    split and in two (a short last chunk)."""
    lens = np.array([64, 128, 320, 512, 576, 768, 1088, 1280, 1344, 1536, 1600, 1283], dtype=np.int32)
    w = wl.WORKLOADS["gqa_batch"].with_(batch=len(lens), num_pages=1000, ctx_lo=64, ctx_hi=1600)
    note(f"wave tile counts {kv_dtype}")
    c = Case(w, kv_dtype, lens=lens)
    c.fill_device()
    for splits in (1, 2):
        _check(c, c.attend(num_splits=splits))


@pytest.mark.parametrize("kv_dtype", DTYPES)
def test_long_context_outliers_page64(kv_dtype):
    """Page size 64, 32 splits with log-sum-exp merge, K outliers x20 past the calibrated range (saturating)."""
    w = wl.WORKLOADS["long"].with_(batch=2, num_pages=300, ctx_lo=8000, ctx_hi=8192)
    note(f"long/outliers {kv_dtype}")
    c = Case(w, kv_dtype)
    if kv_dtype == "fp8":
        # the scale comes from the outlier-free draw, so outliers saturate to +-448
        codes = codec.quantize_e4m3(c.k, c.o_k_scale)
        assert (np.abs(codec.e4m3_decode(codes)) == 448).sum() > 0
    c.fill_device()
    got = c.attend(num_splits=32)
    _check(c, got)
    got1 = c.attend(num_splits=1)
    _check(c, got1)


@pytest.mark.parametrize("kv_dtype", DTYPES)
def test_physical_permutation_is_bit_identical(kv_dtype):
    note(f"permutation {kv_dtype}")
    w = wl.WORKLOADS["tiny"]
    c = Case(w, kv_dtype)
    c.fill_device()
    a = c.attend(num_splits=1)
    # move every physical page elsewhere (device-side copy of the same bytes) and rewrite the table
    perm = np.random.Generator(np.random.PCG64(9)).permutation(w.num_pages)
    blk = w.num_kv_heads * w.page_size * w.head_dim
    kp = c.dkp.view(w.num_pages, blk)
    vp = c.dvp.view(w.num_pages, blk)
    kp2, vp2 = torch.empty_like(kp), torch.empty_like(vp)
    idx = torch.from_numpy(perm).cuda()
    kp2[idx] = kp
    vp2[idx] = vp
    c.dkp, c.dvp = kp2.view(-1), vp2.view(-1)
    c.dpt = dev(np.where(c.pt >= 0, perm[np.maximum(c.pt, 0)], -1).astype(np.int32))
    b = c.attend(num_splits=1)
    assert np.array_equal(a, b)


@pytest.mark.parametrize("kv_dtype", DTYPES)
def test_abort_flags_and_noop_tracker(kv_dtype):
    note(f"abort/no-op {kv_dtype}")
    w = wl.WORKLOADS["gqa_batch"].with_(batch=5, num_pages=600, ctx_lo=100, ctx_hi=900)
    c = Case(w, kv_dtype)
    c.fill_device()
    base = c.attend()
    zero_flags = dev(np.zeros(w.batch, dtype=np.uint32))
    assert np.array_equal(c.attend(flags=zero_flags), base)
    fl = np.array([0, 1, 0, 2, 0], dtype=np.uint32)
    for splits in (0, 1, 3):
        got = c.attend(flags=dev(fl), num_splits=splits)
        for r in range(w.batch):
            if fl[r]:
                assert not got[r].any()
            else:
                assert np.array_equal(got[r], base[r]) or splits != 0
        _check(c, got, flags=fl)


@pytest.mark.parametrize("kv_dtype", DTYPES)
def test_invalid_requests_give_zero_rows(kv_dtype):
    """Tracker off: a bad page id, L <= 0, L beyond the table or beyond max_ctx_len all give zero rows."""
    note(f"invalid requests {kv_dtype}")
    w = wl.WORKLOADS["gqa_batch"].with_(batch=6, num_pages=800, ctx_lo=300, ctx_hi=700)
    c = Case(w, kv_dtype)
    c.fill_device()
    base = c.attend(num_splits=2)
    pt = c.pt.copy()
    pt[1, 3] = w.num_pages + 5
    pt[2, 0] = -4
    lens = c.lens.copy()
    lens[3] = 0
    lens[4] = -9
    c.dpt = dev(pt)
    c.dlens = dev(lens)
    for splits in (1, 2, 5):
        got = c.attend(num_splits=splits)
        for r in (1, 2, 3, 4):
            assert not got[r].any(), (r, splits)
        assert np.max(attention.row_rel_error(codec.f64_from_bf16(got[0]), codec.f64_from_bf16(base[0]))) <= 2.0 ** -7
    # a context longer than max_ctx_len is refused on the device (zero rows), not read past the grid
    c.dpt = dev(c.pt)
    lens = c.lens.copy()
    c.dlens = dev(lens)
    short = int(lens.max()) - 1
    big = int(np.argmax(lens))
    got = c.attend(max_ctx=short, num_splits=1)
    assert not got[big].any()


def test_empty_batch_and_argument_errors():
    note("empty batch / errors")
    desc = kv.pool_desc(4, 16, 1, 128)
    q = torch.zeros((0, 8, 128), dtype=torch.int16, device="cuda")
    out = torch.zeros((0, 8, 128), dtype=torch.int16, device="cuda")
    pools = torch.zeros(4 * 16 * 128, dtype=torch.uint8, device="cuda")
    pt = torch.zeros((0, 1), dtype=torch.int32, device="cuda")
    lens = torch.zeros(0, dtype=torch.int32, device="cuda")
    kv.paged_decode_attn_fp8(desc, q, pools, pools, pt, lens, 16, out, k_scale=1.0, v_scale=1.0)
    q1 = torch.zeros((1, 8, 128), dtype=torch.int16, device="cuda")
    out1 = torch.zeros((1, 8, 128), dtype=torch.int16, device="cuda")
    pt1 = torch.zeros((1, 1), dtype=torch.int32, device="cuda")
    lens1 = torch.ones(1, dtype=torch.int32, device="cuda")
    with pytest.raises(kv.KvFp8Error) as e:      # a page-table row too short for max_ctx_len
        kv.paged_decode_attn_fp8(desc, q1, pools, pools, pt1, lens1, 17, out1, k_scale=1.0, v_scale=1.0)
    assert e.value.status == -2
    with pytest.raises(kv.KvFp8Error) as e:      # bad scale
        kv.paged_decode_attn_fp8(desc, q1, pools, pools, pt1, lens1, 16, out1, k_scale=0.0, v_scale=1.0)
    assert e.value.status == -7
    with pytest.raises(kv.KvFp8Error) as e:      # more splits than 64-token tiles
        kv.paged_decode_attn_fp8(desc, q1, pools, pools, pt1, lens1, 16, out1, k_scale=1.0, v_scale=1.0,
                                 num_splits=2, workspace=torch.zeros(1 << 16, device="cuda"))
    assert e.value.status == -2
    desc17 = kv.pool_desc(4, 16, 1, 64)
    with pytest.raises(kv.KvFp8Error) as e:      # head_dim outside the compiled set
        kv.paged_decode_attn_fp8(desc17, q1, pools, pools, pt1, lens1, 16, out1, k_scale=1.0, v_scale=1.0)
    assert e.value.status == -3


@pytest.mark.parametrize("kv_dtype", DTYPES)
def test_group_sizes(kv_dtype):
    """Query-head groups of 1, 3, 8 and 16 per KV head (padding columns of the MFMA tile)."""
    for hq, hkv in ((2, 2), (6, 2), (8, 1), (32, 2)):
        note(f"group {hq}/{hkv} {kv_dtype}")
        w = wl.Workload("grp", batch=3, num_q_heads=hq, num_kv_heads=hkv, head_dim=128, v_dim=128, page_size=32,
                        num_pages=200, ctx_lo=40, ctx_hi=900, seed=21)
        c = Case(w, kv_dtype)
        c.fill_device()
        _check(c, c.attend())


@pytest.mark.parametrize("kv_dtype", DTYPES)
def test_default_softmax_scale_is_inverse_sqrt_dim(kv_dtype):
    """sm_scale 0 asks the library for 1/sqrt(D): the output equals, bit for bit, the one with the scale
    given explicitly as fl32(1/sqrt(128)), and a different scale changes it."""
    note(f"default softmax scale {kv_dtype}")
    c = Case(wl.WORKLOADS["tiny"], kv_dtype)
    c.fill_device()
    c.sm_scale = float(np.float32(1.0) / np.sqrt(np.float32(128.0)))
    explicit = c.attend(num_splits=2)
    c.sm_scale = 0.0
    default = c.attend(num_splits=2)
    assert np.array_equal(explicit, default)
    c.sm_scale = 0.05
    assert not np.array_equal(c.attend(num_splits=2), default)


@pytest.mark.parametrize("kv_dtype,splits", [("fp8", 16), ("bf16", 16), ("fp8", 62), ("fp8", 3), ("fp8", 0)])
def test_workspace_reuse_never_mixes_launches(kv_dtype, splits):
    """Launches alternating between two query sets share one workspace (partials, and with the library's
    split choice the per-request split counts): every result equals, bit for bit, the one computed with a
    fresh workspace, so no merge reads what another launch left."""
    w = wl.WORKLOADS["gqa_batch"].with_(batch=3, num_pages=1600, ctx_lo=1, ctx_hi=4000)
    lens = np.array([4000, 2500, 300], dtype=np.int32)
    note(f"workspace reuse, alternating queries {kv_dtype} splits={splits}")
    c = Case(w, kv_dtype, lens=lens)
    c.fill_device()
    q1 = c.dq
    q2 = dev(wl.queries(w.with_(seed=w.seed + 101)))
    refs = []
    for q in (q1, q2):
        c.dq = q
        refs.append(c.attend(num_splits=splits))
    assert not np.array_equal(refs[0], refs[1])
    c.dq = q1
    _check(c, refs[0])
    n = splits or kv.paged_decode_attn_auto_splits(w.batch, w.num_kv_heads, c.max_ctx)
    ws = c.workspace(n)
    out = c.out_tensor()
    for i in range(40):
        q = (q1, q2)[i % 2]
        if kv_dtype == "fp8":
            kv.paged_decode_attn_fp8(c.desc, q, c.dkp, c.dvp, c.dpt, c.dlens, c.max_ctx, out, k_scale=c.d_k_scale,
                                     v_scale=c.d_v_scale, sm_scale=c.sm_scale, num_splits=splits, workspace=ws)
        else:
            kv.paged_decode_attn_bf16(c.desc, q, c.dkp, c.dvp, c.dpt, c.dlens, c.max_ctx, out,
                                      sm_scale=c.sm_scale, num_splits=splits, workspace=ws)
        if i % 5 == 4 or i < 4:
            torch.cuda.synchronize()
            assert np.array_equal(host(out, np.uint16), refs[i % 2]), i
