"""GPU parity of a whole decode step (tag check -> append -> attention), small and at full size."""
import numpy as np
import pytest
import torch

import fp8_paged_kv_append_amd as kv
from kvsynth import workloads as wl
from oracle import attention, codec, paged, step
from tests.gpu_util import ATTN_TOL, Case, attn_error, dev, host, note

pytestmark = pytest.mark.gpu


def _device_step(c, k_new, v_new, req, pos, tracker=True, num_splits=0, one_launch=False, fused=False):
    """The step through decode_step: three launches with explicit token positions, or with one_launch
    (positions implicit at L - 1) kv_decode_step_* over one layer: the check + write launch, then the
    attention; with fused, the check inside the attention launch (one launch for the GQA cache)."""
    w = c.w
    if one_launch:
        assert np.array_equal(pos, c.lens[req] - 1)
        req = pos = None
    out = c.out_tensor()
    flags = torch.full((w.batch,), -1, dtype=torch.int32, device="cuda") if tracker else None
    splits = num_splits or kv.paged_decode_attn_auto_splits(w.batch, w.num_kv_heads, c.max_ctx)
    kv.decode_step(c.desc, c.kv_dtype, c.dkp, c.dvp, c.dpt, c.dlens, c.max_ctx, c.dq, dev(k_new),
                   None if v_new is None else dev(v_new), None if req is None else dev(req),
                   None if pos is None else dev(pos), out,
                   page_tags=c.dtags if tracker else None, expected_tags=c.dexp if tracker else None,
                   abort_flags=flags, k_scale=c.d_k_scale, v_scale=c.d_v_scale, sm_scale=c.sm_scale,
                   num_splits=num_splits, workspace=c.workspace(splits), fused_check=fused)
    torch.cuda.synchronize()
    return (None if flags is None else host(flags, np.uint32)), host(out, np.uint16)


@pytest.mark.parametrize("one_launch,fused", [(False, False), (True, False), (True, True)])
@pytest.mark.parametrize("kv_dtype", ["fp8", "bf16"])
def test_step_with_stale_request(kv_dtype, one_launch, fused):
    """16 requests, one with a stale expected tag: its flag is set, its page is not written, its rows are 0
    (three launches; the library's step: check + write launch, then attention; or, fused, one launch that
    checks, writes and attends)."""
    w = wl.WORKLOADS["sweep_b16"].with_(num_pages=3000, ctx_lo=700, ctx_hi=700)
    note(f"step stale {kv_dtype} one_launch={one_launch} fused={fused}")
    c = Case(w, kv_dtype)
    c.fill_device()
    k_new, v_new, req, pos = c.step_inputs()
    # the new rows differ from what is stored, so a skipped write is visible
    k_new = k_new ^ np.uint16(0x0040)
    st = dict(dtype=kv_dtype, k_pool=c.okp, v_pool=c.ovp, page_table=c.pt, ctx_lens=c.lens, page_tags=c.tags,
              expected_tags=c.exp, num_kv_heads=w.num_kv_heads, page_size=w.page_size, head_dim=w.head_dim,
              v_dim=w.v_dim, k_scale=c.o_k_scale, v_scale=c.o_v_scale, sm_scale=c.sm_scale, latent=False)
    o_flags, o_out = step.decode_step(st, c.q, k_new, v_new, req, pos)
    g_flags, g_out = _device_step(c, k_new, v_new, req, pos, one_launch=one_launch, fused=fused)
    assert np.array_equal(g_flags, o_flags)
    assert np.flatnonzero(g_flags).tolist() == c.stale.tolist()
    et = np.uint8 if kv_dtype == "fp8" else np.uint16
    assert c.pools_match()
    err = attn_error(g_out, o_out)
    note(f"  step error {err:.3e}")
    assert err <= ATTN_TOL
    for r in c.stale:
        assert not g_out[r].any()
    # the no-op tracker: no check, every request attended
    g2_flags, g2_out = _device_step(c, k_new, v_new, req, pos, tracker=False, one_launch=one_launch, fused=fused)
    assert g2_flags is None and all(g2_out[r].any() for r in range(w.batch))


@pytest.mark.parametrize("b,kv_dtype,fused", [(64, "fp8", False), (64, "bf16", False), (64, "fp8", True),
                                              (1, "fp8", False), (8, "fp8", False), (16, "fp8", False),
                                              (32, "fp8", False), (1, "bf16", False), (8, "bf16", False),
                                              (16, "bf16", False), (32, "bf16", False)])
def test_full_size_sweep_sampled(b, kv_dtype, fused):
    """The concurrency workload at full size, B requests x 8192 tokens (64/8 heads, page 16, 40k-page pool,
    1 % stale), in the bench's launch configuration (the library's split choice: 16/4/2/1/1 splits at
    B = 1/8/16/32/64; the check + write launch, then attention, or fused in one launch): all flags
    bit-exact, scales bit-exact, sampled requests' first and last pages byte-exact and their attention
    rows within tolerance of the oracle."""
    w = wl.WORKLOADS[f"sweep_b{b}"]
    note(f"full {b}x8192 {kv_dtype} fused={fused}: generating")
    c = Case(w, kv_dtype, oracle_fill=False)
    assert c.d_k_scale == float(c.o_k_scale) and c.d_v_scale == float(c.o_v_scale)
    note(f"  filling (splits {kv.paged_decode_attn_auto_splits(w.batch, w.num_kv_heads, c.max_ctx)})")
    c.fill_device()
    k_new, v_new, req, pos = c.step_inputs()
    g_flags, g_out = _device_step(c, k_new, v_new, req, pos, one_launch=True, fused=fused)
    o_flags = paged.tag_check(c.tags, c.pt, c.exp, c.lens, w.page_size)
    assert np.array_equal(g_flags, o_flags) and (o_flags.sum() > 0) == (b >= 8)
    sample = sorted(set([r for r in (0, 17, b - 1) if r < b] + c.stale.tolist()))
    et = np.uint8 if kv_dtype == "fp8" else np.uint16
    g = kv.kv_gather_fp8 if kv_dtype == "fp8" else kv.kv_gather_bf16
    S = w.page_size
    for r in sample:
        note(f"  request {r}")
        if g_flags[r]:
            assert not g_out[r].any()
            continue
        a, e = int(c.off[r]), int(c.off[r + 1])
        idx = np.r_[a:a + S, e - S:e]                         # first and last page (the step's token)
        didx = dev(idx.astype(np.int64))
        ko = torch.empty((idx.size, w.num_kv_heads, w.head_dim), dtype=c.dkp.dtype, device="cuda")
        vo = torch.empty((idx.size, w.num_kv_heads, w.v_dim), dtype=c.dkp.dtype, device="cuda")
        g(c.desc, c.dkp, c.dvp, c.dreq[didx].contiguous(), c.dpos[didx].contiguous(), c.dpt, ko, vo)
        torch.cuda.synchronize()
        if kv_dtype == "fp8":
            assert np.array_equal(host(ko, et), codec.quantize_e4m3(c.k[idx], c.o_k_scale))
            assert np.array_equal(host(vo, et), codec.quantize_e4m3(c.v[idx], c.o_v_scale))
        else:
            assert np.array_equal(host(ko, et), c.k[idx]) and np.array_equal(host(vo, et), c.v[idx])
        ref = c.oracle_request(r)
        err = float(np.max(attention.row_rel_error(codec.f64_from_bf16(g_out[r]), ref)))
        note(f"    row error {err:.3e}")
        assert err <= ATTN_TOL


def _fused_case(kv_dtype, latent):
    """A batch with planted faults for the fused check + write: stale tags, a page-table hole inside a used
    range, an empty request; the new rows differ from what is stored so a skipped write is visible."""
    if latent:
        w = wl.WORKLOADS["latent"].with_(batch=9, num_q_heads=16, num_pages=400, ctx_lo=1, ctx_hi=600)
    else:
        w = wl.WORKLOADS["sweep_b16"].with_(num_pages=3000, ctx_lo=1, ctx_hi=700)
    lens = wl.ctx_lens(w)
    lens[3] = 0
    c = Case(w, kv_dtype, lens=lens, stale=[1, 6])
    c.fill_device()
    hole = 5                                             # its middle used entry becomes -1 after the fill
    c.pt[hole, (int(c.lens[hole]) - 1) // w.page_size // 2] = -1
    c.dpt = dev(c.pt)
    k_new, v_new, req, pos = c.step_inputs()
    k_new = k_new ^ np.uint16(0x0040)
    return c, k_new, v_new, req, pos, hole


@pytest.mark.parametrize("latent,two_launch", [(False, False), (False, True), (True, True)])
@pytest.mark.parametrize("kv_dtype", ["fp8", "bf16"])
def test_fused_check_append_step(kv_dtype, latent, two_launch):
    """One token per request at L - 1, the check and the write fused: for the GQA cache as one launch
    (decode_step with implicit tokens: every attention block checks its request's pages, the block
    holding L - 1 writes the token) or as kv_tag_check_append_* then the attention; the latent cache
    takes the latter.  Flags and both pools bit-exact to the oracle's check -> append, attention rows
    within tolerance, faulty requests zero."""
    note(f"fused check+append {kv_dtype} latent={latent} two_launch={two_launch}")
    c, k_new, v_new, req, pos, hole = _fused_case(kv_dtype, latent)
    w = c.w
    st = dict(dtype=kv_dtype, k_pool=c.okp, v_pool=c.ovp, page_table=c.pt, ctx_lens=c.lens, page_tags=c.tags,
              expected_tags=c.exp, num_kv_heads=w.num_kv_heads, page_size=w.page_size, head_dim=w.head_dim,
              v_dim=w.v_dim, k_scale=c.o_k_scale, v_scale=c.o_v_scale, sm_scale=c.sm_scale, latent=latent)
    o_flags, o_out = step.decode_step(st, c.q, k_new, v_new, req, pos)
    assert o_flags[hole] == paged.FLAG_BAD_PAGE and o_flags[1] and o_flags[6] and not o_flags[3]
    flags = torch.full((w.batch,), -1, dtype=torch.int32, device="cuda")
    out = c.out_tensor()
    if latent:
        # the step's write through the fused launch, then the latent attention
        f = kv.kv_tag_check_append_fp8 if kv_dtype == "fp8" else kv.kv_tag_check_append_bf16
        kw = dict(k_scale=c.d_k_scale, v_scale=c.d_v_scale) if kv_dtype == "fp8" else {}
        f(c.desc, c.dkp, None, dev(k_new), None, c.dpt, c.dlens, c.dtags, c.dexp, flags, **kw)
        splits = kv.paged_decode_attn_latent_auto_splits(w.batch, w.num_q_heads, c.max_ctx)
        ws = c.workspace(splits)
        if kv_dtype == "fp8":
            kv.paged_decode_attn_latent_fp8(c.desc, c.dq, c.dkp, c.dpt, c.dlens, c.max_ctx, out, flags,
                                            scale=c.d_k_scale, sm_scale=c.sm_scale, workspace=ws)
        else:
            kv.paged_decode_attn_latent_bf16(c.desc, c.dq, c.dkp, c.dpt, c.dlens, c.max_ctx, out, flags,
                                             sm_scale=c.sm_scale, workspace=ws)
    elif two_launch:
        splits = kv.paged_decode_attn_auto_splits(w.batch, w.num_kv_heads, c.max_ctx)
        ws = c.workspace(splits)
        if kv_dtype == "fp8":
            kv.kv_tag_check_append_fp8(c.desc, c.dkp, c.dvp, dev(k_new), dev(v_new), c.dpt, c.dlens, c.dtags, c.dexp,
                                       flags, k_scale=c.d_k_scale, v_scale=c.d_v_scale)
            kv.paged_decode_attn_fp8(c.desc, c.dq, c.dkp, c.dvp, c.dpt, c.dlens, c.max_ctx, out, flags,
                                     k_scale=c.d_k_scale, v_scale=c.d_v_scale, sm_scale=c.sm_scale, workspace=ws)
        else:
            kv.kv_tag_check_append_bf16(c.desc, c.dkp, c.dvp, dev(k_new), dev(v_new), c.dpt, c.dlens, c.dtags,
                                        c.dexp, flags)
            kv.paged_decode_attn_bf16(c.desc, c.dq, c.dkp, c.dvp, c.dpt, c.dlens, c.max_ctx, out, flags,
                                      sm_scale=c.sm_scale, workspace=ws)
    else:
        splits = kv.paged_decode_attn_auto_splits(w.batch, w.num_kv_heads, c.max_ctx)
        kv.decode_step(c.desc, kv_dtype, c.dkp, c.dvp, c.dpt, c.dlens, c.max_ctx, c.dq, dev(k_new), dev(v_new),
                       None, None, out, page_tags=c.dtags, expected_tags=c.dexp, abort_flags=flags,
                       k_scale=c.d_k_scale, v_scale=c.d_v_scale, sm_scale=c.sm_scale, workspace=c.workspace(splits))
    torch.cuda.synchronize()
    g_flags, g_out = host(flags, np.uint32), host(out, np.uint16)
    assert np.array_equal(g_flags, o_flags)
    et = np.uint8 if kv_dtype == "fp8" else np.uint16
    assert np.array_equal(c.device_k(), c.okp)
    if not latent:
        assert np.array_equal(c.device_v(), c.ovp)
    err = attn_error(g_out, o_out)
    note(f"  step error {err:.3e}")
    assert err <= ATTN_TOL
    for r in np.flatnonzero(o_flags).tolist() + [3]:
        assert not g_out[r].any()


@pytest.mark.parametrize("kv_dtype", ["fp8", "bf16"])
def test_fused_matches_separate_launches(kv_dtype):
    """The fused launch and kv_tag_check + kv_append_* on two copies of one device cache: identical bytes."""
    note(f"fused vs separate {kv_dtype}")
    c, k_new, v_new, req, pos, _ = _fused_case(kv_dtype, False)
    w = c.w
    kp2, vp2 = c.dkp.clone(), c.dvp.clone()
    f1 = torch.zeros(w.batch, dtype=torch.int32, device="cuda")
    f2 = torch.full((w.batch,), 7, dtype=torch.int32, device="cuda")
    dk, dv = dev(k_new), dev(v_new)
    kv.kv_tag_check(c.dtags, c.dpt, c.dexp, c.dlens, w.page_size, f1)
    if kv_dtype == "fp8":
        kv.kv_append_fp8(c.desc, c.dkp, c.dvp, dk, dv, dev(req), dev(pos), c.dpt, f1, k_scale=c.d_k_scale,
                         v_scale=c.d_v_scale)
        kv.kv_tag_check_append_fp8(c.desc, kp2, vp2, dk, dv, c.dpt, c.dlens, c.dtags, c.dexp, f2,
                                   k_scale=c.d_k_scale, v_scale=c.d_v_scale)
    else:
        kv.kv_append_bf16(c.desc, c.dkp, c.dvp, dk, dv, dev(req), dev(pos), c.dpt, f1)
        kv.kv_tag_check_append_bf16(c.desc, kp2, vp2, dk, dv, c.dpt, c.dlens, c.dtags, c.dexp, f2)
    torch.cuda.synchronize()
    assert torch.equal(f1, f2)
    assert torch.equal(c.dkp, kp2) and torch.equal(c.dvp, vp2)


@pytest.mark.parametrize("fused", [False, True])
@pytest.mark.parametrize("latent,num_splits", [(False, 0), (False, 3), (True, 0), (True, 3)])
@pytest.mark.parametrize("kv_dtype", ["fp8", "bf16"])
def test_step_length_beyond_max_ctx(kv_dtype, latent, num_splits, fused):
    """A request longer than max_ctx_len is a caller error.  In the library's step (separate check + write
    launch, or the check fused into the attention launch) its pages are still checked (its flag is the tag
    check's), its rows are zero and its token is not written, for the GQA and the latent cache alike; a
    stale request is aborted as usual and the others match the oracle, pools element for element."""
    note(f"step, L > max_ctx {kv_dtype} latent={latent} splits={num_splits} fused={fused}")
    if latent:
        w = wl.WORKLOADS["latent"].with_(batch=4, num_q_heads=16, num_pages=100, ctx_lo=300, ctx_hi=600)
    else:
        w = wl.WORKLOADS["sweep_b16"].with_(batch=4, num_pages=3000, ctx_lo=300, ctx_hi=600)
    lens = np.array([300, 500, 400, 350], dtype=np.int32)
    max_ctx = 450                                          # request 1 exceeds it
    c = Case(w, kv_dtype, lens=lens, stale=[3])
    c.fill_device()
    k_new, v_new, req, pos = c.step_inputs()
    k_new = k_new ^ np.uint16(0x0040)                      # a write shows
    v_new = None if latent else v_new ^ np.uint16(0x0040)
    o_flags = paged.tag_check(c.tags, c.pt, c.exp, c.lens, w.page_size)
    assert o_flags.tolist() == [0, 0, 0, paged.FLAG_TAG_MISMATCH]
    skip = o_flags.copy()
    skip[1] = 1                                            # the caller error: not written, zero rows
    if kv_dtype == "fp8":
        paged.append_fp8(c.okp, c.ovp, k_new, v_new, req, pos, c.pt, c.o_k_scale, c.o_v_scale, skip)
    else:
        paged.append(c.okp, c.ovp, k_new, v_new, req, pos, c.pt, skip)
    ref = c.oracle_attend(flags=skip, requests=[0, 2])
    flags = torch.full((w.batch,), -1, dtype=torch.int32, device="cuda")
    out = c.out_tensor()
    if latent:
        splits = num_splits or kv.paged_decode_attn_latent_auto_splits(w.batch, w.num_q_heads, max_ctx)
    else:
        splits = num_splits or kv.paged_decode_attn_auto_splits(w.batch, w.num_kv_heads, max_ctx)
    kv.decode_step(c.desc, kv_dtype, c.dkp, c.dvp, c.dpt, c.dlens, max_ctx, c.dq, dev(k_new),
                   None if latent else dev(v_new), None, None, out, page_tags=c.dtags, expected_tags=c.dexp,
                   abort_flags=flags, k_scale=c.d_k_scale, v_scale=c.d_v_scale, sm_scale=c.sm_scale,
                   num_splits=num_splits, workspace=c.workspace(splits), fused_check=fused)
    torch.cuda.synchronize()
    assert np.array_equal(host(flags, np.uint32), o_flags)
    assert c.pools_match()
    g_out = host(out, np.uint16)
    assert not g_out[1].any() and not g_out[3].any()
    err = attn_error(g_out, ref)
    note(f"  step error {err:.3e}")
    assert err <= ATTN_TOL


@pytest.mark.parametrize("name,kv_dtype,calib_outliers", [("gqa_batch", "fp8", False), ("gqa_batch", "bf16", False),
                                                           ("long", "fp8", False), ("long", "bf16", False),
                                                           ("long", "fp8", True)])
def test_full_size_other_gqa_workloads_sampled(kv_dtype, name, calib_outliers):
    """The ragged batch (32 requests of 1024-8192 tokens, 40k-page pool, the library's split choice) and the
    long context (4 x 131072 tokens, page 64, 32 splits, K outliers x20 against the outlier-free scale) at
    full size, in the bench's launch configuration (one launch, plus the merge when split): flags bit-exact,
    sampled requests' pages byte-exact (their first and last pages, where the step's token sits) and their
    attention rows within tolerance of the oracle.  The long context runs both readings of its outliers: the
    K scale from the outlier-free draw, so the outliers saturate at +-448 * scale, and (calib_outliers) the
    K scale over K as drawn, outliers included, so nothing saturates and the other values sit closer to
    the subnormals."""
    w = wl.WORKLOADS[name]
    note(f"full {name} {kv_dtype} calib_outliers={calib_outliers}: generating")
    c = Case(w, kv_dtype, oracle_fill=False, calib_outliers=calib_outliers)
    assert c.d_k_scale == float(c.o_k_scale) and c.d_v_scale == float(c.o_v_scale)
    note("  filling")
    c.fill_device()
    k_new, v_new, req, pos = c.step_inputs()
    if kv_dtype == "fp8" and w.outlier_frac:
        kmax = float(codec.f32_from_bf16(np.array([np.max(c.k & np.uint16(0x7FFF))], dtype=np.uint16))[0])
        # a value saturates when it lies above 464, the midpoint between 448 and the next e4m3 step (480)
        # of the unsaturated format: only then does rounding leave 448 behind
        saturates = kmax / c.d_k_scale > 464.0
        note(f"  K scale {c.d_k_scale:.6g}: outliers saturate: {saturates}")
        assert saturates != calib_outliers
    g_flags, g_out = _device_step(c, k_new, v_new, req, pos, num_splits=w.num_splits, one_launch=True)
    o_flags = paged.tag_check(c.tags, c.pt, c.exp, c.lens, w.page_size)
    assert np.array_equal(g_flags, o_flags)
    if name == "gqa_batch":   # the longest and the shortest request, and one between
        order = np.argsort(c.lens, kind="stable")
        sample = sorted({int(order[0]), int(order[-1]), int(order[len(order) // 2])})
    else:
        sample = [w.batch - 1]                                   # ~1 min of oracle work each
    et = np.uint8 if kv_dtype == "fp8" else np.uint16
    g = kv.kv_gather_fp8 if kv_dtype == "fp8" else kv.kv_gather_bf16
    for r in sample:
        note(f"  request {r} (L = {int(c.lens[r])})")
        assert not g_flags[r]
        a, b = int(c.off[r]), int(c.off[r + 1])
        S = w.page_size
        idx = np.r_[a:min(b, a + S), max(a, b - S):b]          # first and last page of the request
        didx = dev(idx.astype(np.int64))
        ko = torch.empty((idx.size, w.num_kv_heads, w.head_dim), dtype=c.dkp.dtype, device="cuda")
        vo = torch.empty((idx.size, w.num_kv_heads, w.v_dim), dtype=c.dkp.dtype, device="cuda")
        g(c.desc, c.dkp, c.dvp, c.dreq[didx].contiguous(), c.dpos[didx].contiguous(), c.dpt, ko, vo)
        torch.cuda.synchronize()
        if kv_dtype == "fp8":
            assert np.array_equal(host(ko, et), codec.quantize_e4m3(c.k[idx], c.o_k_scale))
            assert np.array_equal(host(vo, et), codec.quantize_e4m3(c.v[idx], c.o_v_scale))
        else:
            assert np.array_equal(host(ko, et), c.k[idx]) and np.array_equal(host(vo, et), c.v[idx])
        ref = c.oracle_request(r)
        err = float(np.max(attention.row_rel_error(codec.f64_from_bf16(g_out[r]), ref)))
        note(f"    row error {err:.3e}")
        assert err <= ATTN_TOL


@pytest.mark.parametrize("fused", [False, True])
@pytest.mark.parametrize("num_splits", [1, 3])
@pytest.mark.parametrize("kv_dtype", ["fp8", "bf16"])
def test_long_rows_page_id_batches_and_windows(kv_dtype, num_splits, fused):
    """Contexts of 40,000, 17,000 and 33,000 tokens at page 16 (2,500, 1,063 and 2,063 pages): blocks stage
    page ids in batches of 1,024 entries, so these rows take a second (and third) batch, and at one split the
    40,000- and 33,000-token chunks span more than one 2,047-page id window.  Request 2 has a stale tag past
    its first 1,024 entries.  Checked against the oracle: the one-launch step with the check in the launch
    (flags, pools and rows; the check as its own launch, or fused: in the attention launch, where the
    blocks stage their ids in several batches), the same step with no tracker, and plain attention reading
    the flags."""
    w = wl.WORKLOADS["sweep_b16"].with_(batch=3, num_q_heads=8, num_kv_heads=1, num_pages=6000, ctx_lo=1, ctx_hi=1,
                                        stale=False)
    lens = np.array([40000, 17000, 33000], dtype=np.int32)
    note(f"long rows {kv_dtype} splits={num_splits} fused={fused}")
    c = Case(w, kv_dtype, lens=lens, stale=[])
    c.fill_device()
    c.exp[2, 1500] = c.exp[2, 1500] - np.uint32(1)       # stale, in the second batch of 1,024 entries
    c.dexp = dev(c.exp)
    k_new, v_new, req, pos = c.step_inputs()
    k_new = k_new ^ np.uint16(0x0040)                     # a skipped write stays visible
    st = dict(dtype=kv_dtype, k_pool=c.okp, v_pool=c.ovp, page_table=c.pt, ctx_lens=c.lens, page_tags=c.tags,
              expected_tags=c.exp, num_kv_heads=w.num_kv_heads, page_size=w.page_size, head_dim=w.head_dim,
              v_dim=w.v_dim, k_scale=c.o_k_scale, v_scale=c.o_v_scale, sm_scale=c.sm_scale, latent=False)
    o_flags, o_out = step.decode_step(st, c.q, k_new, v_new, req, pos)
    assert o_flags.tolist() == [0, 0, 1]
    g_flags, g_out = _device_step(c, k_new, v_new, req, pos, num_splits=num_splits, one_launch=True, fused=fused)
    assert np.array_equal(g_flags, o_flags)
    assert c.pools_match()
    assert not g_out[2].any()
    err = attn_error(g_out, {r: o_out[r] for r in (0, 1)})
    note(f"  tracker on: error {err:.3e}")
    assert err <= ATTN_TOL
    # plain attention reading the flags the step wrote
    got = c.attend(flags=dev(g_flags.view(np.int32)), num_splits=num_splits)
    assert not got[2].any()
    err = attn_error(got, {r: o_out[r] for r in (0, 1)})
    note(f"  flags read: error {err:.3e}")
    assert err <= ATTN_TOL
    # no tracker: every request attended (request 2 too), the pools already hold the step's tokens of 0 and 1
    _, g2_out = _device_step(c, k_new, v_new, req, pos, tracker=False, num_splits=num_splits, one_launch=True,
                             fused=fused)
    _, o2_out = step.decode_step(st, c.q, k_new, v_new, req, pos, tracker=False)
    err = attn_error(g2_out, o2_out)
    note(f"  no tracker: error {err:.3e}")
    assert err <= ATTN_TOL
    assert c.pools_match()


@pytest.mark.parametrize("fused", [False, True])
@pytest.mark.parametrize("kv_dtype", ["fp8", "bf16"])
def test_latent_step_128_head_kernel(kv_dtype, fused):
    """The latent step through kv_decode_step_* over one layer where the library picks the 128-head kernel
    (64 requests of 2,100-2,600 tokens, 128 heads: the wave-pair kernel's splits would exceed 1,024 tokens;
    4 splits): the check + write launch and the attention, or (fused) for the FP8 cache one launch whose
    blocks check their request's pages and store the token (BF16 keeps the two launches).  Stale tags, a page-table hole and an empty request;
    flags and the pool bit-exact to the oracle's check -> append, every row within tolerance, faulty
    requests zero."""
    w = wl.WORKLOADS["latent"].with_(batch=64, num_q_heads=128, num_pages=3000, ctx_lo=2100, ctx_hi=2600)
    note(f"latent step, 128-head kernel, {kv_dtype} fused={fused}")
    lens = wl.ctx_lens(w)
    lens[3] = 0
    c = Case(w, kv_dtype, lens=lens, stale=[1, 6])
    c.fill_device()
    hole = 5
    c.pt[hole, (int(c.lens[hole]) - 1) // w.page_size // 2] = -1
    c.dpt = dev(c.pt)
    k_new, _, req, pos = c.step_inputs()
    k_new = k_new ^ np.uint16(0x0040)
    st = dict(dtype=kv_dtype, k_pool=c.okp, v_pool=None, page_table=c.pt, ctx_lens=c.lens, page_tags=c.tags,
              expected_tags=c.exp, num_kv_heads=w.num_kv_heads, page_size=w.page_size, head_dim=w.head_dim,
              v_dim=w.v_dim, k_scale=c.o_k_scale, v_scale=c.o_v_scale, sm_scale=c.sm_scale, latent=True)
    o_flags, o_out = step.decode_step(st, c.q, k_new, None, req, pos)
    assert o_flags[hole] == paged.FLAG_BAD_PAGE and o_flags[1] and o_flags[6] and not o_flags[3]
    flags = torch.full((w.batch,), -1, dtype=torch.int32, device="cuda")
    out = c.out_tensor()
    splits = kv.paged_decode_attn_latent_auto_splits(w.batch, w.num_q_heads, c.max_ctx)
    assert splits == 4
    kv.decode_step(c.desc, kv_dtype, c.dkp, None, c.dpt, c.dlens, c.max_ctx, c.dq, dev(k_new), None, None, None, out,
                   page_tags=c.dtags, expected_tags=c.dexp, abort_flags=flags, k_scale=c.d_k_scale,
                   v_scale=c.d_v_scale, sm_scale=c.sm_scale, workspace=c.workspace(splits), fused_check=fused)
    torch.cuda.synchronize()
    g_flags, g_out = host(flags, np.uint32), host(out, np.uint16)
    assert np.array_equal(g_flags, o_flags)
    et = np.uint8 if kv_dtype == "fp8" else np.uint16
    assert np.array_equal(c.device_k(), c.okp)
    err = attn_error(g_out, o_out)
    note(f"  step error {err:.3e}")
    assert err <= ATTN_TOL
    for r in np.flatnonzero(o_flags).tolist() + [3]:
        assert not g_out[r].any()
