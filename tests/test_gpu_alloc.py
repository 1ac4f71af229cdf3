"""The tag lifecycle end to end on the GPU: the library's page allocator hands request A's pages to
request C after A's pages were freed (their tags change), and a decode step that still carries A's
old page table and tags aborts A -- its new token is not written into C's pages and its rows are zero
-- while B and C match the oracle (agentlenshq summary, section "KV Cache 完整性检查"; xujun.org note,
section "一个不能出错的共享缓存")."""
import math

import numpy as np
import pytest
import torch

import fp8_paged_kv_append_amd as kv
from kvsynth import workloads as wl
from oracle import attention, codec, paged
from tests.gpu_util import ATTN_TOL, dev, host, note

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("kv_dtype", ["fp8", "bf16"])
def test_stale_holder_aborts_after_reallocation(kv_dtype):
    note(f"allocator stale holder {kv_dtype}")
    w = wl.Workload("alloc", batch=3, num_q_heads=8, num_kv_heads=1, head_dim=128, v_dim=128, page_size=16,
                    num_pages=24, ctx_lo=70, ctx_hi=100, seed=21)
    S, P, D = w.page_size, w.num_pages, w.head_dim
    lens = np.array([100, 70, 90], dtype=np.int32)          # A, B, C (C arrives after A is freed)
    need = [math.ceil(int(L) / S) for L in lens]
    alloc = kv.PageAllocator(P)
    pa, ta = alloc.alloc(need[0])
    pb, tb = alloc.alloc(need[1])
    stride = max(need)
    pt = np.full((3, stride), -1, dtype=np.int32)
    exp = np.zeros((3, stride), dtype=np.uint32)
    pt[0, :need[0]], exp[0, :need[0]] = pa, ta
    pt[1, :need[1]], exp[1, :need[1]] = pb, tb
    k = [wl.request_k(w, r, int(lens[r])) for r in range(3)]
    v = [wl.request_v(w, r, int(lens[r])) for r in range(3)]
    fp8 = kv_dtype == "fp8"
    et = np.uint8 if fp8 else np.uint16
    tdt = torch.uint8 if fp8 else torch.int16
    desc = kv.pool_desc(P, S, 1, D)
    dkp = torch.zeros(P * S * D, dtype=tdt, device="cuda")
    dvp = torch.zeros(P * S * D, dtype=tdt, device="cuda")
    allk = np.concatenate(k)
    allv = np.concatenate(v)
    ks = codec.calibrate_scale(allk) if fp8 else np.float32(1)
    vs = codec.calibrate_scale(allv) if fp8 else np.float32(1)

    def append(rows_k, rows_v, req, pos, page_table):
        if fp8:
            kv.kv_append_fp8(desc, dkp, dvp, dev(rows_k), dev(rows_v), dev(req), dev(pos), dev(page_table),
                             k_scale=float(ks), v_scale=float(vs))
        else:
            kv.kv_append_bf16(desc, dkp, dvp, dev(rows_k), dev(rows_v), dev(req), dev(pos), dev(page_table))

    # A and B fill their pages (all but the token appended by the step)
    for r in (0, 1):
        L = int(lens[r]) - 1
        append(k[r][:L], v[r][:L], np.full(L, r, np.int32), np.arange(L, dtype=np.int32), pt)
    # A is evicted: its pages go back; C is admitted and reuses them (last freed, first handed out)
    alloc.free(pa)
    pc, tc = alloc.alloc(need[2])
    assert set(pc.tolist()) & set(pa.tolist()), "C should reuse A's pages"
    pt[2, :need[2]], exp[2, :need[2]] = pc, tc
    L = int(lens[2]) - 1
    append(k[2][:L], v[2][:L], np.full(L, 2, np.int32), np.arange(L, dtype=np.int32), pt)
    tags = alloc.tags()
    # one decode step, A still holding its old page-table row and tags: fused check + append, attention
    q = wl.queries(w)
    new_k = np.stack([k[r][-1] for r in range(3)])
    new_v = np.stack([v[r][-1] for r in range(3)])
    flags = torch.full((3,), -1, dtype=torch.int32, device="cuda")
    out = torch.empty((3, w.num_q_heads, D), dtype=torch.int16, device="cuda")
    sm = 1.0 / math.sqrt(D)
    kv.decode_step(desc, kv_dtype, dkp, dvp, dev(pt), dev(lens), int(lens.max()), dev(q), dev(new_k), dev(new_v),
                   None, None, out, page_tags=dev(tags), expected_tags=dev(exp), abort_flags=flags,
                   k_scale=float(ks), v_scale=float(vs), sm_scale=sm)
    torch.cuda.synchronize()
    g_flags = host(flags, np.uint32)
    assert g_flags.tolist() == [paged.FLAG_TAG_MISMATCH, 0, 0]
    assert np.array_equal(g_flags, paged.tag_check(tags, pt, exp, lens, S))
    g_out = host(out, np.uint16)
    assert not g_out[0].any()
    # C's pages hold C's rows only (A's new token went nowhere), B's its own
    for r in (1, 2):
        Lr = int(lens[r])
        ko = torch.empty((Lr, 1, D), dtype=tdt, device="cuda")
        vo = torch.empty((Lr, 1, D), dtype=tdt, device="cuda")
        g = kv.kv_gather_fp8 if fp8 else kv.kv_gather_bf16
        g(desc, dkp, dvp, dev(np.full(Lr, r, np.int32)), dev(np.arange(Lr, dtype=np.int32)), dev(pt), ko, vo)
        torch.cuda.synchronize()
        want_k = codec.quantize_e4m3(k[r], ks) if fp8 else k[r]
        want_v = codec.quantize_e4m3(v[r], vs) if fp8 else v[r]
        assert np.array_equal(host(ko, et), want_k) and np.array_equal(host(vo, et), want_v)
        kh = codec.dequantize_e4m3(want_k, ks) if fp8 else codec.f64_from_bf16(want_k)
        vh = codec.dequantize_e4m3(want_v, vs) if fp8 else codec.f64_from_bf16(want_v)
        ref = attention.request_attention(codec.f64_from_bf16(q[r]), kh, vh, 1, sm)
        err = float(np.max(attention.row_rel_error(codec.f64_from_bf16(g_out[r]), ref)))
        note(f"  request {r}: row error {err:.3e}")
        assert err <= ATTN_TOL
