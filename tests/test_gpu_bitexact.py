"""GPU parity, bit-exact tier: e4m3 encode, e4m3 decode, append/scatter, gather, tag-check flags, absmax.

Every call goes through the library's C ABI (via the thin binding); every
expected value comes from the oracle or from the generator's planted faults.
"""
import numpy as np
import pytest
import torch

import fp8_paged_kv_append_amd as kv
from kvsynth import workloads as wl
from oracle import attention, codec, paged, step
from tests import layout
from tests.gpu_util import Case, dev, host, note

pytestmark = pytest.mark.gpu

ALL_BF16 = np.arange(65536, dtype=np.uint32).astype(np.uint16)


# ----------------------------------------------------------------------------- encode

@pytest.mark.parametrize("scale", [1.0, 2.0 ** -3, 2.0 ** -6, 4.5 / 448, 5.3125 / 448, 3.0e-3, 1e-30, 3e38])
def test_encode_every_bf16_value(scale):
    """All 65,536 bf16 inputs through kv_append_fp8 (K rows and transposed V rows) vs the oracle encoder."""
    note(f"encode all bf16, scale={scale}")
    S, D, N = 16, 128, 512
    P = N // S
    x = ALL_BF16.reshape(N, 1, D)
    xv = ALL_BF16[::-1].copy().reshape(N, 1, D)
    pt = np.arange(P, dtype=np.int32)[None, :]
    req = np.zeros(N, dtype=np.int32)
    pos = np.arange(N, dtype=np.int32)
    desc = kv.pool_desc(P, S, 1, D)
    dk = torch.zeros(P * S * D, dtype=torch.uint8, device="cuda")
    dvp = torch.zeros(P * S * D, dtype=torch.uint8, device="cuda")
    kv.kv_append_fp8(desc, dk, dvp, dev(x), dev(xv), dev(req), dev(pos), dev(pt), k_scale=scale, v_scale=scale)
    ok = np.zeros((P, 1, S, D), dtype=np.uint8)
    ov = np.zeros((P, 1, S, D), dtype=np.uint8)
    paged.append_fp8(ok, ov, x, xv, req, pos, pt, np.float32(scale), np.float32(scale))
    gk = layout.from_device(host(dk, np.uint8), "k", ok.shape, 1)
    gv = layout.from_device(host(dvp, np.uint8), "v", ov.shape, 1)
    bad = np.flatnonzero(gk != ok)
    assert bad.size == 0, f"{bad.size} K codes differ, e.g. got {gk.ravel()[bad[:5]]} want {ok.ravel()[bad[:5]]}"
    assert np.array_equal(gv, ov)


# ----------------------------------------------------------------------------- decode

@pytest.mark.parametrize("v_scale", [1.0, 0.0123, 7.75])
def test_decode_every_code_single_token(v_scale):
    """L = 1: the output is the dequantised V row, bf16(fl32(dec(c) * v_scale)), for all 256 codes."""
    note(f"decode all codes, v_scale={v_scale}")
    S, D, B, G = 16, 128, 2, 4
    P = 4
    kp = np.random.Generator(np.random.PCG64(1)).integers(0, 0x78, (P, 1, S, D), dtype=np.uint8)  # finite K
    vp = np.zeros((P, 1, S, D), dtype=np.uint8)
    pt = np.array([[3], [1]], dtype=np.int32)
    codes = np.arange(256, dtype=np.uint8).reshape(2, D)
    for r in range(B):
        paged.append(np.zeros_like(kp), vp, codes[r].reshape(1, 1, D), codes[r].reshape(1, 1, D), [r], [0], pt)
    q = wl.to_bf16_bits(np.random.Generator(np.random.PCG64(2)).standard_normal((B, G, D)).astype(np.float32))
    lens = np.ones(B, dtype=np.int32)
    desc = kv.pool_desc(P, S, 1, D)
    out = torch.empty((B, G, D), dtype=torch.int16, device="cuda")
    kv.paged_decode_attn_fp8(desc, dev(q), dev(layout.to_device(kp, "k", 1)), dev(layout.to_device(vp, "v", 1)),
                             dev(pt), dev(lens), 1, out, k_scale=0.5, v_scale=v_scale, sm_scale=D ** -0.5,
                             num_splits=1)
    got = host(out, np.uint16)
    ref = attention.decode_attention(q, kp, vp, pt, lens, num_kv_heads=1, page_size=S, head_dim=D, v_dim=D,
                                     dtype="fp8", k_scale=np.float32(0.5), v_scale=np.float32(v_scale))
    for r in range(B):
        want = step.output_bf16(ref[r])
        nan = np.isnan(codec.f32_from_bf16(want))
        assert np.array_equal(np.isnan(codec.f32_from_bf16(got[r])), nan)
        assert np.array_equal(got[r][~nan], want[~nan]), r


# ----------------------------------------------------------------------------- append / gather

def _reduced(name, **kw):
    base = dict(batch=6, num_pages=600, ctx_lo=70, ctx_hi=700)
    base.update(kw)
    return wl.WORKLOADS[name].with_(**base)


@pytest.mark.parametrize("kv_dtype", ["fp8", "bf16"])
@pytest.mark.parametrize("name,kw", [("gqa_batch", {}), ("long", dict(num_pages=100, ctx_lo=300, ctx_hi=900)),
                                     ("latent", dict(num_pages=64, ctx_lo=100, ctx_hi=400))])
def test_fill_whole_pool_bytes(kv_dtype, name, kw):
    """Bulk append of every token: the whole device pool (untouched pages included) equals the oracle's."""
    w = _reduced(name, **kw)
    note(f"fill {name} {kv_dtype} B={w.batch}")
    c = Case(w, kv_dtype)
    assert c.d_k_scale == float(c.o_k_scale) and c.d_v_scale == float(c.o_v_scale)
    c.fill_device()
    torch.cuda.synchronize()
    et = c.et
    assert c.pools_match()
    # read back through the page table
    ko = torch.empty((len(c.req), w.num_kv_heads, w.head_dim), dtype=c.dkp.dtype, device="cuda")
    vo = None if w.latent else torch.empty((len(c.req), w.num_kv_heads, w.v_dim), dtype=c.dkp.dtype, device="cuda")
    g = kv.kv_gather_fp8 if kv_dtype == "fp8" else kv.kv_gather_bf16
    g(c.desc, c.dkp, c.dvp, c.dreq, c.dpos, c.dpt, ko, vo)
    torch.cuda.synchronize()
    for r in range(w.batch):
        ok_, ov_ = paged.gather(c.okp, c.ovp, c.pt, r, int(c.lens[r]))
        a, b = c.off[r], c.off[r + 1]
        assert np.array_equal(host(ko, et)[a:b], ok_)
        if not w.latent:
            assert np.array_equal(host(vo, et)[a:b], ov_)


@pytest.mark.parametrize("kv_dtype", ["fp8", "bf16"])
def test_append_skips_flagged_and_out_of_range(kv_dtype):
    note(f"append skip rules {kv_dtype}")
    H, S, D, P = 2, 16, 128, 6
    et = np.uint8 if kv_dtype == "fp8" else np.uint16
    pt = np.array([[0, 1], [2, -1], [3, 9], [4, 5]], dtype=np.int32)
    rng = np.random.Generator(np.random.PCG64(3))
    rows = wl.to_bf16_bits(rng.standard_normal((7, H, D)).astype(np.float32))
    req = np.array([0, 1, 1, 2, 2, 7, 3], dtype=np.int32)
    pos = np.array([1, 0, 17, 2, 20, 0, 40], dtype=np.int32)   # r1@17 -> entry -1; r2@20 -> page 9; r7; pos 40
    flags = np.array([1, 0, 0, 0], dtype=np.uint32)
    elt = 1 if kv_dtype == "fp8" else 2
    kp0 = rng.integers(0, 256, P * H * S * D * elt, dtype=np.uint8).view(et).reshape(P, H, S, D)
    vp0 = rng.integers(0, 256, P * H * S * D * elt, dtype=np.uint8).view(et).reshape(P, H, S, D)
    desc = kv.pool_desc(P, S, H, D)
    dk, dvv = dev(layout.to_device(kp0, "k", elt)), dev(layout.to_device(vp0, "v", elt))
    if kv_dtype == "fp8":
        kv.kv_append_fp8(desc, dk, dvv, dev(rows), dev(rows), dev(req), dev(pos), dev(pt), dev(flags),
                         k_scale=0.01, v_scale=0.02)
        ok, ov = kp0.copy(), vp0.copy()
        paged.append_fp8(ok, ov, rows, rows, req, pos, pt, np.float32(0.01), np.float32(0.02), flags)
    else:
        kv.kv_append_bf16(desc, dk, dvv, dev(rows), dev(rows), dev(req), dev(pos), dev(pt), dev(flags))
        ok, ov = kp0.copy(), vp0.copy()
        paged.append(ok, ov, rows, rows, req, pos, pt, flags)
    torch.cuda.synchronize()
    assert np.array_equal(layout.from_device(host(dk, et), "k", ok.shape, elt), ok)
    assert np.array_equal(layout.from_device(host(dvv, et), "v", ov.shape, elt), ov)
    assert not np.array_equal(ok, kp0)          # something was written


# ----------------------------------------------------------------------------- tag check

def _flags(tags, pt, exp, lens, S):
    out = torch.full((pt.shape[0],), -1, dtype=torch.int32, device="cuda")
    kv.kv_tag_check(dev(tags), dev(pt), dev(exp), dev(lens), S, out)
    torch.cuda.synchronize()
    return host(out, np.uint32)


@pytest.mark.parametrize("b", [1, 8, 16, 32, 64])
def test_tag_check_planted_stale(b):
    w = wl.WORKLOADS[f"sweep_b{b}"]
    note(f"tag check sweep B={b}")
    lens = wl.ctx_lens(w)
    pt, _ = wl.page_table(w, lens)
    tags = wl.page_tags(w)
    stale = wl.stale_requests(w)
    exp = wl.expected_tags(w, pt, lens, tags, stale)
    got = _flags(tags, pt, exp, lens, w.page_size)
    want = np.zeros(b, dtype=np.uint32)
    want[stale] = 1
    assert np.array_equal(got, want)
    assert np.array_equal(got, paged.tag_check(tags, pt, exp, lens, w.page_size))
    assert (b >= 8) == bool(got.any())


def test_tag_check_edge_cases_and_random_faults():
    note("tag check edges")
    rng = np.random.Generator(np.random.PCG64(4))
    B, S, P = 300, 16, 5000
    lens = rng.integers(-3, 700, B).astype(np.int32)
    lens[:4] = [0, -1, 1, 16 * 48]
    stride = 48
    need = np.maximum((lens.astype(np.int64) + S - 1) // S, 0)
    lens[5] = 16 * 48 + 1                                   # needs 49 entries: row too short
    pt = rng.integers(0, P, (B, stride)).astype(np.int32)
    tags = rng.integers(0, 2 ** 32, P, dtype=np.uint32)
    exp = tags[pt].copy()
    for r in rng.choice(B, 40, replace=False):              # random stale entries, some past the used ones
        i = int(rng.integers(0, stride))
        exp[r, i] += np.uint32(1)
    for r in rng.choice(B, 20, replace=False):              # random bad page ids
        i = int(rng.integers(0, stride))
        pt[r, i] = [-1, P, P + 7, -2 ** 31][int(rng.integers(0, 4))]
    got = _flags(tags, pt, exp, lens, S)
    want = paged.tag_check(tags, pt, exp, lens, S)
    assert np.array_equal(got, want)
    assert (want == 1).any() and (want == 2).any() and want[5] & 2 and want[0] == 0 and want[1] == 0
    assert need.max() > 0


# ----------------------------------------------------------------------------- scale calibration

def test_absmax_matches_oracle():
    note("absmax")
    rng = np.random.Generator(np.random.PCG64(5))
    for n in [1, 7, 8, 9, 1000, 65537, 1 << 20]:
        x = wl.to_bf16_bits(rng.standard_normal(n).astype(np.float32) * np.float32(rng.uniform(0.1, 100)))
        if n > 10:
            x[3] = 0x7FC1                                    # NaN: ignored
            x[4] = 0xFF90
        acc = torch.zeros(1, dtype=torch.int32, device="cuda")
        kv.kv_absmax_bf16(dev(x), acc)
        bits = int(host(acc, np.uint32)[0])
        assert bits == int(codec.absmax_bits(x)), n
        assert kv.kv_scale_from_absmax(bits) == float(codec.scale_from_absmax(np.uint32(bits).view(np.float32)))
    # +inf counts
    x = np.array([0x3F80, 0x7F80, 0x4000], dtype=np.uint16)
    acc = torch.zeros(1, dtype=torch.int32, device="cuda")
    kv.kv_absmax_bf16(dev(x), acc)
    assert int(host(acc, np.uint32)[0]) == 0x7F800000
