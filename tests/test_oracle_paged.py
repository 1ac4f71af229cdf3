"""Pins of the oracle's paged structures: tag check, append, gather (CPU only)."""
import numpy as np
import pytest

from kvsynth import workloads as wl
from oracle import codec, paged


def _small(name="sweep_b64", **kw):
    base = dict(batch=16, num_pages=2048, ctx_lo=100, ctx_hi=600)
    base.update(kw)
    return wl.WORKLOADS[name].with_(**base)


# ----------------------------------------------------------------------------- tag check

def test_tag_check_planted_stale_requests():
    """The generator knows which requests it corrupted: flags are known without any implementation."""
    w = _small(batch=64, ctx_lo=8192 // 16, ctx_hi=8192 // 16)
    lens = wl.ctx_lens(w)
    pt, _ = wl.page_table(w, lens)
    tags = wl.page_tags(w)
    stale = wl.stale_requests(w)
    assert len(stale) == 1                     # max(1, round(1% of 64))
    exp = wl.expected_tags(w, pt, lens, tags, stale)
    flags = paged.tag_check(tags, pt, exp, lens, w.page_size)
    want = np.zeros(w.batch, dtype=np.uint32)
    want[stale] = paged.FLAG_TAG_MISMATCH
    assert np.array_equal(flags, want)


def test_tag_check_every_position_detected():
    """A stale tag anywhere among the used entries is caught, and nowhere past them."""
    w = _small(batch=3, stale=False, ctx_lo=37, ctx_hi=37)      # 3 pages each, last one partial
    lens = wl.ctx_lens(w)
    pt, stride = wl.page_table(w, lens, stride=5)
    tags = wl.page_tags(w)
    exp = wl.expected_tags(w, pt, lens, tags)
    assert not paged.tag_check(tags, pt, exp, lens, w.page_size).any()
    for i in range(stride):
        e2 = exp.copy()
        e2[1, i] ^= 0x80000000
        f = paged.tag_check(tags, pt, e2, lens, w.page_size)
        assert f[0] == 0 and f[2] == 0
        assert f[1] == (paged.FLAG_TAG_MISMATCH if i < 3 else 0)
    # reallocation of a page bumps its tag: every holder of the old tag is caught
    t2 = tags.copy()
    t2[pt[2, 2]] = np.uint32(int(t2[pt[2, 2]]) + 1)
    f = paged.tag_check(t2, pt, exp, lens, w.page_size)
    assert f.tolist() == [0, 0, paged.FLAG_TAG_MISMATCH]
    # a tag generation counter wraps modulo 2^32
    t3 = tags.copy()
    t3[pt[0, 0]] = np.uint32(0xFFFFFFFF)
    e3 = exp.copy()
    e3[0, 0] = np.uint32(0xFFFFFFFF)
    assert paged.tag_check(t3, pt, e3, lens, w.page_size).tolist() == [0, 0, 0]


def test_tag_check_bad_page_ids_and_lengths():
    w = _small(batch=4, stale=False, ctx_lo=40, ctx_hi=40)
    lens = wl.ctx_lens(w)
    pt, _ = wl.page_table(w, lens, stride=3)
    tags = wl.page_tags(w)
    exp = wl.expected_tags(w, pt, lens, tags)
    pt2 = pt.copy()
    pt2[0, 1] = w.num_pages            # out of range
    pt2[1, 2] = -7
    lens2 = lens.copy()
    lens2[2] = 3 * 16 + 1              # needs a 4th page, the row has 3
    lens2[3] = 0                       # empty request: nothing to check
    f = paged.tag_check(tags, pt2, exp, lens2, w.page_size)
    assert f.tolist() == [paged.FLAG_BAD_PAGE, paged.FLAG_BAD_PAGE, paged.FLAG_BAD_PAGE, 0]
    # both bits together
    exp2 = exp.copy()
    exp2[0, 0] += np.uint32(1)
    f = paged.tag_check(tags, pt2, exp2, lens2, w.page_size)
    assert f[0] == paged.FLAG_BAD_PAGE | paged.FLAG_TAG_MISMATCH


# ----------------------------------------------------------------------------- layout / append / gather

def test_layout_offsets_by_hand():
    """Hand-worked offsets of the pool layout."""
    # e4m3 K, Hkv=2, S=16, D=64 (one 64-byte slice per row, NI=1): element (page 2, head 1, slot 13, d 37)
    #   block (2*2+1)*16*64 = 5120; token 13 = 4*3+1 (s=3, i=1); chunk 37//16 = 2 (q=2, k=0)
    #   chunk position ((3*1+0)*4+2)*4+1 = 57 -> 5120 + 57*16 + 37%16 = 6037
    assert paged.k_offset(2, 1, 13, 37, 2, 16, 64, 1) == 6037
    # e4m3 K, Hkv=1, S=32, D=64: (page 1, head 0, slot 17, d 0) -> 2048 + sub-page 1 (1024) + chunk 1 (16)
    assert paged.k_offset(1, 0, 17, 0, 1, 32, 64, 1) == 3088
    # bf16 K, Hkv=1, S=16, D=128 (8 elements a chunk, NI=4): (page 0, head 0, slot 5, d 100)
    #   token 5 (s=1, i=1); chunk 100//8 = 12 (q=3, k=0); position ((1*4+0)*4+3)*4+1 = 77 -> 77*8 + 4
    assert paged.k_offset(0, 0, 5, 100, 1, 16, 128, 2) == 620
    # e4m3 K, D=128 (NI=2): the 32 bytes lane group q reads of token 4s+i start at 512s + 64q + 16i
    # (first half, k=0) and 256 bytes later (second half, k=1)
    for s_ in range(4):
        for q in range(4):
            for i in range(4):
                assert paged.k_offset(0, 0, 4 * s_ + i, 32 * q, 1, 16, 128, 1) == 512 * s_ + 64 * q + 16 * i
                assert paged.k_offset(0, 0, 4 * s_ + i, 32 * q + 16, 1, 16, 128, 1) == 512 * s_ + 256 + 64 * q + 16 * i
    # V element (page 2, head 1, slot 3, d 4), Hkv=2, S=4, Dv=5: ((2*2+1)*5+4)*4+3 = 119
    assert paged.v_offset(2, 1, 3, 4, 2, 4, 5) == 119
    assert paged.v_offset(0, 0, 1, 0, 2, 4, 5) == 1


def test_latent_layout_offsets_by_hand():
    """A latent pool (no V pool) is row-major: element (page 3, slot 5, d 7) of a 576-wide, 16-slot pool
    sits (3*16 + 5)*576 + 7 = 30535 elements in; a page's tokens are consecutive 576-element rows."""
    assert paged.c_offset(3, 0, 5, 7, 1, 16, 576) == 30535
    assert paged.c_offset(0, 0, 0, 0, 1, 64, 576) == 0
    assert paged.c_offset(2, 0, 63, 575, 1, 64, 576) == 3 * 64 * 576 - 1   # last element of page 2
    slot, d = np.meshgrid(np.arange(64), np.arange(576), indexing="ij")
    assert np.array_equal(paged.c_offset(1, 0, slot, d, 1, 64, 576).ravel(), 64 * 576 + np.arange(64 * 576))


def test_latent_append_writes_contiguous_rows():
    """Appending into a latent pool (v_pool None) writes each token's whole row at row-major offsets."""
    S, D, P = 16, 576, 4
    cp = np.zeros(P * S * D, dtype=np.uint8)
    pt = np.array([[3, 1]], dtype=np.int32)
    rows = (np.arange(2 * D) % 251 + 1).astype(np.uint8).reshape(2, 1, D)
    paged.append(cp, None, rows, None, [0, 0], [2, 17], pt, 1, S)   # slot 2 of page 3, slot 1 of page 1
    assert np.array_equal(cp[(3 * S + 2) * D:(3 * S + 3) * D], rows[0, 0])
    assert np.array_equal(cp[(1 * S + 1) * D:(1 * S + 2) * D], rows[1, 0])
    assert cp.astype(np.int64).sum() == rows.astype(np.int64).sum()
    k, v = paged.gather(cp, None, pt, 0, 18, 1, S, D, 0)
    assert v is None and np.array_equal(k[17, 0], rows[1, 0]) and np.array_equal(k[2, 0], rows[0, 0])


@pytest.mark.parametrize("S,D,elt", [(16, 128, 1), (16, 128, 2), (64, 128, 1), (32, 576, 1), (16, 576, 2), (16, 64, 1)])
def test_k_layout_is_a_bijection_per_block(S, D, elt):
    slot, d = np.meshgrid(np.arange(S), np.arange(D), indexing="ij")
    off = paged.k_offset(1, 1, slot, d, 2, S, D, elt)
    base = (1 * 2 + 1) * S * D
    assert np.array_equal(np.sort(off.ravel()), base + np.arange(S * D))


def test_append_writes_exactly_the_addressed_elements():
    H, S, D, P = 2, 16, 64, 3
    kp = np.zeros(P * H * S * D, dtype=np.uint8)
    vp = np.zeros(P * H * S * D, dtype=np.uint8)
    pt = np.array([[2, 0]], dtype=np.int32)
    k_new = np.arange(1, 1 + H * D, dtype=np.uint8).reshape(1, H, D)
    v_new = (100 + np.arange(H * D) % 100).astype(np.uint8).reshape(1, H, D)
    paged.append(kp, vp, k_new, v_new, [0], [19], pt, H, S)       # token 19 -> page pt[0][1] = 0, slot 3
    for h in range(H):
        for d in range(D):
            assert kp[paged.k_offset(0, h, 3, d, H, S, D, 1)] == k_new[0, h, d]
    vv = vp.reshape(P, H, D, S)
    assert np.array_equal(vv[0, :, :, 3], v_new[0])
    assert kp.astype(np.int64).sum() == k_new.astype(np.int64).sum()
    assert vp.astype(np.int64).sum() == v_new.astype(np.int64).sum()


def test_append_gather_roundtrip_and_untouched_bytes():
    w = _small(batch=5, stale=False)
    lens = wl.ctx_lens(w)
    pt, _ = wl.page_table(w, lens)
    k, v = wl.all_kv(w, lens, threads=1)
    req, pos = wl.token_index(lens)
    kp0 = wl.pool_bytes(w, "k", 1)
    vp0 = wl.pool_bytes(w, "v", 1)
    kp, vp = kp0.copy(), vp0.copy()
    ks, vs = codec.calibrate_scale(k), codec.calibrate_scale(v)
    paged.append_fp8(kp, vp, k, v, req, pos, pt, w.num_kv_heads, w.page_size, ks, vs)
    off = np.concatenate([[0], np.cumsum(lens)])
    for r in range(w.batch):
        gk, gv = paged.gather(kp, vp, pt, r, int(lens[r]), w.num_kv_heads, w.page_size, w.head_dim, w.v_dim)
        assert np.array_equal(gk, codec.quantize_e4m3(k[off[r]:off[r + 1]], ks))
        assert np.array_equal(gv, codec.quantize_e4m3(v[off[r]:off[r + 1]], vs))
    # pages no request owns keep their random bytes
    used = set(pt[pt >= 0].tolist())
    blk = w.num_kv_heads * w.page_size * w.head_dim
    for p in range(w.num_pages):
        if p not in used:
            assert np.array_equal(kp[p * blk:(p + 1) * blk], kp0[p * blk:(p + 1) * blk])
            assert np.array_equal(vp[p * blk:(p + 1) * blk], vp0[p * blk:(p + 1) * blk])


def test_append_skips_flagged_and_out_of_range():
    H, S, D, P = 1, 16, 32, 4
    kp = np.zeros(P * H * S * D, dtype=np.uint16)
    vp = np.zeros(P * H * S * D, dtype=np.uint16)
    pt = np.array([[0, 1], [2, -1], [3, 9]], dtype=np.int32)
    k_new = np.full((5, H, D), 7, dtype=np.uint16)
    req = [0, 1, 1, 2, 2]
    pos = [1, 0, 17, 2, 18]      # r1 pos17 -> entry -1 (skip); r2 pos18 -> page 9 (skip)
    flags = np.array([1, 0, 0], dtype=np.uint32)                 # r0 aborted
    paged.append(kp, vp, k_new, k_new, req, pos, pt, H, S, flags=flags)
    blk = H * S * D
    assert kp[:2 * blk].sum() == 0
    got = lambda page, slot: kp[paged.k_offset(page, 0, slot, np.arange(D), H, S, D, 2)]
    assert (got(2, 0) == 7).all() and (got(3, 2) == 7).all()
    assert kp.astype(np.int64).sum() == 7 * D * 2
    # positions beyond the page-table row are skipped too
    kp2 = np.zeros_like(kp)
    paged.append(kp2, None, k_new[:1], None, [2], [32], pt, H, S)
    assert kp2.sum() == 0


def test_kv_bytes_formula_and_capacity_doubling():
    """KV bytes = requests x tokens x layers x KV heads x head_dim x 2 x bytes (zdabc.icu article,
    section on why memory bounds long-context inference).  At a fixed byte budget FP8 holds twice
    the tokens of BF16; the Cloudflare post ("Quantized KV cache") reports about 686,000 -> about
    1.37 million tokens on Kimi K2.6, a ratio of 1.997 that rounding of "about" accounts for."""
    assert paged.kv_bytes(1, 1, 1, 1, 1, 1) == 2
    assert paged.kv_bytes(64, 8192, 1, 8, 128, 1) == 1073741824         # one layer, 64 x 8192, FP8
    budget = 10 ** 12
    per_tok_bf16 = paged.kv_bytes(1, 1, 61, 8, 128, 2)
    per_tok_fp8 = paged.kv_bytes(1, 1, 61, 8, 128, 1)
    assert budget // per_tok_fp8 == 2 * (budget // per_tok_bf16) or \
        budget // per_tok_fp8 == 2 * (budget // per_tok_bf16) + 1
    assert abs(1.37e6 / 686000 - 2.0) < 0.01
