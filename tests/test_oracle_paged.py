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

def test_append_writes_exactly_the_addressed_elements():
    """Token 19 of a request whose second page-table entry is page 0 lands at page 0, slot 3, for every
    kv head, in K and V; nothing else changes."""
    H, S, D, P = 2, 16, 64, 3
    kp = np.zeros((P, H, S, D), dtype=np.uint8)
    vp = np.zeros((P, H, S, 16), dtype=np.uint8)
    pt = np.array([[2, 0]], dtype=np.int32)
    k_new = np.arange(1, 1 + H * D, dtype=np.uint8).reshape(1, H, D)
    v_new = (100 + np.arange(H * 16) % 100).astype(np.uint8).reshape(1, H, 16)
    paged.append(kp, vp, k_new, v_new, [0], [19], pt)
    assert np.array_equal(kp[0, :, 3, :], k_new[0]) and np.array_equal(vp[0, :, 3, :], v_new[0])
    assert kp.astype(np.int64).sum() == k_new.astype(np.int64).sum()
    assert vp.astype(np.int64).sum() == v_new.astype(np.int64).sum()
    got_k, got_v = paged.gather(kp, vp, pt, 0, 20)
    assert np.array_equal(got_k[19], k_new[0]) and np.array_equal(got_v[19], v_new[0])
    assert not got_k[:19].any()


def test_latent_append_writes_whole_rows():
    """Appending into a latent pool (v_pool None) writes each token's whole 576-wide row."""
    S, D, P = 16, 576, 4
    cp = np.zeros((P, 1, S, D), dtype=np.uint8)
    pt = np.array([[3, 1]], dtype=np.int32)
    rows = (np.arange(2 * D) % 251 + 1).astype(np.uint8).reshape(2, 1, D)
    paged.append(cp, None, rows, None, [0, 0], [2, 17], pt)   # slot 2 of page 3, slot 1 of page 1
    assert np.array_equal(cp[3, 0, 2], rows[0, 0]) and np.array_equal(cp[1, 0, 1], rows[1, 0])
    assert cp.astype(np.int64).sum() == rows.astype(np.int64).sum()
    k, v = paged.gather(cp, None, pt, 0, 18)
    assert v is None and np.array_equal(k[17, 0], rows[1, 0]) and np.array_equal(k[2, 0], rows[0, 0])


def test_later_token_wins_on_one_slot():
    kp = np.zeros((2, 1, 16, 4), dtype=np.uint16)
    pt = np.array([[1]], dtype=np.int32)
    rows = np.array([[[1, 1, 1, 1]], [[2, 2, 2, 2]]], dtype=np.uint16)
    paged.append(kp, None, rows, None, [0, 0], [5, 5], pt)
    assert kp[1, 0, 5].tolist() == [2, 2, 2, 2]


def test_append_gather_roundtrip_and_untouched_bytes():
    w = _small(batch=5, stale=False)
    lens = wl.ctx_lens(w)
    pt, _ = wl.page_table(w, lens)
    k, v = wl.all_kv(w, lens, threads=1)
    req, pos = wl.token_index(lens)
    kp0 = wl.pool_init(w, "k", 1)
    vp0 = wl.pool_init(w, "v", 1)
    kp, vp = kp0.copy(), vp0.copy()
    ks, vs = codec.calibrate_scale(k), codec.calibrate_scale(v)
    paged.append_fp8(kp, vp, k, v, req, pos, pt, ks, vs)
    off = np.concatenate([[0], np.cumsum(lens)])
    for r in range(w.batch):
        gk, gv = paged.gather(kp, vp, pt, r, int(lens[r]))
        assert np.array_equal(gk, codec.quantize_e4m3(k[off[r]:off[r + 1]], ks))
        assert np.array_equal(gv, codec.quantize_e4m3(v[off[r]:off[r + 1]], vs))
    # pages no request owns keep their random bytes
    unused = sorted(set(range(w.num_pages)) - set(pt[pt >= 0].tolist()))
    assert np.array_equal(kp[unused], kp0[unused]) and np.array_equal(vp[unused], vp0[unused])
    # slots past a request's last token keep their random bytes too
    r = int(np.argmin(lens % w.page_size == 0))
    p_last, s_last = pt[r, (lens[r] - 1) // w.page_size], (lens[r] - 1) % w.page_size
    assert np.array_equal(kp[p_last, :, s_last + 1:], kp0[p_last, :, s_last + 1:])


def test_append_skips_flagged_and_out_of_range():
    H, S, D, P = 1, 16, 32, 4
    kp = np.zeros((P, H, S, D), dtype=np.uint16)
    vp = np.zeros((P, H, S, D), dtype=np.uint16)
    pt = np.array([[0, 1], [2, -1], [3, 9]], dtype=np.int32)
    k_new = np.full((5, H, D), 7, dtype=np.uint16)
    req = [0, 1, 1, 2, 2]
    pos = [1, 0, 17, 2, 18]      # r1 pos17 -> entry -1 (skip); r2 pos18 -> page 9 (skip)
    flags = np.array([1, 0, 0], dtype=np.uint32)                 # r0 aborted
    paged.append(kp, vp, k_new, k_new, req, pos, pt, flags=flags)
    assert kp[:2].sum() == 0
    assert (kp[2, 0, 0] == 7).all() and (kp[3, 0, 2] == 7).all()
    assert kp.astype(np.int64).sum() == 7 * D * 2
    assert np.array_equal(kp, vp)
    # positions beyond the page-table row are skipped too
    kp2 = np.zeros_like(kp)
    paged.append(kp2, None, k_new[:1], None, [2], [32], pt)
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
