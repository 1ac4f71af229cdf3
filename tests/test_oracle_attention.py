"""Pins of the oracle's decode attention (CPU only): closed forms, invariances, brute force."""
import math

import numpy as np
import pytest

from kvsynth import workloads as wl
from oracle import attention, codec, paged, step


def _cache(w, dtype, lens=None, pool_pages=None):
    """A filled cache for workload w: (state dict for oracle.step, K bits, V bits, lens)."""
    lens = wl.ctx_lens(w) if lens is None else np.asarray(lens, dtype=np.int32)
    pt, _ = wl.page_table(w, lens)
    k, v = wl.all_kv(w, lens, threads=1)
    req, pos = wl.token_index(lens)
    elt = 1 if dtype == "fp8" else 2
    kp = wl.pool_init(w, "k", elt)
    vp = None if w.latent else wl.pool_init(w, "v", elt)
    ks = codec.calibrate_scale(k) if dtype == "fp8" else np.float32(1)
    vs = (codec.calibrate_scale(v) if not w.latent else ks) if dtype == "fp8" else np.float32(1)
    if dtype == "fp8":
        paged.append_fp8(kp, vp, k, None if w.latent else v, req, pos, pt, ks, vs)
    else:
        paged.append(kp, vp, k, None if w.latent else v, req, pos, pt)
    tags = wl.page_tags(w)
    st = dict(dtype=dtype, k_pool=kp, v_pool=vp, page_table=pt, ctx_lens=lens, page_tags=tags,
              expected_tags=wl.expected_tags(w, pt, lens, tags), num_kv_heads=w.num_kv_heads,
              page_size=w.page_size, head_dim=w.head_dim, v_dim=w.v_dim, k_scale=ks, v_scale=vs,
              sm_scale=1.0 / math.sqrt(w.head_dim), latent=w.latent)
    return st, k, v, lens


def _attn(st, q, flags=None, requests=None):
    return attention.decode_attention(q, st["k_pool"], st["v_pool"], st["page_table"], st["ctx_lens"],
                                      num_kv_heads=st["num_kv_heads"], page_size=st["page_size"],
                                      head_dim=st["head_dim"], v_dim=st["v_dim"], dtype=st["dtype"],
                                      k_scale=st["k_scale"], v_scale=st["v_scale"],
                                      sm_scale=st["sm_scale"], flags=flags, requests=requests,
                                      latent=st["latent"])


TINY = wl.WORKLOADS["tiny"]


@pytest.mark.parametrize("dtype", ["fp8", "bf16"])
def test_single_token_returns_dequantised_value(dtype):
    w = TINY.with_(ctx_lo=1, ctx_hi=1)
    st, k, v, lens = _cache(w, dtype)
    q = wl.queries(w)
    o = _attn(st, q)[0]
    if dtype == "fp8":
        ref = codec.e4m3_decode(codec.quantize_e4m3(v[0, 0], st["v_scale"])) * np.float64(st["v_scale"])
    else:
        ref = codec.f64_from_bf16(v[0, 0])
    for h in range(w.num_q_heads):
        assert np.array_equal(o[h], ref)


@pytest.mark.parametrize("dtype", ["fp8", "bf16"])
def test_equal_keys_give_mean_of_values(dtype):
    w = TINY.with_(ctx_lo=37, ctx_hi=37)
    st, k, v, lens = _cache(w, dtype)
    # overwrite every K row with token 0's row: all scores are equal, softmax is uniform
    k_same = np.broadcast_to(k[:1], k.shape).copy()
    req, pos = wl.token_index(lens)
    if dtype == "fp8":
        # V is rewritten with its own rows (same codes); a call without the V pool would address a latent pool
        paged.append_fp8(st["k_pool"], st["v_pool"], k_same, v, req, pos, st["page_table"], st["k_scale"],
                         st["v_scale"])
        vhat = codec.e4m3_decode(codec.quantize_e4m3(v, st["v_scale"])) * np.float64(st["v_scale"])
    else:
        paged.append(st["k_pool"], st["v_pool"], k_same, v, req, pos, st["page_table"])
        vhat = codec.f64_from_bf16(v)
    o = _attn(st, wl.queries(w))[0]
    ref = vhat[:, 0, :].mean(axis=0)
    for h in range(w.num_q_heads):
        np.testing.assert_allclose(o[h], ref, rtol=0, atol=1e-13)


def _decoder(dtype):
    if dtype == "fp8":
        return lambda c: float(codec.e4m3_decode([c])[0])
    return lambda b: float(codec.f32_from_bf16([b])[0])


def _softmax_rows(q, keys, values):
    """Pure-Python softmax attention of one query row over lists of key and value rows."""
    scores = [sum(a * b for a, b in zip(q, kk)) for kk in keys]
    mx = max(scores)
    e = [math.exp(s - mx) for s in scores]
    z = sum(e)
    o = [0.0] * len(values[0])
    for t, vv in enumerate(values):
        for d, x in enumerate(vv):
            o[d] += e[t] / z * x
    return o


def _brute_force(q_bits, k_pool, v_pool, pt, lens, H, S, D, Dv, Hq, dtype, ks, vs, sm):
    """Pure-Python loops straight from the definition, reading the pools element by element."""
    dec = _decoder(dtype)
    out = []
    G = Hq // H
    for r in range(len(lens)):
        rows = []
        for h in range(Hq):
            g = h // G
            q = [sm * float(codec.f32_from_bf16([q_bits[r, h, d]])[0]) for d in range(D)]
            keys, values = [], []
            for t in range(lens[r]):
                page, slot = int(pt[r, t // S]), t % S
                keys.append([dec(k_pool[page, g, slot, d]) * ks for d in range(D)])
                values.append([dec(v_pool[page, g, slot, d]) * vs for d in range(Dv)])
            rows.append(_softmax_rows(q, keys, values))
        out.append(rows)
    return np.array(out)


@pytest.mark.parametrize("dtype", ["fp8", "bf16"])
def test_brute_force_tiny_shapes(dtype):
    w = wl.Workload("bf", batch=3, num_q_heads=4, num_kv_heads=2, head_dim=16, v_dim=16, page_size=16,
                    num_pages=12, ctx_lo=1, ctx_hi=40, seed=99)
    lens = np.array([40, 17, 1], dtype=np.int32)
    st, k, v, _ = _cache(w, dtype, lens=lens)
    q = wl.queries(w)
    got = _attn(st, q)
    ref = _brute_force(q, st["k_pool"], st["v_pool"], st["page_table"], lens, 2, 16, 16, 16, 4, dtype,
                       float(st["k_scale"]), float(st["v_scale"]), st["sm_scale"])
    for r in range(3):
        np.testing.assert_allclose(got[r], ref[r], rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("dtype", ["fp8", "bf16"])
def test_brute_force_latent_tiny_shapes(dtype):
    """Latent cache: every head scores against the whole cached vector and averages its first Dv dims."""
    w = wl.Workload("bfl", batch=3, num_q_heads=4, num_kv_heads=1, head_dim=24, v_dim=16, page_size=16,
                    num_pages=10, ctx_lo=1, ctx_hi=40, seed=98, latent=True)
    lens = np.array([33, 1, 16], dtype=np.int32)
    st, k, _, _ = _cache(w, dtype, lens=lens)
    q = wl.queries(w)
    got = _attn(st, q)
    dec = _decoder(dtype)
    sc = float(st["k_scale"])
    for r in range(3):
        for h in range(4):
            qq = [st["sm_scale"] * float(codec.f32_from_bf16([q[r, h, d]])[0]) for d in range(24)]
            rows = []
            for t in range(lens[r]):
                page, slot = int(st["page_table"][r, t // 16]), t % 16
                rows.append([dec(st["k_pool"][page, 0, slot, d]) * sc for d in range(24)])
            ref = _softmax_rows(qq, rows, [row[:16] for row in rows])
            np.testing.assert_allclose(got[r][h], ref, rtol=1e-12, atol=1e-13)


def test_score_shift_invariance():
    rng = np.random.Generator(np.random.PCG64(5))
    q = rng.standard_normal((3, 16))
    k = rng.standard_normal((29, 16))
    v = rng.standard_normal((29, 8))
    base = attention.softmax_attention(q, k, v, 0.25)
    # adding u to every key with <q_h, u> = c adds sm*c to all of head h's scores
    for h in range(3):
        u = q[h] * (7.5 / (q[h] @ q[h]))
        shifted = attention.softmax_attention(q[h:h + 1], k + u, v, 0.25)
        np.testing.assert_allclose(shifted[0], base[h], rtol=1e-12, atol=1e-13)


def test_two_token_closed_form():
    q = np.array([[1.0, 0.0]])
    k = np.array([[2.0, 0.0], [0.0, 5.0]])
    v = np.array([[1.0, 3.0], [-1.0, 0.5]])
    o = attention.softmax_attention(q, k, v, 0.5)
    a = 1.0 / (1.0 + math.exp(-1.0))          # scores 1 and 0
    np.testing.assert_allclose(o[0], a * v[0] + (1 - a) * v[1], rtol=1e-15)


def test_physical_page_permutation_invariance():
    w = wl.WORKLOADS["tiny"]
    st, k, v, lens = _cache(w, "fp8")
    q = wl.queries(w)
    o1 = _attn(st, q)[0]
    # move every page to another physical slot and rewrite the table: identical output
    P = w.num_pages
    perm = np.random.Generator(np.random.PCG64(3)).permutation(P)
    kp2 = np.empty_like(st["k_pool"])
    vp2 = np.empty_like(st["v_pool"])
    kp2[perm] = st["k_pool"]
    vp2[perm] = st["v_pool"]
    st2 = dict(st, k_pool=kp2, v_pool=vp2, page_table=np.where(st["page_table"] >= 0,
                                                               perm[np.maximum(st["page_table"], 0)], -1))
    o2 = _attn(st2, q)[0]
    assert np.array_equal(o1, o2)


def test_gqa_group_mapping_against_single_head_runs():
    """Head h of a 4-head/2-group cache equals a 1-KV-head run over group h // 2."""
    w = wl.Workload("g", batch=1, num_q_heads=4, num_kv_heads=2, head_dim=16, v_dim=16, page_size=16,
                    num_pages=4, ctx_lo=20, ctx_hi=20, seed=11)
    st, k, v, lens = _cache(w, "bf16")
    q = wl.queries(w)
    o = _attn(st, q)[0]
    for h in range(4):
        g = h // 2
        ref = attention.softmax_attention(codec.f64_from_bf16(q[0, h:h + 1]), codec.f64_from_bf16(k[:, g]),
                                          codec.f64_from_bf16(v[:, g]), st["sm_scale"])
        np.testing.assert_allclose(o[h], ref[0], rtol=1e-13, atol=1e-14)


def test_aborted_and_empty_requests_give_zero_rows():
    w = wl.WORKLOADS["tiny"].with_(batch=3, num_pages=48, ctx_lo=20, ctx_hi=40)
    st, k, v, lens = _cache(w, "fp8")
    q = wl.queries(w)
    flags = np.array([0, 1, 0], dtype=np.uint32)
    lens2 = lens.copy()
    lens2[2] = 0
    st2 = dict(st, ctx_lens=lens2)
    o = _attn(st2, q, flags=flags)
    assert np.abs(o[0]).sum() > 0
    assert not o[1].any() and not o[2].any()


def test_latent_matches_gqa_formula():
    """The latent cache is one shared K of width 576 whose first 512 dims are V."""
    w = wl.Workload("lat", batch=2, num_q_heads=4, num_kv_heads=1, head_dim=24, v_dim=16, page_size=16,
                    num_pages=8, ctx_lo=30, ctx_hi=30, seed=12, latent=True)
    st, k, _, lens = _cache(w, "fp8")
    q = wl.queries(w)
    o = _attn(st, q)
    off = np.concatenate([[0], np.cumsum(lens)])
    for r in range(2):
        c = codec.e4m3_decode(codec.quantize_e4m3(k[off[r]:off[r + 1], 0], st["k_scale"])) * np.float64(st["k_scale"])
        ref = attention.softmax_attention(codec.f64_from_bf16(q[r]), c, c[:, :16], 1 / math.sqrt(24))
        np.testing.assert_allclose(o[r], ref, rtol=1e-13, atol=1e-14)


def test_decode_step_order_check_before_append():
    """The stale request is flagged, its append is skipped and its row is zero."""
    w = wl.WORKLOADS["sweep_b8"].with_(num_pages=1024, ctx_lo=50, ctx_hi=50)
    st, k, v, lens = _cache(w, "fp8")
    stale = wl.stale_requests(w)
    assert len(stale) == 1
    kp_before = st["k_pool"].copy()
    off = np.concatenate([[0], np.cumsum(lens)])
    last = off[1:] - 1
    # new token rows that differ from what is stored, to see which ones got written
    k_new = k[last] ^ np.uint16(0x0040)
    v_new = v[last]
    flags, out = step.decode_step(st, wl.queries(w), k_new, v_new, np.arange(w.batch, dtype=np.int32),
                                  lens - 1)
    assert np.flatnonzero(flags).tolist() == stale.tolist()
    r = int(stale[0])
    assert not out[r].any()
    # the flagged request's last page is untouched; another request's changed
    p_stale = st["page_table"][r, (lens[r] - 1) // w.page_size]
    assert np.array_equal(st["k_pool"][p_stale], kp_before[p_stale])
    r2 = (r + 1) % w.batch
    p2 = st["page_table"][r2, (lens[r2] - 1) // w.page_size]
    assert not np.array_equal(st["k_pool"][p2], kp_before[p2])
    # the step without a tracker writes every request and zeroes none
    flags2, out2 = step.decode_step(st, wl.queries(w), k_new, v_new, np.arange(w.batch, dtype=np.int32),
                                    lens - 1, tracker=False)
    assert flags2 is None and out2[r].any()


def test_row_rel_error_metric():
    ref = np.array([[1.0, -2.0], [0.0, 0.0]])
    got = np.array([[1.0, -1.98], [0.0, 0.0]])
    e = attention.row_rel_error(got, ref)
    np.testing.assert_allclose(e, [0.01, 0.0])
