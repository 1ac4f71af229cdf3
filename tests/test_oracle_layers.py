"""The oracle's multi-layer step (CPU): layers that share one page table and one set of tags take one
tag check, and its outcome holds in every layer (agentlenshq summary, section "KV Cache 完整性检查": a
stale request is aborted before anything reads the cache).  Pins: a stale request is zero and its
new token is written in no layer; permuting the layers permutes the results; with nothing stale each
layer equals the single-layer step (itself pinned by closed forms and brute force)."""
import math

import numpy as np
import pytest

from kvsynth import workloads as wl
from oracle import codec, paged, step

L = 3


def _states(kv_dtype, stale):
    w = wl.WORKLOADS["tiny"].with_(batch=4, num_pages=60, ctx_lo=20, ctx_hi=150, seed=5)
    lens = wl.ctx_lens(w)
    pt, _ = wl.page_table(w, lens)
    tags = wl.page_tags(w)
    exp = wl.expected_tags(w, pt, lens, tags, np.asarray(stale, dtype=np.int64))
    req, pos = wl.token_index(lens)
    last = np.cumsum(lens.astype(np.int64)) - 1
    elt = 1 if kv_dtype == "fp8" else 2
    states, qs, kns, vns = [], [], [], []
    for l in range(L):
        wl_ = w.with_(seed=w.seed + 17 * (l + 1))
        k, v = wl.all_kv(wl_, lens)
        ks = codec.calibrate_scale(k) if elt == 1 else np.float32(1)
        vs = codec.calibrate_scale(v) if elt == 1 else np.float32(1)
        kp, vp = wl.pool_init(w, "k", elt), wl.pool_init(w, "v", elt)
        if elt == 2:
            paged.append(kp, vp, k, v, req, pos, pt)
        else:
            paged.append_fp8(kp, vp, k, v, req, pos, pt, ks, vs)
        states.append(dict(dtype=kv_dtype, k_pool=kp, v_pool=vp, page_table=pt, ctx_lens=lens, page_tags=tags,
                           expected_tags=exp, num_kv_heads=w.num_kv_heads, page_size=w.page_size,
                           head_dim=w.head_dim, v_dim=w.v_dim, k_scale=ks, v_scale=vs,
                           sm_scale=1 / math.sqrt(w.head_dim), latent=False))
        qs.append(wl.queries(wl_))
        kns.append(k[last] ^ np.uint16(0x0100))          # differs from what is stored
        vns.append(v[last] ^ np.uint16(0x0100))
    return states, qs, kns, vns, np.arange(w.batch, dtype=np.int32), (lens - 1).astype(np.int32)


@pytest.mark.parametrize("kv_dtype", ["fp8", "bf16"])
def test_stale_request_untouched_in_every_layer(kv_dtype):
    states, qs, kns, vns, req, pos = _states(kv_dtype, stale=[2])
    before = [(s["k_pool"].copy(), s["v_pool"].copy()) for s in states]
    flags, outs = step.decode_step_layers(states, qs, kns, vns, req, pos)
    assert flags.tolist() == [0, 0, paged.FLAG_TAG_MISMATCH, 0]
    S = states[0]["page_size"]
    pt, lens = states[0]["page_table"], states[0]["ctx_lens"]
    for s, (k0, v0), o in zip(states, before, outs):
        assert not o[2].any()
        changed_pages = np.flatnonzero((s["k_pool"] != k0).any(axis=(1, 2, 3)))
        assert changed_pages.size > 0                     # the other requests' tokens went in
        # nothing changed in request 2's pages
        own = sorted(set(pt[2, :(int(lens[2]) + S - 1) // S].tolist()))
        assert not (set(changed_pages.tolist()) & set(own))
        assert np.array_equal(s["v_pool"][own], v0[own])


def test_layer_permutation_permutes_results():
    a = _states("fp8", stale=[1])
    b = _states("fp8", stale=[1])
    perm = [2, 0, 1]
    fa, oa = step.decode_step_layers(*a)
    states, qs, kns, vns, req, pos = b
    fb, ob = step.decode_step_layers([states[i] for i in perm], [qs[i] for i in perm], [kns[i] for i in perm],
                                     [vns[i] for i in perm], req, pos)
    assert np.array_equal(fa, fb)
    for j, i in enumerate(perm):
        for r in oa[i]:
            assert np.array_equal(oa[i][r], ob[j][r])
        assert np.array_equal(a[0][i]["k_pool"], states[i]["k_pool"])


@pytest.mark.parametrize("tracker", [True, False])
def test_each_layer_equals_the_single_layer_step(tracker):
    a = _states("bf16", stale=[] if tracker else [3])
    b = _states("bf16", stale=[] if tracker else [3])
    fa, oa = step.decode_step_layers(*a, tracker=tracker)
    states, qs, kns, vns, req, pos = b
    for l in range(L):
        f1, o1 = step.decode_step(states[l], qs[l], kns[l], vns[l], req, pos, tracker=tracker)
        if tracker:
            assert np.array_equal(fa, f1)
        else:
            assert fa is None and f1 is None
        assert np.array_equal(a[0][l]["k_pool"], states[l]["k_pool"])
        for r in o1:
            assert np.array_equal(oa[l][r], o1[r])
