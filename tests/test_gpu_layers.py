"""One decode step over a stack of layers through kv_decode_step_* (one launch sequence: the tag check
once, fused with layer 0's write, then every layer's write and attention; for the GQA cache, layers
after the first write the token from the attention launch), against the oracle's
multi-layer step: flags and every layer's pools bit-exact, every layer's attention within tolerance,
aborted and empty requests zero in every layer (agentlenshq summary, section "KV Cache 完整性检查":
one batched check before any read).  The same step captured in a HIP graph replays bit-identically."""
import math

import numpy as np
import pytest
import torch

import fp8_paged_kv_append_amd as kv
from kvsynth import workloads as wl
from oracle import codec, paged, step
from tests import layout
from tests.gpu_util import ATTN_TOL, attn_error, dev, host, note

pytestmark = pytest.mark.gpu

LAYERS = 3


class Stack:
    """LAYERS layers over one page table / tag set: oracle pools (numpy) and device stacks side by side."""

    def __init__(self, kv_dtype, latent, stale=(1, 6), hole=True, lens=None, splits=0):
        if latent:
            w = wl.WORKLOADS["latent"].with_(batch=9, num_q_heads=16, num_pages=400, ctx_lo=1, ctx_hi=600)
        else:
            w = wl.WORKLOADS["sweep_b16"].with_(batch=9, num_pages=2000, ctx_lo=1, ctx_hi=700)
        self.w, self.kv_dtype, self.latent = w, kv_dtype, latent
        fp8 = kv_dtype == "fp8"
        if lens is None:
            lens = wl.ctx_lens(w)
            lens[3] = 0
        else:
            lens = np.asarray(lens, dtype=np.int32)
        pt, _ = wl.page_table(w, lens)
        tags = wl.page_tags(w)
        exp = wl.expected_tags(w, pt, lens, tags, np.asarray(stale, dtype=np.int64))
        req, pos = wl.token_index(lens)
        last = np.maximum(np.cumsum(lens.astype(np.int64)) - 1, 0)
        elt = 1 if fp8 else 2
        et = np.uint8 if fp8 else np.uint16
        self.lens, self.tags, self.exp, self.et = lens, tags, exp, et
        self.desc = kv.pool_desc(w.num_pages, w.page_size, w.num_kv_heads, w.head_dim, w.v_dim)
        self.sm_scale = 1.0 / math.sqrt(w.head_dim)
        self.states, self.q, self.k_new, self.v_new = [], [], [], []
        dkp, dvp, ks_d, vs_d = [], [], [], []
        for l in range(LAYERS):
            wl_ = w.with_(seed=w.seed + 31 * (l + 1))
            k, v = wl.all_kv(wl_, lens)
            ks = codec.calibrate_scale(k) if fp8 else np.float32(1)
            vs = (ks if latent else codec.calibrate_scale(v)) if fp8 else np.float32(1)
            kp = wl.pool_init(w, "k", elt)
            vp = None if latent else wl.pool_init(w, "v", elt)
            # device: this layer's pools, the same elements in the library's layout, filled through its append
            dk_l = dev(layout.to_device(kp, "latent" if latent else "k", elt))
            dv_l = None if latent else dev(layout.to_device(vp, "v", elt))
            if fp8:
                k_s = kv.calibrate_scale(dev(k))
                v_s = k_s if latent else kv.calibrate_scale(dev(v))
                assert np.float32(k_s) == ks and np.float32(v_s) == vs
                kv.kv_append_fp8(self.desc, dk_l, dv_l, dev(k), None if latent else dev(v), dev(req), dev(pos),
                                 dev(pt), k_scale=k_s, v_scale=v_s)
            else:
                kv.kv_append_bf16(self.desc, dk_l, dv_l, dev(k), None if latent else dev(v), dev(req), dev(pos),
                                  dev(pt))
            dkp.append(dk_l)
            dvp.append(dv_l)
            ks_d.append(float(ks))
            vs_d.append(float(vs))
            # oracle: the same fill
            if fp8:
                paged.append_fp8(kp, vp, k, v, req, pos, pt, ks, vs)
            else:
                paged.append(kp, vp, k, v, req, pos, pt)
            self.states.append(dict(dtype=kv_dtype, k_pool=kp, v_pool=vp, page_table=pt, ctx_lens=lens,
                                    page_tags=tags, expected_tags=exp, num_kv_heads=w.num_kv_heads,
                                    page_size=w.page_size, head_dim=w.head_dim, v_dim=w.v_dim, k_scale=ks,
                                    v_scale=vs, sm_scale=self.sm_scale, latent=latent))
            self.q.append(wl.queries(wl_))
            self.k_new.append(k[last] ^ np.uint16(0x0040))      # differs from what is stored: a write shows
            self.v_new.append(None if latent else v[last] ^ np.uint16(0x0040))
        if hole:                                                  # a page-table hole inside a used range
            self.hole = 5
            pt[self.hole, (int(lens[self.hole]) - 1) // w.page_size // 2] = -1
        self.pt = pt
        torch.cuda.synchronize()
        self.dkp = torch.stack(dkp)
        self.dvp = None if latent else torch.stack(dvp)
        del dkp, dvp
        self.ks, self.vs = ks_d, vs_d
        self.dpt, self.dlens, self.dtags, self.dexp = dev(pt), dev(lens), dev(tags), dev(exp)
        self.dq = dev(np.stack(self.q))
        self.dk_new = dev(np.stack(self.k_new))
        self.dv_new = None if latent else dev(np.stack(self.v_new))
        self.max_ctx = int(lens.max())
        self.latent, self.elt = latent, elt
        B, Hq = w.batch, w.num_q_heads
        self.splits = splits
        if splits == 0 and latent:
            splits = kv.paged_decode_attn_latent_auto_splits(B, Hq, self.max_ctx)
        elif splits == 0:
            splits = kv.paged_decode_attn_auto_splits(B, w.num_kv_heads, self.max_ctx)
        n = kv.paged_decode_attn_workspace_bytes(B, Hq, w.v_dim, splits)
        self.ws = torch.zeros(max(n, 16) // 4 + 4, dtype=torch.float32, device="cuda")
        self.out = torch.empty((LAYERS, B, Hq, w.v_dim), dtype=torch.int16, device="cuda")
        self.flags = torch.full((B,), -1, dtype=torch.int32, device="cuda")

    def layer_pools_match(self, l):
        """Layer l's device pools, mapped to logical order, equal the oracle's element by element."""
        st = self.states[l]
        k = layout.from_device(host(self.dkp[l], self.et), "latent" if self.latent else "k", st["k_pool"].shape,
                               self.elt)
        if not np.array_equal(k, st["k_pool"]):
            return False
        if self.latent:
            return True
        v = layout.from_device(host(self.dvp[l], self.et), "v", st["v_pool"].shape, self.elt)
        return np.array_equal(v, st["v_pool"])

    def run(self, tracker=True, fused=False):
        kv.decode_step_layers(self.desc, self.kv_dtype, self.dkp, self.dvp, self.dpt, self.dlens, self.max_ctx,
                              self.dq, self.dk_new, self.dv_new, self.out,
                              page_tags=self.dtags if tracker else None, expected_tags=self.dexp if tracker else None,
                              abort_flags=self.flags if tracker else None,
                              k_scales=self.ks if self.kv_dtype == "fp8" else None,
                              v_scales=self.vs if self.kv_dtype == "fp8" and not self.latent else None,
                              sm_scale=self.sm_scale, num_splits=self.splits, workspace=self.ws, fused_check=fused)

    def oracle(self, tracker=True):
        B = self.w.batch
        return step.decode_step_layers(self.states, self.q, self.k_new, self.v_new, np.arange(B, dtype=np.int32),
                                       (self.lens - 1).astype(np.int32), tracker=tracker)


@pytest.mark.parametrize("fused", [False, True])
@pytest.mark.parametrize("latent", [False, True])
@pytest.mark.parametrize("kv_dtype", ["fp8", "bf16"])
def test_layer_stack_step_matches_oracle(kv_dtype, latent, fused):
    """The step over a layer stack with the tag check as its own launch (default) or inside layer 0's
    attention launch (fused): flags, every layer's pools and rows against the oracle's multi-layer step."""
    note(f"layer stack {kv_dtype} latent={latent} fused={fused}")
    s = Stack(kv_dtype, latent)
    s.run(fused=fused)
    torch.cuda.synchronize()
    o_flags, o_outs = s.oracle()
    g_flags = host(s.flags, np.uint32)
    assert np.array_equal(g_flags, o_flags)
    assert g_flags[1] and g_flags[6] and g_flags[s.hole] == paged.FLAG_BAD_PAGE and not g_flags[3]
    g_out = host(s.out, np.uint16)
    for l in range(LAYERS):
        assert s.layer_pools_match(l), l
        err = attn_error(g_out[l], o_outs[l])
        note(f"  layer {l}: error {err:.3e}")
        assert err <= ATTN_TOL
        for r in np.flatnonzero(o_flags).tolist() + [3]:
            assert not g_out[l, r].any()


@pytest.mark.parametrize("latent", [False, True])
@pytest.mark.parametrize("splits", [1, 4])
@pytest.mark.parametrize("kv_dtype", ["fp8", "bf16"])
def test_layer_stack_token_at_chunk_edges(kv_dtype, splits, latent):
    """Layers after the first write the step's token from their attention launch, in the block(s) whose
    split holds position L - 1 (GQA: added from LDS; latent: stored before the tile copies and read
    back).  Lengths put that position alone in its split (129, 257, 385 with 128-token splits), last in
    one (128, 512), first of the context (L = 1) and mid-tile; pools bit-exact and outputs within
    tolerance in every layer.  Latent FP8 runs the wave-pair kernel here, latent BF16 the 128-head one."""
    note(f"layer stack chunk edges {kv_dtype} splits={splits} latent={latent}")
    lens = [1, 129, 0, 128, 512, 385, 64, 65, 257]
    s = Stack(kv_dtype, latent, stale=(6,), hole=False, lens=lens, splits=splits)
    s.run()
    torch.cuda.synchronize()
    o_flags, o_outs = s.oracle()
    assert np.array_equal(host(s.flags, np.uint32), o_flags)
    g_out = host(s.out, np.uint16)
    for l in range(LAYERS):
        assert s.layer_pools_match(l), l
        err = attn_error(g_out[l], o_outs[l])
        note(f"  layer {l}: error {err:.3e}")
        assert err <= ATTN_TOL
        assert not g_out[l, 6].any() and not g_out[l, 2].any()


@pytest.mark.parametrize("latent", [False, True])
@pytest.mark.parametrize("kv_dtype", ["fp8", "bf16"])
def test_layer_stack_no_op_tracker(kv_dtype, latent):
    """page_tags None: no check, nothing flagged; stale requests are written and attended in every layer."""
    note(f"layer stack no-op tracker {kv_dtype} latent={latent}")
    s = Stack(kv_dtype, latent, hole=False)
    s.run(tracker=False)
    torch.cuda.synchronize()
    o_flags, o_outs = s.oracle(tracker=False)
    assert o_flags is None
    g_out = host(s.out, np.uint16)
    for l in range(LAYERS):
        assert s.layer_pools_match(l), l
        assert attn_error(g_out[l], o_outs[l]) <= ATTN_TOL
        assert g_out[l, 1].any() and g_out[l, 6].any()


@pytest.mark.parametrize("kv_dtype,latent,fused", [("fp8", False, False), ("bf16", False, False),
                                                   ("fp8", True, False), ("fp8", False, True)])
def test_layer_stack_graph_replays_match_eager(kv_dtype, latent, fused):
    note(f"layer stack graph {kv_dtype} latent={latent} fused={fused}")
    s = Stack(kv_dtype, latent)
    s.run(fused=fused)
    torch.cuda.synchronize()
    want_out, want_flags, want_k = s.out.clone(), s.flags.clone(), s.dkp.clone()
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        s.run(fused=fused)
    torch.cuda.current_stream().wait_stream(side)
    with torch.cuda.graph(g):
        s.run(fused=fused)
    junk = torch.empty(1 << 20, dtype=torch.float32, device="cuda")
    for i in range(4):
        s.out.fill_(0x5555)
        s.flags.fill_(-1)
        junk.normal_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(s.out, want_out), i
        assert torch.equal(s.flags, want_flags), i
        assert torch.equal(s.dkp, want_k), i
