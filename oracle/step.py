"""One decode step of one attention layer, composed from the oracle's parts (test infrastructure).

Order, as the integrity-check passages describe it (agentlenshq summary,
section "KV Cache 完整性检查"; xujun.org note, section "一个不能出错的共享缓存"):
the batched tag check runs first and on its own, before anything reads the
cache; the new token of every surviving request is then quantised and
written (the write touches the request's own last page, which the check
covered); then attention reads the pages.  With no tracker (the "no-op
tracker" of the xujun.org note) the check is skipped and flags are None.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

from . import attention, codec, paged


def decode_step(state, q_bits, k_new_bits, v_new_bits, tok_req, tok_pos, *, tracker=True, workers=1,
                requests=None):
    """Run tag check -> append -> attention on `state` (a dict holding the cache; pools updated in place).

    state keys: dtype ("fp8"|"bf16"), k_pool, v_pool, page_table, ctx_lens, page_tags,
    expected_tags, num_kv_heads, page_size, head_dim, v_dim, k_scale, v_scale,
    sm_scale, latent.
    Returns (flags or None, {r: fp64 [Hq][Dv]}).
    """
    s = state
    flags = None
    if tracker:
        flags = paged.tag_check(s["page_tags"], s["page_table"], s["expected_tags"], s["ctx_lens"],
                                s["page_size"])
    if s["dtype"] == "fp8":
        paged.append_fp8(s["k_pool"], s["v_pool"], k_new_bits, v_new_bits, tok_req, tok_pos,
                         s["page_table"], s["k_scale"], s["v_scale"], flags)
    else:
        paged.append(s["k_pool"], s["v_pool"], k_new_bits, v_new_bits, tok_req, tok_pos, s["page_table"],
                     flags)
    B = q_bits.shape[0]
    reqs = list(range(B)) if requests is None else list(requests)

    def one(r):
        return attention.decode_attention(
            q_bits, s["k_pool"], s["v_pool"], s["page_table"], s["ctx_lens"],
            num_kv_heads=s["num_kv_heads"], page_size=s["page_size"], head_dim=s["head_dim"],
            v_dim=s["v_dim"], dtype=s["dtype"], k_scale=s["k_scale"], v_scale=s["v_scale"],
            sm_scale=s["sm_scale"], flags=flags, requests=[r], latent=s.get("latent", False))[r]

    if workers <= 1:
        out = {r: one(r) for r in reqs}
    else:
        with ThreadPoolExecutor(min(workers, os.cpu_count() or 1)) as ex:
            out = dict(zip(reqs, ex.map(one, reqs)))
    return flags, out


def decode_step_layers(states, q_bits, k_new_bits, v_new_bits, tok_req, tok_pos, *, tracker=True):
    """One decode step over several attention layers that share the page table, the page tags and the
    context lengths (one page id names the same logical slot in every layer's pool).

    The check runs once, first, over the shared pages, so it covers every read of the step (the
    passages place it before any read, as its own batched pass); each layer then writes its new token
    and attends with those flags.  states: one state dict per layer (see decode_step) whose page_table,
    ctx_lens, page_tags and expected_tags are the same arrays; q_bits, k_new_bits, v_new_bits: one per
    layer (v_new_bits entries None for the latent cache).  Returns (flags or None, [{r: fp64 [Hq][Dv]}
    per layer]).
    """
    s0 = states[0]
    flags = None
    if tracker:
        flags = paged.tag_check(s0["page_tags"], s0["page_table"], s0["expected_tags"], s0["ctx_lens"],
                                s0["page_size"])
    outs = []
    for s, q, kn, vn in zip(states, q_bits, k_new_bits, v_new_bits):
        if s["dtype"] == "fp8":
            paged.append_fp8(s["k_pool"], s["v_pool"], kn, vn, tok_req, tok_pos, s["page_table"],
                             s["k_scale"], s["v_scale"], flags)
        else:
            paged.append(s["k_pool"], s["v_pool"], kn, vn, tok_req, tok_pos, s["page_table"], flags)
        outs.append(attention.decode_attention(
            q, s["k_pool"], s["v_pool"], s["page_table"], s["ctx_lens"], num_kv_heads=s["num_kv_heads"],
            page_size=s["page_size"], head_dim=s["head_dim"], v_dim=s["v_dim"], dtype=s["dtype"],
            k_scale=s["k_scale"], v_scale=s["v_scale"], sm_scale=s["sm_scale"], flags=flags,
            latent=s.get("latent", False)))
    return flags, outs


def output_bf16(o_f64):
    """The step's bf16 output: fp64 -> fp32 -> bf16 (round to nearest even at each step)."""
    return codec.bf16_from_f32(np.asarray(o_f64, dtype=np.float64).astype(np.float32))
