"""A decode step captured in a HIP graph replays bit-identically to the eager step.

The step (tag check -> append -> attention, split count > 1 so the merge
kernel is in the graph too) is captured once, then replayed several times
with unrelated eager device work and synchronisations between replays;
every replay's flags, output and pools must equal the eager step's.
"""
import numpy as np
import pytest
import torch

import fp8_paged_kv_append_amd as kv
from kvsynth import workloads as wl
from tests.gpu_util import Case, dev, host, note

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("kv_dtype", ["fp8", "bf16"])
@pytest.mark.parametrize("splits", [1, 3])
def test_step_graph_replays_match_eager(kv_dtype, splits):
    w = wl.WORKLOADS["sweep_b16"].with_(num_pages=3000, ctx_lo=700, ctx_hi=700)
    note(f"graph replay {kv_dtype} splits={splits}")
    c = Case(w, kv_dtype, oracle_fill=False)
    c.fill_device()
    k_new, v_new, req, pos = c.step_inputs()
    dk_new, dv_new, dreq, dpos = dev(k_new), dev(v_new), dev(req), dev(pos)
    out = c.out_tensor()
    flags = torch.zeros(w.batch, dtype=torch.int32, device="cuda")
    ws = c.workspace(splits)

    def step():
        kv.decode_step(c.desc, kv_dtype, c.dkp, c.dvp, c.dpt, c.dlens, c.max_ctx, c.dq, dk_new, dv_new, dreq, dpos,
                       out, page_tags=c.dtags, expected_tags=c.dexp, abort_flags=flags, k_scale=c.d_k_scale,
                       v_scale=c.d_v_scale, sm_scale=c.sm_scale, num_splits=splits, workspace=ws)

    step()
    torch.cuda.synchronize()
    want_out, want_flags = out.clone(), flags.clone()
    want_k, want_v = c.dkp.clone(), c.dvp.clone()
    assert host(want_flags, np.uint32).any()

    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    with torch.cuda.graph(g):
        step()
    junk = torch.empty(1 << 20, dtype=torch.float32, device="cuda")
    for i in range(4):
        out.fill_(0x5555)
        flags.fill_(-1)
        junk.normal_()                                     # unrelated eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, want_out), i
        assert torch.equal(flags, want_flags), i
        assert torch.equal(c.dkp, want_k) and torch.equal(c.dvp, want_v), i
