"""The allocation-free attention entry point, paged_decode_attn_fp8_noalloc (the split partials in the
library's own device scratch), against paged_decode_attn_fp8 with a caller workspace: identical bits on
the same inputs, over two calls in a row, the second on a smaller batch, with several split counts and
an aborted request; and a split count whose partials exceed the scratch refused with a status."""
import numpy as np
import pytest
import torch

import fp8_paged_kv_append_amd as kv
from kvsynth import workloads as wl
from tests.gpu_util import ATTN_TOL, Case, attn_error, dev, host, note

pytestmark = pytest.mark.gpu


def _noalloc(c, num_splits, flags=None):
    out = c.out_tensor()
    kv.paged_decode_attn_fp8_noalloc(c.desc, c.dq, c.dkp, c.dvp, c.dpt, c.dlens, c.max_ctx, out, flags,
                                     k_scale=c.d_k_scale, v_scale=c.d_v_scale, sm_scale=c.sm_scale,
                                     num_splits=num_splits)
    torch.cuda.synchronize()
    return host(out, np.uint16)


def test_noalloc_matches_the_workspace_entry_point():
    base = wl.WORKLOADS["gqa_batch"].with_(num_pages=1500)
    big = Case(base.with_(batch=6, ctx_lo=1, ctx_hi=1500), "fp8",
               lens=np.array([1, 15, 17, 700, 1500, 333], dtype=np.int32))
    big.fill_device()
    for splits in (3, 0, 1, 24):
        note(f"no-alloc, 6 requests, splits={splits}")
        want = big.attend(num_splits=splits)
        got = _noalloc(big, splits)
        assert np.array_equal(got, want), splits
        assert attn_error(got, big.oracle_attend()) <= ATTN_TOL
    # a second call on a smaller batch right after: its own bits, not the first call's leftovers
    small = Case(base.with_(batch=2, ctx_lo=1, ctx_hi=900, seed=7), "fp8", lens=np.array([900, 65], dtype=np.int32))
    small.fill_device()
    fl = dev(np.array([0, 1], dtype=np.uint32))
    for splits in (2, 7):
        note(f"no-alloc, 2 requests, splits={splits}")
        want = small.attend(flags=fl, num_splits=splits)
        got = _noalloc(small, splits, flags=fl)
        assert np.array_equal(got, want), splits
        assert not got[1].any() and got[0].any()


def test_noalloc_refuses_partials_beyond_its_scratch():
    B, Hq, D = 64, 64, 128
    desc = kv.pool_desc(16, 16, 8, D, D)
    q = torch.zeros((B, Hq, D), dtype=torch.int16, device="cuda")
    pool = torch.zeros(16 * 8 * 16 * D, dtype=torch.uint8, device="cuda")
    pt = torch.zeros((B, 16), dtype=torch.int32, device="cuda")
    lens = torch.ones(B, dtype=torch.int32, device="cuda")
    out = torch.empty((B, Hq, D), dtype=torch.int16, device="cuda")
    with pytest.raises(kv.KvFp8Error) as e:
        kv.paged_decode_attn_fp8_noalloc(desc, q, pool, pool, pt, lens, 256, out, k_scale=1.0, v_scale=1.0,
                                         num_splits=4)
    assert e.value.status == -4
    torch.cuda.synchronize()
