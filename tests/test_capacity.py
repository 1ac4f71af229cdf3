"""Fixed-budget admission through the library's page allocator (host code, no GPU): the FP8 cache
holds about twice the tokens of the BF16 cache in the same bytes, minus what the per-page tag and
page-table words cost (agentlenshq summary of the Cloudflare post, opening section: the freed memory
buys concurrency, not speed)."""
import os
import sys

import numpy as np
import pytest

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))

kv = pytest.importorskip("fp8_paged_kv_append_amd")
import bench  # noqa: E402
from kvsynth import workloads as wl  # noqa: E402


def _lib_or_skip():
    try:
        kv.lib()
    except RuntimeError as e:
        pytest.skip(str(e))


@pytest.mark.parametrize("ref", [1, 3, 8])
def test_admission_fp8_vs_bf16(ref):
    _lib_or_skip()
    w = wl.WORKLOADS["sweep_b64"].with_(stale=False, ctx_lo=1000, ctx_hi=1000)
    S, need = w.page_size, -(-1000 // w.page_size)
    elem = S * w.num_kv_heads * (w.head_dim + w.v_dim)
    budget = ref * need * (2 * elem + 12)
    b = bench.capacity_admission(kv, w, "bf16", budget)
    f = bench.capacity_admission(kv, w, "fp8", budget)
    assert b["admitted"] == ref and b["pages_left"] == 0
    # FP8 pages cost elem + 12 bytes: floor((budget - 8) / (elem + 12)) pages, then whole requests
    pf = (budget - 8) // (elem + 12)
    assert f["num_pages"] == pf and f["admitted"] == pf // need and f["pages_left"] == pf - (pf // need) * need
    assert 2 * ref - 1 <= f["admitted"] <= 2 * ref
    for a in (b, f):
        t = a["page_table"]
        assert t.shape == (a["admitted"], need)
        assert len(np.unique(t)) == t.size and t.min() >= 0 and t.max() < a["num_pages"]
        # churned once (every page allocated), then the admitted pages allocated again
        want = np.ones(a["num_pages"], dtype=np.uint32)
        want[t.ravel()] = 2
        assert np.array_equal(a["tags"], want)


def test_admission_empty_budget():
    _lib_or_skip()
    w = wl.WORKLOADS["sweep_b64"].with_(stale=False)
    elem = w.page_size * w.num_kv_heads * (w.head_dim + w.v_dim)
    a = bench.capacity_admission(kv, w, "bf16", 10 * (2 * elem + 12))   # 10 pages: less than one request
    assert a["admitted"] == 0 and a["page_table"].shape == (0, 512) and a["pages_left"] == 10
