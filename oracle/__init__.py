"""CPU oracle for paged decode attention over an FP8 (e4m3) or BF16 KV cache.

TEST INFRASTRUCTURE.  This package is the plain, slow, obviously correct
reference that the GPU library is checked against.  Only the test suite,
the smoke check in __graft_entry__ and the CPU-baseline leg of bench.py may
import it; the library itself never does, and the oracle imports nothing
from the library.  It shares no code with the GPU path: its inputs come from
the seeded generator in kvsynth, which holds no arithmetic of the method.

What it computes is fixed by the pages this work follows:

* the Cloudflare blog post "Smaller, faster, safer: running Kimi and GLM at
  scale", section "Quantized KV cache": K and V are stored as FP8 e4m3 in
  place of BF16 and the attention kernel converts them as it reads them;
* the agentlenshq summary of that post, section "KV Cache 完整性检查", and the
  xujun.org note on it, section "一个不能出错的共享缓存": every physical page
  carries a tag that changes when the page is reallocated, the server keeps
  each request's expected (page, tag) list, checks it in one batched pass
  before decode reads the cache, and aborts the request on a mismatch;
* the zdabc.icu article, section "显存为什么会成为长上下文推理的瓶颈":
  KV bytes = requests x tokens x layers x KV heads x head_dim x 2 x bytes/element.

Where the pages are silent (which e4m3, rounding, overflow, scale, layout,
flag bits) the readings are listed in the module docstrings that use them.
Floating point is fp64 except where a step is defined in fp32 (the scale,
its reciprocal and the product x*inv that is encoded).

Parity pins: every function here is checked by tests/test_oracle_*.py
against something other than itself (closed forms, brute force, library
routines, planted faults).  No function here is "parity unpinned".
"""
from . import codec, paged, attention, step  # noqa: F401
