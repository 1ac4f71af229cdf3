"""The library's host code (argument checks of every entry point, the page allocator over a caller-owned
buffer) under AddressSanitizer and UndefinedBehaviorSanitizer, on the CPU: the library is rebuilt with the
host-side sanitizers, and the allocator-parity, C-ABI and capacity tests run against it in a process with
the ASan runtime preloaded.  A short host buffer handed to the allocator must be reported, which shows the
sanitizer is live."""
import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
RUNTIME = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))


@pytest.fixture(scope="module")
def sanitized(tmp_path_factory):
    from fp8_paged_kv_append_amd import build
    if not RUNTIME:
        pytest.skip("no clang ASan runtime")
    try:
        build.hipcc()
    except RuntimeError:
        pytest.skip("no hipcc")
    out = str(tmp_path_factory.mktemp("san") / "libkvfp8_san.so")
    build.build(extra=build.HOST_SANITIZER_FLAGS + ["-O1"], out=out)
    env = dict(os.environ, KVFP8_LIB=out, LD_PRELOAD=RUNTIME[-1],
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1", UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    return env


def test_host_code_is_clean_under_asan_and_ubsan(sanitized):
    tests = [os.path.join(ROOT, "tests", t) for t in ("test_alloc_parity.py", "test_abi.py", "test_capacity.py")]
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider", *tests], cwd=ROOT,
                       env=sanitized, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]
    assert "passed" in r.stdout


def test_the_sanitizer_reports_a_short_host_buffer(sanitized):
    code = ("import numpy as np\n"
            "import fp8_paged_kv_append_amd as kv\n"
            "a = kv.PageAllocator(4096)\n"
            "short = np.zeros(8, dtype=np.uint32)\n"
            "kv.lib().kv_page_alloc_tags(a._state.ctypes.data, short.ctypes.data)\n")
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=sanitized, capture_output=True, text=True,
                       timeout=120)
    assert r.returncode != 0 and "AddressSanitizer" in r.stderr, r.stderr[-2000:]
