"""Build libkvfp8.so (the gfx950 HIP kernels and the C ABI) in-tree with hipcc.

    python -m fp8_paged_kv_append_amd.build [--verbose]
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libkvfp8.so")

SOURCES = ["api.hip", "kv_small.hip", "attn_gqa.hip", "attn_latent.hip", "attn_latent_pairs.hip", "page_alloc.hip",
           "wgemm.hip", "read_stream.hip"]
ARCH = os.environ.get("KVFP8_ARCH", "gfx950")


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm is required to build libkvfp8.so)")


def flags() -> list:
    return [
        f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
        # packed fp32 VALU ops are kept out of the generated code
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-Wall", "-Wno-unused-function",
        f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}",
    ]


def build(verbose: bool = False, extra: list | None = None, out: str | None = None) -> str:
    """Compile every source into libkvfp8.so (or `out`), with `extra` hipcc flags appended."""
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    target = out or LIB
    tmp = target + ".tmp"
    cmd = [hipcc()] + flags() + (extra or []) + srcs + ["-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed ({r.returncode}):\n{r.stdout}\n{r.stderr}")
    if verbose and r.stderr.strip():
        print(r.stderr, file=sys.stderr)
    os.replace(tmp, target)
    return target


# Host-code sanitizers (AddressSanitizer, UndefinedBehaviorSanitizer) on the CPU side only: the device code
# is compiled as usual.  The result needs the clang ASan runtime preloaded into the process that loads it.
HOST_SANITIZER_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                        "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-shared-libsan", "-g"]


if __name__ == "__main__":
    print(build(verbose="--verbose" in sys.argv))
