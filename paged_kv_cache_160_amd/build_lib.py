"""Build libpagedkv.so in-tree with hipcc for gfx950.

    python -m paged_kv_cache_160_amd.build_lib        # or __graft_entry__.build()
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
REPO = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
INCLUDE = os.path.join(REPO, "include")
LIB_NAME = "libpagedkv.so"
LIB_PATH = os.path.join(PKG_DIR, LIB_NAME)

SOURCES = ["api.cpp", "allocator.cpp", "cache_write.hip", "decode.hip", "prefill.hip", "noalloc.hip"]
ARCH = os.environ.get("PKV_OFFLOAD_ARCH", "gfx950")

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-Wall",
    # packed fp32 arithmetic stays off for all device code on this hardware
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-fno-gpu-flush-denormals-to-zero",
    # every symbol resolved at link time: a kernel whose host-side launch stub
    # the compiler failed to emit is a build error, not a load-time one
    "-Wl,-z,defs",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def build(verbose: bool = False, extra_flags=None, out: str = LIB_PATH) -> str:
    """Compile every source into ``out`` (LIB_PATH by default; always
    recompiles).  ``extra_flags`` such as ``-DPKV_DECODE_QK_VALU=1`` select
    the measured alternatives the kernels keep as build options."""
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    tmp = out + ".tmp"
    cmd = [hipcc(), *HIPCC_FLAGS, *(extra_flags or []), "-I", INCLUDE, "-I", CSRC, *srcs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass warns that it does not know the packed-fp32 feature
    noise = "is not a recognized feature for this target"
    msgs = [ln for ln in (res.stdout + res.stderr).splitlines() if noise not in ln]
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(msgs))
    if verbose and msgs:
        print("\n".join(msgs))
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    import argparse
    ap = argparse.ArgumentParser(description="build libpagedkv.so for gfx950")
    ap.add_argument("-v", action="store_true", help="print the hipcc command")
    ap.add_argument("--define", action="append", default=[], metavar="NAME=VALUE",
                    help="a kernel build option, e.g. PKV_DECODE_QK_VALU=1 (a variant library; use --out)")
    ap.add_argument("--out", default=LIB_PATH, help="library path (default: the package's libpagedkv.so)")
    args = ap.parse_args()
    print(build(verbose=args.v, extra_flags=[f"-D{d}" for d in args.define], out=os.path.abspath(args.out)))
