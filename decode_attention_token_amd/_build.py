"""Builds libkvq.so in-tree with hipcc for gfx950."""
from __future__ import annotations

import os
import shutil
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libkvq.so")

SOURCES = ["kvq_api.cpp", "kvq_quant.hip", "kvq_attn.hip", "kvq_attn_gqa.hip", "kvq_innerq.hip", "kvq_probe.hip",
           "kvq_noalloc.hip"]

# -packed-fp32-ops keeps the compiler from forming packed fp32 arithmetic;
# correctly rounded fp32 division (the hipcc default) is required for the
# bit-exact quantizer, so no fast-math flags appear here.
# The atomic optimizer is off: it rewrites a work-queue ticket grab into a
# read of the result right after the atomic, behind a wait for every load in
# flight, while the kernels read a ticket a whole super-chunk later.
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-mllvm", "-amdgpu-atomic-optimizer-strategy=None",
    "-Wno-unused-command-line-argument",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found; a ROCm toolchain is required to build libkvq")


def build(extra_flags=(), out=LIB, verbose=False) -> str:
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    tmp = out + ".tmp"
    cmd = [hipcc(), *FLAGS, *extra_flags, "-I", os.path.join(ROOT, "include"), "-o", tmp, *srcs]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + res.stdout + res.stderr)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
