"""Compile the HIP library libgdn.so for gfx950 (in-tree, next to this file).

Run as ``python -m gated_delta_rule_bwd_amd.build``; ``__graft_entry__.build()`` calls
``build()``.  hipcc cross-compiles without a GPU present.
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libgdn.so")
SOURCES = ["gdn_api.hip", "gdn_kernels.hip", "gdn_mf.hip", "ssm_conv.hip", "l2norm.hip",
           "ssm_scan.hip", "ssm_chunk.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    # packed FP32 instructions are kept out of every kernel on this hardware
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-fno-fast-math", "-Wall",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
]


def build(extra_flags=(), out=LIB, verbose=False) -> str:
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    tmp = f"{out}.tmp{os.getpid()}"
    cmd = [HIPCC, *FLAGS, *extra_flags, *srcs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass does not know the device-only feature name; that warning is harmless
    err = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed ({r.returncode}):\n{err}")
    if err.strip() and verbose:
        print(err, file=sys.stderr)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
