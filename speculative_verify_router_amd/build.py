"""Compile the HIP library for gfx950 in-tree.

    python -m speculative_verify_router_amd.build

writes ``speculative_verify_router_amd/lib/libsvr_moe.so``.  hipcc
cross-compiles, so this works on a host without a GPU.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIBDIR = os.path.join(PKG, "lib")
LIB = os.path.join(LIBDIR, "libsvr_moe.so")
SOURCES = [os.path.join(CSRC, "moe_layer.hip"), os.path.join(CSRC, "accept.hip")]
HEADERS = [os.path.join(CSRC, f) for f in ("common.h", "quant.h", "route.h", "ffn.h", "phases.h", "misc.h",
                                           "flow.h", "gemm.h")] + [
    os.path.join(ROOT, "include", h) for h in ("moe_layer.h", "moe_accept.h")]

ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the HIP library)")


def compile_flags(extra=()) -> list:
    return [
        "-O3", "-std=c++17", f"--offload-arch={ARCH}", "-fPIC", "-shared",
        # No packed-FP32 instructions anywhere in the device code.
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        # MFMA results straight into VGPRs (no AGPR round trip).
        "-mllvm", "-amdgpu-mfma-vgpr-form",
        "-Wno-unused-command-line-argument",
        "-I", os.path.join(ROOT, "include"), "-I", CSRC, *extra,
    ]


def build(verbose: bool = False, extra=()) -> str:
    os.makedirs(LIBDIR, exist_ok=True)
    tmp = LIB + ".tmp"
    cmd = [hipcc(), *compile_flags(extra), "-o", tmp, *SOURCES]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed with status {res.returncode}")
    if verbose and res.stderr.strip():
        # hipcc's host pass warns that it does not know the packed-fp32 feature.
        lines = [l for l in res.stderr.splitlines() if "packed-fp32-ops" not in l]
        if lines:
            sys.stderr.write("\n".join(lines) + "\n")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
