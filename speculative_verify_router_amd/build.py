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
import time

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIBDIR = os.path.join(PKG, "lib")
LIB = os.path.join(LIBDIR, "libsvr_moe.so")
# Translation units, compiled in parallel (the expert-kernel families are
# split out of moe_layer.hip so that no one unit holds every instantiation).
SOURCES = [os.path.join(CSRC, f) for f in (
    "moe_layer.hip", "launch_expert.hip", "launch_ffn.hip", "launch_ffn_q8_0.hip",
    "launch_ffn_q4_k.hip", "launch_ffn_q2_k.hip", "launch_ffn_q3_k.hip", "launch_ffn_q6_k.hip",
    "accept.hip")]
HEADERS = [os.path.join(CSRC, f) for f in ("common.h", "quant.h", "route.h", "ffn.h", "phases.h", "misc.h",
                                           "gemm.h", "launch.h", "launch_ffn.h")] + [
    os.path.join(ROOT, "include", h) for h in ("moe_layer.h", "moe_accept.h")]

ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the HIP library)")


def compile_flags(extra=()) -> list:
    return [
        "-O3", "-std=c++17", f"--offload-arch={ARCH}", "-fPIC",
        # No packed-FP32 instructions anywhere in the device code.
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        # MFMA results straight into VGPRs (no AGPR round trip).
        "-mllvm", "-amdgpu-mfma-vgpr-form",
        "-Wno-unused-command-line-argument",
        "-I", os.path.join(ROOT, "include"), "-I", CSRC, *extra,
    ]


def _report(res, what: str, verbose: bool) -> None:
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"{what} failed with status {res.returncode}")
    if verbose and res.stderr.strip():
        # hipcc's host pass warns that it does not know the packed-fp32 feature.
        lines = [l for l in res.stderr.splitlines() if "packed-fp32-ops" not in l]
        if lines:
            sys.stderr.write("\n".join(lines) + "\n")


def build(verbose: bool = False, extra=()) -> str:
    objdir = os.path.join(LIBDIR, "obj")
    os.makedirs(objdir, exist_ok=True)
    objs, procs = [], []
    t0 = time.time()
    for src in SOURCES:
        obj = os.path.join(objdir, os.path.splitext(os.path.basename(src))[0] + ".o")
        cmd = [hipcc(), *compile_flags(extra), "-c", "-o", obj, src]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append(subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True))
        objs.append(obj)
    for src, p in zip(SOURCES, procs):
        out, err = p.communicate()
        _report(subprocess.CompletedProcess(p.args, p.returncode, out, err), f"hipcc {src}", verbose)
        if verbose:
            print(f"# {os.path.basename(src)} compiled by {time.time() - t0:.0f} s", flush=True)
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    _report(subprocess.run(cmd, capture_output=True, text=True), "link", verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
