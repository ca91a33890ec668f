"""Barrier structure of the single-launch kernel, checked in its gfx950 assembly.

Each workgroup of k_flow must pass every barrier exactly once.  The kernel
is written so that all barriers lie on its straight-line path; this test
compiles every instantiated variant to assembly (hipcc, no GPU needed) and
checks what the compiler made of it:
  * no backward branch (a loop) spans a barrier, and
  * no exec-mask skip (s_cbranch_execz) jumps forward over a barrier,
so no wave can pass a barrier a different number of times than the others.
"""

import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "speculative_verify_router_amd", "csrc")
HIPCC = "/opt/rocm/bin/hipcc"

TU = """
#include "flow.h"
namespace svr {
#define SVR_INST(A, B, C, D, E, G, H) template __global__ void k_flow<A, B, C, D, E, G, H>(FlowArgs);
SVR_FLOW_VARIANTS(SVR_INST)
}
"""


def _functions(asm: str):
    lines = asm.split("\n")
    start = None
    for i, line in enumerate(lines):
        m = re.match(r"^(_Z\S+):", line)
        if m:
            start = (m.group(1), i)
        if start and "s_endpgm" in line:
            yield start[0], lines[start[1]:i + 1]
            start = None


def _barrier_hazards(body):
    labels = {}
    for i, line in enumerate(body):
        m = re.match(r"^(\.LBB\S+):", line)
        if m:
            labels[m.group(1)] = i
    bars = [i for i, line in enumerate(body) if re.search(r"\bs_barrier\b", line)]
    loops, skips = [], []
    for i, line in enumerate(body):
        m = re.search(r"\bs_(cbranch_\w+|branch)\s+(\.LBB\S+)", line)
        if not m or m.group(2) not in labels:
            continue
        j = labels[m.group(2)]
        if j < i and any(j <= b <= i for b in bars):
            loops.append((i, j))
        if m.group(1) == "cbranch_execz" and j > i and any(i < b < j for b in bars):
            skips.append((i, j))
    return bars, loops, skips


@pytest.mark.skipif(not os.path.exists(HIPCC),
                    reason="hipcc not available")
def test_every_wave_passes_each_barrier_once(tmp_path):
    src = tmp_path / "flow_variants.hip"
    src.write_text(TU)
    out = tmp_path / "flow_variants.s"
    subprocess.run([HIPCC, "-O3", "-std=c++17", "--offload-arch=gfx950", "--cuda-device-only", "-S",
                    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                    "-mllvm", "-amdgpu-mfma-vgpr-form",
                    "-Wno-unused-command-line-argument", "-I", os.path.join(ROOT, "include"),
                    "-I", CSRC, "-o", str(out), str(src)], check=True, capture_output=True)
    kernels = [(n, b) for n, b in _functions(out.read_text()) if "k_flow" in n]
    assert len(kernels) >= 4
    for name, body in kernels:
        bars, loops, skips = _barrier_hazards(body)
        assert bars, name
        assert not loops, f"{name}: a loop spans a barrier {loops[:3]}"
        assert not skips, f"{name}: an exec-mask branch skips a barrier {skips[:3]}"
