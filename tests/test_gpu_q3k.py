"""GPU parity of Q3_K routed matrices and of a routed down type that differs
from the gate/up type: HIP library vs the CPU oracle.

The Q2_K-Protected2 recipe stores routed gate/up in Q2_K and routed down in
Q3_K ("Step-5 Preview GGUF", Tensor-type table).  Block decoding must be
bit-exact; layers must match the oracle's ids exactly, routing weights
within 1e-6 and outputs within 2e-3 x RMS on every launch sequence: pair
slots (1 to 4 tokens), expert lists (5 to 16) and the grouped GEMMs on the
matrix cores beyond 16 tokens (1 + Q/128 bf16 operands against activations
masked to each 16-column half of a step; gate/up and down types apart).
"""

import numpy as np
import pytest
import torch

from oracle import moe_oracle as om
import synth
from _support import conditioned_tokens, read_fixture, run_oracle, scale_fields, small_config
from gpu_common import check_routing, check_y, dev, gpu_forward, log, upload
import speculative_verify_router_amd as svr

pytestmark = pytest.mark.gpu


def _case(cfg, inp=None, x=None):
    log(f"case {cfg.name}: H={cfg.hidden} E={cfg.n_experts} k={cfg.top_k} F={cfg.ffn} "
        f"Fs={cfg.shared_ffn} {cfg.expert_type}+{cfg.routed_down_type}/{cfg.shared_type} "
        f"M={cfg.n_tokens}")
    inp = inp or synth.draw_layer(cfg)
    if x is None:
        x, _ = conditioned_tokens(inp)
    ref = run_oracle(inp, x)
    y, ids, w = gpu_forward(cfg, upload(inp), x)
    check_routing(ids, w, ref)
    check_y(y, ref["y"], cfg.name)
    return y, ref


def test_dequant_fixture_bit_exact():
    rows, cols, buf, _ = read_fixture("q3_k_planar.txt")
    ref = om.dequant("q3_k", buf, rows, cols).astype(np.float32)
    out = torch.empty((rows, cols), dtype=torch.float32, device="cuda")
    svr.moe_dequant_rows("q3_k", dev(buf), rows, cols, 0, rows, out)
    torch.cuda.synchronize()
    assert np.array_equal(out.cpu().numpy().view(np.uint32), ref.view(np.uint32))


@pytest.mark.parametrize("cols", [4096, 1536, 1280])
def test_dequant_random_bit_exact(cols):
    cfg = small_config(hidden=512, ffn=cols, n_experts=3, expert_type="q2_k", down_type="q3_k",
                       seed_index=320)
    inp = synth.draw_layer(cfg)
    rows = 3 * 512
    buf = inp.down.copy()
    f = scale_fields("q3_k", buf, rows, cols)     # d of every super-block
    f[:7] = np.array([0, 1, 2, 0x3FF, 0x200, 0x8001, 0], dtype=np.uint16).reshape(7, 1)
    ref = om.dequant("q3_k", buf, rows, cols, 5, 300).astype(np.float32)
    out = torch.empty((300, cols), dtype=torch.float32, device="cuda")
    svr.moe_dequant_rows("q3_k", dev(buf), rows, cols, 5, 300, out)
    torch.cuda.synchronize()
    assert np.array_equal(out.cpu().numpy().view(np.uint32), ref.view(np.uint32))


@pytest.mark.parametrize("M", [1, 2, 3, 4, 5, 9, 16, 17, 40])
def test_q2_k_gate_up_q3_k_down(M):
    # the recipe's pairing; H = 1024 (16 chunks of 64), F = 512 (8 chunks)
    cfg = small_config(hidden=1024, n_experts=16, top_k=4, ffn=512, shared_ffn=256,
                       expert_type="q2_k", down_type="q3_k", n_tokens=M, router_std=0.2,
                       seed_index=800 + M)
    _case(cfg)


@pytest.mark.parametrize("M,E,k", [(200, 16, 4), (96, 40, 8)])
def test_q2_k_gate_up_q3_k_down_batched(M, E, k):
    cfg = small_config(hidden=1024, n_experts=E, top_k=k, ffn=512, shared_ffn=256,
                       expert_type="q2_k", down_type="q3_k", n_tokens=M, router_std=0.2,
                       seed_index=820 + M)
    _case(cfg)


@pytest.mark.parametrize("M", [1, 4, 6, 33])
def test_all_q3_k(M):
    cfg = small_config(hidden=512, n_experts=8, top_k=2, ffn=256, shared_ffn=128,
                       expert_type="q3_k", n_tokens=M, router_std=0.3, seed_index=850 + M)
    _case(cfg)


@pytest.mark.parametrize("M", [3, 20])
def test_q4_k_gate_up_q8_0_down(M):
    # a down type other than the gate/up type on the Q4_K/Q8_0 kernels,
    # including a batch that the matrix-core path would take if the types matched
    cfg = small_config(hidden=512, n_experts=8, top_k=2, ffn=256, shared_ffn=64,
                       expert_type="q4_k", down_type="q8_0", n_tokens=M, router_std=0.3,
                       seed_index=860 + M)
    _case(cfg)


@pytest.mark.parametrize("M", [2, 6])
def test_q3_k_partial_lane_groups(M):
    # F = 1280: 20 chunks per down row (32 lanes, twelve positions past the end)
    cfg = small_config(hidden=768, n_experts=6, top_k=3, ffn=1280, shared_ffn=256,
                       expert_type="q2_k", down_type="q3_k", n_tokens=M, router_std=0.2,
                       seed_index=870 + M)
    _case(cfg)


def test_q3_k_zero_and_subnormal_scales():
    F = 256
    cfg = small_config(hidden=512, n_experts=4, top_k=2, ffn=F, shared_ffn=64,
                       expert_type="q3_k", n_tokens=3, router_std=0.2, seed_index=880)
    inp = synth.draw_layer(cfg)
    for name, rows, cols in (("gate", 4 * F, 512), ("up", 4 * F, 512), ("down", 4 * 512, F)):
        buf = getattr(inp, name).copy()
        f = scale_fields("q3_k", buf, rows, cols)
        f[::5] = 0                                   # zero d
        f[1::7] = f[1::7] & 0x83FF                   # subnormal (exponent field 0)
        setattr(inp, name, buf)
    _case(cfg, inp=inp)
