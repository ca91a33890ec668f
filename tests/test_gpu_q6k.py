"""GPU parity of Q6_K routed matrices: HIP library vs the CPU oracle.

Q6_K is the recipes' type for the MTP heads' matrices ("Step-5 Preview
GGUF", Tensor-type table); here it is a routed-expert type like the other
K-quants.  Block decoding must be bit-exact; layers must match the oracle's
ids exactly, routing weights within 1e-6 and outputs within 2e-3 x RMS on
pair slots (1 to 4 tokens), expert lists (5 to 16) and the matrix-core
grouped GEMMs beyond 16 tokens.
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
    rows, cols, buf, _ = read_fixture("q6_k_planar.txt")
    ref = om.dequant("q6_k", buf, rows, cols).astype(np.float32)
    out = torch.empty((rows, cols), dtype=torch.float32, device="cuda")
    svr.moe_dequant_rows("q6_k", dev(buf), rows, cols, 0, rows, out)
    torch.cuda.synchronize()
    assert np.array_equal(out.cpu().numpy().view(np.uint32), ref.view(np.uint32))


@pytest.mark.parametrize("cols", [4096, 1536, 1280])
def test_dequant_random_bit_exact(cols):
    cfg = small_config(hidden=cols, ffn=256, n_experts=3, expert_type="q6_k", seed_index=330)
    inp = synth.draw_layer(cfg)
    rows = 3 * 256
    buf = inp.gate.copy()
    f = scale_fields("q6_k", buf, rows, cols)     # d of every super-block
    f[:7] = np.array([0, 1, 2, 0x3FF, 0x200, 0x8001, 0], dtype=np.uint16).reshape(7, 1)
    ref = om.dequant("q6_k", buf, rows, cols, 5, 300).astype(np.float32)
    out = torch.empty((300, cols), dtype=torch.float32, device="cuda")
    svr.moe_dequant_rows("q6_k", dev(buf), rows, cols, 5, 300, out)
    torch.cuda.synchronize()
    assert np.array_equal(out.cpu().numpy().view(np.uint32), ref.view(np.uint32))


@pytest.mark.parametrize("M", [1, 2, 3, 4, 5, 9, 16, 17, 40])
def test_small_q6_k_with_shared(M):
    # H = 1024: 32 chunks of 32 per gate/up row; F = 768: 24 chunks per down row
    cfg = small_config(hidden=1024, n_experts=16, top_k=4, ffn=768, shared_ffn=256,
                       expert_type="q6_k", n_tokens=M, router_std=0.2, seed_index=900 + M)
    _case(cfg)


@pytest.mark.parametrize("M", [2, 6])
def test_q6_k_partial_lane_groups_and_q4_k_down(M):
    # F = 1280: 40 chunks per down row (16 lanes x 3, eight positions past the
    # end); Q6_K gate/up with Q4_K down, the other pairing of types
    cfg = small_config(hidden=768, n_experts=6, top_k=3, ffn=1280, shared_ffn=256,
                       expert_type="q6_k", n_tokens=M, router_std=0.2, seed_index=940 + M)
    _case(cfg)
    _case(cfg.replace(down_type="q4_k", seed_index=950 + M))


@pytest.mark.parametrize("M,E,k,down", [(200, 16, 4, None), (96, 40, 8, "q2_k"), (33, 8, 2, "q4_k")])
def test_q6_k_batched(M, E, k, down):
    # more than 16 tokens: the matrix-core grouped GEMMs decode Q6_K (and
    # Q6_K gate/up with another down type)
    cfg = small_config(hidden=1024, n_experts=E, top_k=k, ffn=512, shared_ffn=256,
                       expert_type="q6_k", down_type=down, n_tokens=M, router_std=0.2,
                       seed_index=970 + M)
    _case(cfg)
    if down is None:
        _case(cfg.replace(expert_type="q4_k", down_type="q6_k", seed_index=975 + M))


@pytest.mark.parametrize("M", [3, 40])
def test_q6_k_zero_and_subnormal_scales(M):
    F = 256
    cfg = small_config(hidden=512, n_experts=4, top_k=2, ffn=F, shared_ffn=64,
                       expert_type="q6_k", n_tokens=M, router_std=0.2, seed_index=960 + M)
    inp = synth.draw_layer(cfg)
    for name, rows, cols in (("gate", 4 * F, 512), ("up", 4 * F, 512), ("down", 4 * 512, F)):
        buf = getattr(inp, name).copy()
        f = scale_fields("q6_k", buf, rows, cols)
        f[::5] = 0                                   # zero d
        f[1::7] = f[1::7] & 0x83FF                   # subnormal (exponent field 0)
        setattr(inp, name, buf)
    _case(cfg, inp=inp)
