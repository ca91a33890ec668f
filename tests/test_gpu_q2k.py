"""GPU parity of the Q2_K routed-expert path: HIP library vs the CPU oracle.

Q2_K is the 2-bit type of the routed matrices in the 2-bit Step-5 recipes
("Step-5 Preview GGUF", Tensor-type table).  Block decoding must be
bit-exact; layers must match the oracle's ids exactly, routing weights
within 1e-6 and outputs within 2e-3 x RMS, on every launch sequence the
type can take: pair slots (1 to 4 tokens), expert lists (5 to 16), and the
grouped GEMMs on the matrix cores beyond 16 tokens (sc q as bf16 operands,
split activation sums for the two 16-column halves of each step).
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
        f"Fs={cfg.shared_ffn} {cfg.expert_type}/{cfg.shared_type} M={cfg.n_tokens}")
    inp = inp or synth.draw_layer(cfg)
    if x is None:
        x, _ = conditioned_tokens(inp)
    ref = run_oracle(inp, x)
    y, ids, w = gpu_forward(cfg, upload(inp), x)
    check_routing(ids, w, ref)
    check_y(y, ref["y"], cfg.name)
    return y, ref


def test_dequant_fixture_bit_exact():
    rows, cols, buf, _ = read_fixture("q2_k_planar.txt")
    ref = om.dequant("q2_k", buf, rows, cols).astype(np.float32)
    out = torch.empty((rows, cols), dtype=torch.float32, device="cuda")
    svr.moe_dequant_rows("q2_k", dev(buf), rows, cols, 0, rows, out)
    torch.cuda.synchronize()
    assert np.array_equal(out.cpu().numpy().view(np.uint32), ref.view(np.uint32))


@pytest.mark.parametrize("cols", [4096, 1536, 1280])
def test_dequant_random_bit_exact(cols):
    cfg = small_config(hidden=cols, ffn=256, n_experts=3, expert_type="q2_k", seed_index=310)
    inp = synth.draw_layer(cfg)
    rows = 3 * 256
    buf = inp.gate.copy()
    f = scale_fields("q2_k", buf, rows, cols)     # d and dmin of every super-block
    f[:7] = np.array([0, 1, 2, 0x3FF, 0x200, 0x8001, 0], dtype=np.uint16).reshape(7, 1)
    ref = om.dequant("q2_k", buf, rows, cols, 5, 300).astype(np.float32)
    out = torch.empty((300, cols), dtype=torch.float32, device="cuda")
    svr.moe_dequant_rows("q2_k", dev(buf), rows, cols, 5, 300, out)
    torch.cuda.synchronize()
    assert np.array_equal(out.cpu().numpy().view(np.uint32), ref.view(np.uint32))


@pytest.mark.parametrize("M", [1, 2, 3, 4, 5, 9, 16, 17, 40])
def test_small_q2_k_with_shared(M):
    # H = 1024: 16 chunks of 64 per gate/up row; F = 512: 8 chunks per down row.
    cfg = small_config(hidden=1024, n_experts=16, top_k=4, ffn=512, shared_ffn=256,
                       expert_type="q2_k", n_tokens=M, router_std=0.2, seed_index=700 + M)
    _case(cfg)


@pytest.mark.parametrize("M,E,k", [(200, 16, 4), (96, 40, 8)])
def test_q2_k_batched_matrix_core_path(M, E, k):
    # several token tiles per expert, partial tiles, every expert active
    cfg = small_config(hidden=1024, n_experts=E, top_k=k, ffn=512, shared_ffn=256,
                       expert_type="q2_k", n_tokens=M, router_std=0.2, seed_index=720 + M)
    _case(cfg)


@pytest.mark.parametrize("M", [1, 4, 7])
def test_q2_k_without_shared_expert(M):
    cfg = small_config(hidden=512, n_experts=8, top_k=2, ffn=256, shared_ffn=0,
                       expert_type="q2_k", n_tokens=M, router_std=0.3, seed_index=760 + M)
    _case(cfg)


@pytest.mark.parametrize("M", [2, 6])
def test_q2_k_partial_lane_groups(M):
    # H = 768: 12 chunks per gate/up row (16 lanes, four positions past the
    # end); F = 1280: 20 chunks per down row (32 lanes, twelve past the end);
    # 3 x 1280 expert rows end part-way through the row tiles.
    cfg = small_config(hidden=768, n_experts=6, top_k=3, ffn=1280, shared_ffn=256,
                       expert_type="q2_k", n_tokens=M, router_std=0.2, seed_index=770 + M)
    _case(cfg)


def test_q2_k_zero_and_subnormal_scales():
    F = 256
    cfg = small_config(hidden=512, n_experts=4, top_k=2, ffn=F, shared_ffn=64,
                       expert_type="q2_k", n_tokens=3, router_std=0.2, seed_index=780)
    inp = synth.draw_layer(cfg)
    for name, rows, cols in (("gate", 4 * F, 512), ("up", 4 * F, 512), ("down", 4 * 512, F)):
        buf = getattr(inp, name).copy()
        f = scale_fields("q2_k", buf, rows, cols)
        f[::5] = 0                                   # zero d and dmin
        f[1::7] = f[1::7] & 0x83FF                   # subnormal (exponent field 0)
        setattr(inp, name, buf)
    _case(cfg, inp=inp)


def test_q2_k_all_tokens_on_the_same_experts():
    cfg = small_config(hidden=512, n_experts=16, top_k=4, ffn=256, shared_ffn=128,
                       expert_type="q2_k", n_tokens=8, router_std=0.2, seed_index=790)
    inp = synth.draw_layer(cfg)
    x1, _ = conditioned_tokens(inp, n_tokens=1)
    x = np.repeat(x1, 8, axis=0)
    y, ref = _case(cfg, inp=inp, x=x)
    assert len(ref["active"]) == 4
    assert np.array_equal(y, np.repeat(y[:1], 8, axis=0))
