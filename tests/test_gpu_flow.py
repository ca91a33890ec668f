"""GPU parity of the single-launch path (batches of 1 to 4 tokens).

Layers with H = 4096 and F = Fs = 1280 or 1536 run as one k_flow launch:
router rows, top-k, shared and routed gate/up, shared and routed down and
the combine as items of one work queue.  Few experts keep the oracle fast;
the kernels see the full per-expert shapes, several row tiles per pair and
ragged last tiles (1536 rows in tiles of 20).
"""

import dataclasses

import numpy as np
import pytest
import torch

import synth
from _support import conditioned_tokens, run_oracle, small_config
from gpu_common import check_routing, check_y, dev, log, upload
from gpu_common import desc_of as _desc_of, gpu_forward as _gpu_forward
import speculative_verify_router_amd as svr

pytestmark = pytest.mark.gpu

# (ffn, shared_ffn, routed type): the three H = 4096 instantiations.
SHAPES = {
    "q4k_f1280": (1280, 1280, "q4_k"),
    "q4k_f1536": (1536, 1536, "q4_k"),
    "q8_0_f1280": (1280, 1280, "q8_0"),
}


def _cfg(shape, M, seed, E=16, k=8):
    F, Fs, et = SHAPES[shape]
    return small_config(hidden=4096, n_experts=E, top_k=k, ffn=F, shared_ffn=Fs, expert_type=et,
                        shared_type="q8_0", n_tokens=M, router_std=0.02, seed_index=seed)


def desc_of(cfg):
    return dataclasses.replace(_desc_of(cfg), single_launch=True)


def gpu_forward(cfg, weights, x):
    return _gpu_forward(cfg, weights, x, desc=desc_of(cfg))


@pytest.mark.parametrize("shape", sorted(SHAPES))
def test_flow_path_is_one_launch(shape):
    for M in (1, 2, 3, 4):
        d = desc_of(_cfg(shape, M, 600))
        assert svr.moe_stage_count(d, M) == 1
        assert svr.moe_stage_name(d, M, 0) == "layer"
    assert svr.moe_stage_count(desc_of(_cfg(shape, 5, 600)), 5) == 3
    # Without the flag the same shapes run staged.
    assert svr.moe_stage_count(_desc_of(_cfg(shape, 4, 600)), 4) == 3


@pytest.mark.parametrize("shape", sorted(SHAPES))
@pytest.mark.parametrize("M", [1, 2, 3, 4])
def test_flow_layer_matches_oracle(shape, M):
    cfg = _cfg(shape, M, 610 + M)
    log(f"flow case {shape} M={M}")
    inp = synth.draw_layer(cfg)
    x, _ = conditioned_tokens(inp)
    ref = run_oracle(inp, x)
    y, ids, w = gpu_forward(cfg, upload(inp), x)
    check_routing(ids, w, ref)
    check_y(y, ref["y"], f"{shape} M={M}")


def test_flow_reuses_workspace_and_leaves_counters_zero():
    cfg = _cfg("q4k_f1280", 4, 620)
    inp = synth.draw_layer(cfg)
    x, _ = conditioned_tokens(inp)
    w = upload(inp)
    d = desc_of(cfg)
    ws = svr.workspace(d, 4)
    xd = dev(x)
    outs = []
    for _ in range(3):
        y = torch.full((4, cfg.hidden), float("nan"), dtype=torch.float32, device="cuda")
        svr.moe_layer_forward(d, w, xd, y, ws=ws)
        torch.cuda.synchronize()
        assert not torch.any(ws[:svr._binding.COUNTER_BYTES]).item(), "counters not back to zero"
        outs.append(y.cpu().numpy())
    # Fixed reduction and combine orders: repeated calls agree bit for bit.
    assert np.array_equal(outs[0], outs[1]) and np.array_equal(outs[0], outs[2])
    check_y(outs[0], run_oracle(inp, x)["y"], "reused workspace")


def test_flow_rows_do_not_depend_on_the_batch():
    cfg = _cfg("q4k_f1536", 4, 630)
    inp = synth.draw_layer(cfg)
    x, _ = conditioned_tokens(inp)
    w = upload(inp)
    y4, ids4, w4 = gpu_forward(cfg, w, x)
    for t in range(4):
        c1 = _cfg("q4k_f1536", 1, 630)
        y1, ids1, w1 = gpu_forward(c1, w, x[t:t + 1])
        assert np.array_equal(ids1[0], ids4[t])
        assert np.array_equal(y1[0].view(np.uint32), y4[t].view(np.uint32))


def test_flow_all_tokens_on_the_same_experts():
    # Every pair of an expert streams it for its own token; duplicates must
    # not disturb the per-pair hand-offs.
    cfg = _cfg("q4k_f1280", 4, 640, E=8, k=8)
    inp = synth.draw_layer(cfg)
    x, _ = conditioned_tokens(inp)
    ref = run_oracle(inp, x)
    y, ids, w = gpu_forward(cfg, upload(inp), x)
    check_routing(ids, w, ref)
    check_y(y, ref["y"], "k == E")


def test_flow_without_shared_expert_small_shapes():
    # H <= 1024, small Q8_0 experts, no shared expert: the small instantiation.
    for M in (1, 4):
        cfg = small_config(n_experts=8, top_k=2, n_tokens=M, seed_index=650 + M)
        assert svr.moe_stage_count(desc_of(cfg), M) == 1
        inp = synth.draw_layer(cfg)
        x, _ = conditioned_tokens(inp)
        ref = run_oracle(inp, x)
        y, ids, w = gpu_forward(cfg, upload(inp), x)
        check_routing(ids, w, ref)
        check_y(y, ref["y"], f"small M={M}")
