"""GPU parity of the batched path (more than 16 tokens): grouped GEMMs on
the matrix cores, the fp32 MFMA router, token tiles from the bucket lists.

Shapes are chosen so that token tiles end part-way (experts with 1..16+
tokens, several tiles for one expert), row tiles end part-way (F = 96,
H = 640) and Q8_0 rows end part-way through a group of eight sub-blocks
(K = 96, 640).  Ids, order and weights exact as elsewhere; outputs within
2e-3 x RMS of the oracle.
"""

import numpy as np
import pytest
import torch

import synth
from _support import conditioned_tokens, run_oracle, small_config
from gpu_common import check_routing, check_y, desc_of, dev, gpu_forward, gpu_route, log, upload
import speculative_verify_router_amd as svr

pytestmark = pytest.mark.gpu


def _case(cfg):
    log(f"batched case {cfg.name}: H={cfg.hidden} E={cfg.n_experts} k={cfg.top_k} F={cfg.ffn} "
        f"Fs={cfg.shared_ffn} {cfg.expert_type}/{cfg.shared_type} M={cfg.n_tokens}")
    assert svr.moe_stage_name(desc_of(cfg), cfg.n_tokens, 0) == "route"
    inp = synth.draw_layer(cfg)
    x, _ = conditioned_tokens(inp)
    ref = run_oracle(inp, x)
    w = upload(inp)
    y, ids, tw = gpu_forward(cfg, w, x)
    check_routing(ids, tw, ref)
    check_y(y, ref["y"], cfg.name)
    return inp, x, w, y, ref


@pytest.mark.parametrize("M", [17, 40, 130])
def test_q4_k_routed_q8_0_shared(M):
    _case(small_config(hidden=512, n_experts=16, top_k=4, ffn=256, shared_ffn=96,
                       expert_type="q4_k", n_tokens=M, router_std=0.2, seed_index=700 + M))


def test_q8_0_routed_ragged_rows_and_steps():
    # H = 640: 20 sub-blocks per gate/up row, down rows end inside a row block;
    # F = 96: 3 sub-blocks per down row, 6 row tiles.
    _case(small_config(hidden=640, n_experts=12, top_k=3, ffn=96, shared_ffn=160,
                       expert_type="q8_0", n_tokens=33, router_std=0.1, seed_index=710))


def test_one_expert_takes_every_token():
    # E = k = 1: one expert with 40 tokens, three token tiles (16, 16, 8).
    _case(small_config(hidden=512, n_experts=1, top_k=1, ffn=256, expert_type="q4_k",
                       n_tokens=40, seed_index=720))


def test_k_equals_n_experts_with_shared():
    _case(small_config(hidden=256, n_experts=6, top_k=6, ffn=256, shared_ffn=64,
                       expert_type="q4_k", n_tokens=20, router_std=0.3, seed_index=721))


def test_shared_expert_in_q4_k():
    _case(small_config(hidden=512, n_experts=8, top_k=2, ffn=512, shared_ffn=256,
                       expert_type="q4_k", shared_type="q4_k", n_tokens=24, router_std=0.2,
                       seed_index=722))


def test_router_without_mfma_shape():
    # H = 96 is not a multiple of 64: the router falls back to its GEMV kernel.
    _case(small_config(hidden=96, n_experts=8, top_k=2, ffn=64, expert_type="q8_0",
                       n_tokens=20, router_std=0.3, seed_index=723))


def test_step5_shapes_few_experts():
    # The prefill layer's per-expert shapes (H = 4096, F = Fs = 1536) with 32
    # experts, so that most experts see several token tiles.
    _case(small_config(hidden=4096, n_experts=32, top_k=8, ffn=1536, shared_ffn=1536,
                       expert_type="q4_k", n_tokens=64, router_std=0.02, seed_index=724))


def test_repeatable_and_timed():
    cfg = small_config(hidden=512, n_experts=16, top_k=4, ffn=256, shared_ffn=96,
                       expert_type="q4_k", n_tokens=50, router_std=0.2, seed_index=730)
    d = desc_of(cfg)
    assert svr.moe_stage_count(d, 50) == 5
    assert [svr.moe_stage_name(d, 50, i) for i in range(5)] == [
        "route", "shared_gateup", "gateup", "shared_down", "down_combine"]
    inp, x, w, y, ref = _case(cfg)
    y2, _, _ = gpu_forward(cfg, w, x)
    assert np.array_equal(y.view(np.uint32), y2.view(np.uint32))
    # Timed call: same result, one event per stage boundary.
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(6)]
    for e in ev:
        e.record()
    torch.cuda.synchronize()
    yt = torch.empty((50, cfg.hidden), dtype=torch.float32, device="cuda")
    svr.moe_layer_forward_timed(d, w, dev(x), yt, [e.cuda_event for e in ev])
    torch.cuda.synchronize()
    assert np.array_equal(yt.cpu().numpy().view(np.uint32), y.view(np.uint32))
    assert all(ev[i].elapsed_time(ev[i + 1]) >= 0 for i in range(5))


def test_route_lists_of_a_batch():
    cfg = small_config(hidden=512, n_experts=64, top_k=8, n_tokens=100, router_std=0.2,
                       seed_index=740)
    inp = synth.draw_layer(cfg)
    x, _ = conditioned_tokens(inp)
    ref = run_oracle(inp, x)
    r = gpu_route(cfg, dev(inp.router), x)
    check_routing(r["ids"], r["w"], ref)
    assert np.array_equal(r["counts"], ref["counts"])
    assert np.array_equal(r["offsets"], ref["offsets"])
    assert np.array_equal(r["slots"], ref["slots"])
