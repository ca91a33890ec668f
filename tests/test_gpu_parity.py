"""GPU parity on small and edge-case layers: HIP library vs the CPU oracle.

Every call goes through the C ABI.  Expert ids, their order and the bucket
lists must match exactly; routing weights within 1e-6; outputs within
2e-3 x RMS of the oracle's output.  Block decoding must be bit-exact.
"""

import numpy as np
import pytest
import torch

from oracle import moe_oracle as om
import synth
from _support import (conditioned_tokens, copy_expert_rows, read_fixture, run_oracle,
                      scale_fields, small_config)
from gpu_common import (check_routing, check_y, desc_of, dev, gpu_forward, gpu_route, log,
                        upload)
import speculative_verify_router_amd as svr

pytestmark = pytest.mark.gpu


def _layer_case(cfg, x=None, inp=None):
    log(f"case {cfg.name}: H={cfg.hidden} E={cfg.n_experts} k={cfg.top_k} F={cfg.ffn} "
        f"Fs={cfg.shared_ffn} {cfg.expert_type}/{cfg.shared_type} M={cfg.n_tokens}")
    inp = inp or synth.draw_layer(cfg)
    if x is None:
        x, _ = conditioned_tokens(inp)
    ref = run_oracle(inp, x)
    y, ids, w = gpu_forward(cfg, upload(inp), x)
    check_routing(ids, w, ref)
    check_y(y, ref["y"], cfg.name)
    return inp, x, y, ref


# ----------------------------------------------------------------------------- dequant

@pytest.mark.parametrize("fixture,dtype", [("q8_0_planar.txt", "q8_0"), ("q4_k_planar.txt", "q4_k")])
def test_dequant_fixture_bit_exact(fixture, dtype):
    rows, cols, buf, _ = read_fixture(fixture)
    ref = om.dequant(dtype, buf, rows, cols).astype(np.float32)
    out = torch.empty((rows, cols), dtype=torch.float32, device="cuda")
    svr.moe_dequant_rows(dtype, dev(buf), rows, cols, 0, rows, out)
    torch.cuda.synchronize()
    assert np.array_equal(out.cpu().numpy().view(np.uint32), ref.view(np.uint32))


@pytest.mark.parametrize("dtype,cols", [("q8_0", 4096), ("q8_0", 1280), ("q4_k", 4096), ("q4_k", 1536)])
def test_dequant_random_bit_exact(dtype, cols):
    cfg = small_config(hidden=cols, ffn=256, n_experts=3, expert_type=dtype, seed_index=300)
    inp = synth.draw_layer(cfg)
    rows = 3 * 256
    buf = inp.gate.copy()
    # a few subnormal and zero scales
    f = scale_fields(dtype, buf, rows, cols)     # a view into buf
    f[:7] = np.array([0, 1, 2, 0x3FF, 0x200, 0x8001, 0], dtype=np.uint16).reshape(
        (7,) + (1,) * (f.ndim - 1))
    ref = om.dequant(dtype, buf, rows, cols, 5, 300).astype(np.float32)
    out = torch.empty((300, cols), dtype=torch.float32, device="cuda")
    svr.moe_dequant_rows(dtype, dev(buf), rows, cols, 5, 300, out)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))


# ----------------------------------------------------------------------------- routing

@pytest.mark.parametrize("E,k,M", [(8, 2, 1), (8, 8, 3), (8, 1, 5), (288, 8, 4), (352, 8, 64),
                                   (1024, 64, 7), (1, 1, 2), (100, 3, 300)])
def test_route_exact(E, k, M):
    cfg = small_config(n_experts=E, top_k=k, n_tokens=M, hidden=512, router_std=0.3,
                       seed_index=400 + E + k)
    rng = np.random.default_rng(E * 1000 + k)
    router = (rng.standard_normal((E, 512)) * 0.3).astype(np.float32)
    inp = synth.LayerInputs(cfg, router, None, None, None)
    x, _ = conditioned_tokens(inp)
    ref = om.route(router, x, k)
    got = gpu_route(cfg, dev(router), x)
    check_routing(got["ids"], got["w"], ref)
    assert np.array_equal(got["counts"], ref["counts"])
    assert np.array_equal(got["offsets"], ref["offsets"])
    assert np.array_equal(got["slots"][:M * k], ref["slots"])
    na = int(got["n_active"][0])
    assert na == len(ref["active"])
    assert np.array_equal(got["active"][:na], ref["active"])
    assert np.all(got["active"][na:] == -1)


def test_route_ties_go_to_lower_index():
    # Router rows 0..7 identical: every token sees 8 exactly equal logits.
    cfg = small_config(n_experts=8, top_k=3, n_tokens=2, hidden=256)
    router = np.tile(np.random.default_rng(5).standard_normal(256).astype(np.float32), (8, 1))
    x = np.random.default_rng(6).standard_normal((2, 256)).astype(np.float32)
    got = gpu_route(cfg, dev(router), x)
    assert got["ids"].tolist() == [[0, 1, 2], [0, 1, 2]]
    assert np.allclose(got["w"], 1.0 / 3.0, atol=1e-7)


# ----------------------------------------------------------------------------- layer

def test_tiny_config():
    _layer_case(synth.CONFIGS["tiny"])


@pytest.mark.parametrize("M", [1, 2, 3, 4, 5, 9])
def test_small_q4_k_with_shared(M):
    cfg = small_config(hidden=512, n_experts=16, top_k=4, ffn=256, shared_ffn=128,
                       expert_type="q4_k", n_tokens=M, router_std=0.2, seed_index=500 + M)
    _layer_case(cfg)


@pytest.mark.parametrize("M", [1, 4, 6])
def test_small_q8_0_with_shared(M):
    cfg = small_config(hidden=1024, n_experts=12, top_k=3, ffn=320, shared_ffn=192,
                       expert_type="q8_0", n_tokens=M, router_std=0.1, seed_index=520 + M)
    _layer_case(cfg)


def test_shared_expert_in_q4_k():
    cfg = small_config(hidden=512, n_experts=8, top_k=2, ffn=512, shared_ffn=256,
                       expert_type="q4_k", shared_type="q4_k", n_tokens=3, router_std=0.2,
                       seed_index=540)
    _layer_case(cfg)


def test_k_equals_one():
    _layer_case(small_config(n_experts=8, top_k=1, n_tokens=4, seed_index=550))


def test_k_equals_n_experts():
    _layer_case(small_config(n_experts=6, top_k=6, n_tokens=3, shared_ffn=64, seed_index=551))


def test_single_expert_layer():
    _layer_case(small_config(n_experts=1, top_k=1, n_tokens=3, ffn=96, seed_index=552))


def test_ragged_rows_and_lanes():
    # F = 96 (3 Q8_0 blocks: 6 chunks per down row) and H = 640 (20 blocks):
    # row tiles and lane groups both end part-way.
    _layer_case(small_config(hidden=640, n_experts=5, top_k=2, ffn=96, shared_ffn=160,
                             n_tokens=5, router_std=0.2, seed_index=553))


@pytest.mark.parametrize("M", [2, 6])
def test_partial_lane_groups(M):
    # H = 288 (18 Q8_0 chunks per gate/up row: 4 lanes x 5 chunks, two
    # positions past the row end) and F = 1280 Q4_K (40 chunks per down row:
    # 16 lanes x 3 chunks, eight positions past the end).
    _layer_case(small_config(hidden=288, n_experts=6, top_k=2, ffn=96, shared_ffn=96,
                             n_tokens=M, router_std=0.3, seed_index=556 + M))
    _layer_case(small_config(hidden=512, n_experts=4, top_k=2, ffn=1280, shared_ffn=0,
                             expert_type="q4_k", n_tokens=M, router_std=0.2,
                             seed_index=560 + M))


def test_all_tokens_on_the_same_experts():
    cfg = small_config(hidden=512, n_experts=16, top_k=4, ffn=256, shared_ffn=128,
                       expert_type="q4_k", n_tokens=8, router_std=0.2, seed_index=554)
    inp = synth.draw_layer(cfg)
    x1, _ = conditioned_tokens(inp, n_tokens=1)
    x = np.repeat(x1, 8, axis=0)
    _, _, y, ref = _layer_case(cfg, x=x, inp=inp)
    assert len(ref["active"]) == 4
    assert np.array_equal(y, np.repeat(y[:1], 8, axis=0))


def test_zero_and_subnormal_scales():
    for etype in ("q8_0", "q4_k"):
        F = 256
        cfg = small_config(hidden=512, n_experts=4, top_k=2, ffn=F, shared_ffn=64,
                           expert_type=etype, n_tokens=3, router_std=0.2, seed_index=555)
        inp = synth.draw_layer(cfg)
        for name, rows, cols in (("gate", 4 * F, 512), ("up", 4 * F, 512), ("down", 4 * 512, F)):
            buf = getattr(inp, name).copy()
            f = scale_fields(etype, buf, rows, cols)     # a view into buf
            f[::5] = 0                                   # zero blocks
            f[1::7] = f[1::7] & 0x83FF                   # subnormal (exponent field 0)
            setattr(inp, name, buf)
        _layer_case(cfg, inp=inp)


def test_identical_experts_match_across_routing():
    cfg = small_config(hidden=512, n_experts=6, top_k=3, ffn=256, expert_type="q4_k",
                       n_tokens=4, router_std=0.2, seed_index=556)
    inp = synth.draw_layer(cfg)
    inp.gate = copy_expert_rows("q4_k", inp.gate, 256, 512, 6)
    inp.up = copy_expert_rows("q4_k", inp.up, 256, 512, 6)
    inp.down = copy_expert_rows("q4_k", inp.down, 512, 256, 6)
    _layer_case(cfg, inp=inp)


def test_rows_equal_single_token_calls_bitwise():
    # Each token's result does not depend on the other tokens of the batch.
    cfg = small_config(hidden=1024, n_experts=32, top_k=4, ffn=512, shared_ffn=256,
                       expert_type="q4_k", n_tokens=4, router_std=0.1, seed_index=557)
    inp, x, y, _ = _layer_case(cfg)
    w = upload(inp)
    for t in range(4):
        y1, _, _ = gpu_forward(cfg, w, x[t:t + 1])
        assert np.array_equal(y1[0].view(np.uint32), y[t].view(np.uint32)), t


@pytest.mark.parametrize("etype", ["q4_k", "q8_0", "q2_k"])
@pytest.mark.parametrize("rows", [(0, 0, 0, 0), (0, 1, 0, 1), (0, 1, 1, 1), (0, 1, 2, 3)])
def test_experts_shared_by_several_tokens(etype, rows):
    # Verify batches whose tokens select the same experts (all four tokens,
    # two pairs, three and one, partial overlaps): the gate/up pass of an
    # expert serves all of its tokens at once.  Matches the oracle, and each
    # row equals that token's single-token call bit for bit.
    cfg = small_config(hidden=512, n_experts=16, top_k=4, ffn=256, shared_ffn=128,
                       expert_type=etype, n_tokens=4, router_std=0.2, seed_index=570)
    inp = synth.draw_layer(cfg)
    x4, _ = conditioned_tokens(inp)
    x = np.ascontiguousarray(x4[list(rows)])
    inp, x, y, ref = _layer_case(cfg, x=x, inp=inp)
    ids = np.asarray(ref["ids"])
    assert len(np.unique(ids)) < ids.size  # some expert serves several tokens
    w = upload(inp)
    for t in range(4):
        y1, _, _ = gpu_forward(cfg, w, x[t:t + 1])
        assert np.array_equal(y1[0].view(np.uint32), y[t].view(np.uint32)), t


@pytest.mark.parametrize("E,k", [(128, 64), (64, 64), (100, 17)])
def test_shared_experts_with_many_slots(E, k):
    # Four tokens with up to 64 slots each (256 pairs: several pairs per lane
    # when the routing builds the pairs' token words) on few experts, so most
    # experts serve two to four tokens.
    cfg = small_config(hidden=512, n_experts=E, top_k=k, ffn=256, shared_ffn=128,
                       expert_type="q4_k", n_tokens=4, router_std=0.2, seed_index=580 + k)
    inp, x, y, ref = _layer_case(cfg)
    w = upload(inp)
    for t in range(4):
        y1, _, _ = gpu_forward(cfg, w, x[t:t + 1])
        assert np.array_equal(y1[0].view(np.uint32), y[t].view(np.uint32)), t


def test_wide_hidden_takes_the_unfused_routing():
    # H = 9216 is past the fused phase-1 router (H <= 8192): the routing runs
    # as separate launches, and for four tokens the pairs' token words come
    # from their own one-wave launch.  Eight experts, two per token: tokens
    # share experts.
    cfg = small_config(hidden=9216, n_experts=8, top_k=2, ffn=256, shared_ffn=256,
                       expert_type="q4_k", shared_type="q4_k", n_tokens=4, router_std=0.05,
                       seed_index=590)
    inp, x, y, ref = _layer_case(cfg)
    w = upload(inp)
    for t in range(4):
        y1, _, _ = gpu_forward(cfg, w, x[t:t + 1])
        assert np.array_equal(y1[0].view(np.uint32), y[t].view(np.uint32)), t


@pytest.mark.parametrize("M", [1, 4, 16])
def test_largest_routing_shape(M):
    # The layer at the routing limits: 1024 experts, 64 selected per token
    # (256 pairs at four tokens; 1024 (token, slot) pairs over the expert
    # lists at sixteen), with a shared expert.
    cfg = small_config(hidden=512, n_experts=1024, top_k=64, ffn=256, shared_ffn=128,
                       expert_type="q4_k", n_tokens=M, router_std=0.2, seed_index=600 + M)
    _layer_case(cfg)


def test_zero_tokens_is_a_no_op():
    cfg = small_config()
    inp = synth.draw_layer(cfg)
    x = torch.empty((0, cfg.hidden), dtype=torch.float32, device="cuda")
    y = torch.empty((0, cfg.hidden), dtype=torch.float32, device="cuda")
    svr.moe_layer_forward(desc_of(cfg), upload(inp), x, y, ws=torch.empty(256, dtype=torch.uint8,
                                                                            device="cuda"))
    torch.cuda.synchronize()


def test_timed_forward_matches_and_records_events():
    cfg = small_config(hidden=512, n_experts=16, top_k=4, ffn=256, shared_ffn=128,
                       expert_type="q4_k", n_tokens=4, router_std=0.2, seed_index=558)
    inp = synth.draw_layer(cfg)
    x, _ = conditioned_tokens(inp)
    w = upload(inp)
    y0, _, _ = gpu_forward(cfg, w, x)
    n = svr.moe_stage_count(desc_of(cfg), 4) + 1
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(n)]
    for e in evs:
        e.record()
    torch.cuda.synchronize()
    y = torch.empty((4, 512), dtype=torch.float32, device="cuda")
    svr.moe_layer_forward_timed(desc_of(cfg), w, dev(x), y, [e.cuda_event for e in evs])
    torch.cuda.synchronize()
    assert np.array_equal(y.cpu().numpy(), y0)
    ms = [evs[i].elapsed_time(evs[i + 1]) for i in range(n - 1)]
    assert all(m >= 0 for m in ms)
    with pytest.raises(svr.MoeError):
        svr.moe_layer_forward_timed(desc_of(cfg), w, dev(x), y, [e.cuda_event for e in evs[:-1]])


def test_prepared_forward_matches_plain_call():
    cfg = small_config(hidden=512, n_experts=16, top_k=4, ffn=256, shared_ffn=128,
                       expert_type="q4_k", n_tokens=3, router_std=0.2, seed_index=559)
    inp = synth.draw_layer(cfg)
    x, _ = conditioned_tokens(inp)
    w = upload(inp)
    y0, ids0, tw0 = gpu_forward(cfg, w, x)
    y = torch.empty((3, 512), dtype=torch.float32, device="cuda")
    ids = torch.empty((3, 4), dtype=torch.int32, device="cuda")
    tw = torch.empty((3, 4), dtype=torch.float32, device="cuda")
    call = svr.PreparedForward(desc_of(cfg), w, dev(x), y, ids, tw)
    for _ in range(3):  # the workspace is reused call after call
        y.zero_()
        call()
        torch.cuda.synchronize()
        assert np.array_equal(y.cpu().numpy(), y0)
        assert np.array_equal(ids.cpu().numpy(), ids0)


@pytest.mark.parametrize("M", [1, 4, 9, 16])
def test_handoff_areas_return_to_zero(M):
    # The counters and the routing keys at the start of the workspace must
    # be zero before a call and are zero after it, whatever the batch size
    # (their offsets depend on the layer only); one workspace serves calls of
    # different sizes in turn.  The routing wait's diagnostic word stays 0.
    cfg = small_config(hidden=512, n_experts=40, top_k=4, ffn=256, shared_ffn=128,
                       expert_type="q4_k", n_tokens=16, router_std=0.2, seed_index=560)
    inp = synth.draw_layer(cfg)
    x, _ = conditioned_tokens(inp)
    w = upload(inp)
    desc = desc_of(cfg)
    ws = svr.workspace(desc, 16, "cuda")
    handoff = 16384 + (cfg.n_experts * 64 + 255) // 256 * 256
    for m in (M, 16, M):
        y = torch.empty((m, 512), dtype=torch.float32, device="cuda")
        ids = torch.empty((m, 4), dtype=torch.int32, device="cuda")
        svr.moe_layer_forward(desc, w, dev(x[:m]), y, ids, None, ws=ws)
        torch.cuda.synchronize()
        assert int(ws[:handoff].count_nonzero().item()) == 0
        ref = run_oracle(inp, x[:m])
        assert np.array_equal(ids.cpu().numpy(), ref["ids"])
        check_y(y.cpu().numpy(), ref["y"], f"M={m}")
