"""GPU parity at the full workload sizes, in the launch configuration the
benchmark times (same shapes, same token counts, one moe_layer_forward).

Step-3.5-Flash-shaped decode (M=1, Q8_0), the same layer as the 4-token
verify batch (Q4_K routed), the Step-5-shaped verify batch with the four
tokens on disjoint experts (Q4_K, Q2_K, and the Q2_K-Protected2 pairing of
Q2_K gate/up with Q3_K down), the Step-3.5 verify batch with Q6_K routed
experts, and the 512-token prefill micro-batches (Q4_K, Q2_K/Q3_K and Q6_K
routed).  Every output row of every workload is compared with the oracle,
element by element.
"""

import gc

import numpy as np
import pytest

import synth
from _support import conditioned_tokens, oracle_workers, run_oracle
from gpu_common import check_routing, check_y, dev, gpu_forward, gpu_route, log, upload

pytestmark = [pytest.mark.gpu, pytest.mark.slow]

@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", ["step35_decode_m1", "step35_verify_m4", "step5_verify_m4",
                                  "step5_q2k_verify_m4", "step5_q2kp2_verify_m4",
                                  "step35_q6k_verify_m4", "step5_prefill_m512",
                                  "step5_q2kp2_prefill_m512", "step5_q6k_prefill_m512"])
def test_full_config(name):
    cfg = synth.CONFIGS[name]
    log(f"[{name}] drawing layer")
    inp = synth.draw_layer(cfg)
    x, attempts = conditioned_tokens(inp)
    log(f"[{name}] tokens drawn, redraws = {sum(attempts)}")
    w = upload(inp)
    y, ids, tw = gpu_forward(cfg, w, x)
    log(f"[{name}] GPU done")
    ref = run_oracle(inp, x, workers=oracle_workers())
    log(f"[{name}] oracle done, distinct experts = {len(ref['active'])}")
    check_routing(ids, tw, ref)
    assert ref["tokens"] == list(range(cfg.n_tokens))
    check_y(y, ref["y"], name)
    if name in ("step5_verify_m4", "step5_q2k_verify_m4", "step5_q2kp2_verify_m4"):
        assert len(ref["active"]) == 32
    # Routing lists of the whole batch, exactly.
    r = gpu_route(cfg, w.router, x)
    assert np.array_equal(r["counts"], ref["counts"])
    assert np.array_equal(r["offsets"], ref["offsets"])
    assert np.array_equal(r["slots"], ref["slots"])
    assert int(r["n_active"][0]) == len(ref["active"])
    del w, inp
    gc.collect()


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name", ["step35_verify_m4", "step5_verify_m4", "step5_q2k_verify_m4",
                                  "step5_q2kp2_verify_m4"])
def test_verify_batches_of_one_to_four_tokens_agree_bitwise(name):
    # The MTP verify batch is the last accepted token plus up to three drafts,
    # and the draft count changes from round to round ("Support Step3.5/3.7
    # flash mtp3", data-flow trace: the drafting batch grows by one token per
    # head, and adaptive draft lengths shorten it).  Every token's routing
    # and output must not depend on how many drafts share its batch: the
    # rows of a 4-token call equal, bit for bit, the same tokens' rows of
    # 1-, 2- and 3-token calls (and the M=4 result is checked against the
    # oracle in test_full_config).
    cfg = synth.CONFIGS[name]
    log(f"[{name}] drawing layer")
    inp = synth.draw_layer(cfg)
    x, _ = conditioned_tokens(inp)
    w = upload(inp)
    y4, ids4, tw4 = gpu_forward(cfg, w, x)
    for M in (1, 2, 3):
        for t0 in range(0, 4 - M + 1):
            sub = cfg.replace(n_tokens=M)
            y, ids, tw = gpu_forward(sub, w, x[t0:t0 + M])
            log(f"[{name}] M={M} rows {t0}..{t0 + M - 1}")
            assert np.array_equal(ids, ids4[t0:t0 + M])
            assert np.array_equal(tw.view(np.uint32), tw4[t0:t0 + M].view(np.uint32))
            assert np.array_equal(y.view(np.uint32), y4[t0:t0 + M].view(np.uint32))
    del w, inp
    gc.collect()


@pytest.mark.timeout(600)
def test_soak_verify_calls_repeat_bit_for_bit():
    # Repeated calls on one workspace: 2000 calls of the Step-3.5 verify
    # layer, rotating four layer instances, each output (routing ids and
    # weights, y) equal bit for bit to that instance's first output.  The
    # calls exercise the in-launch hand-offs (router keys polled by the
    # routing workgroup and cleared for the next call, the per-pair token
    # words) under back-to-back reuse of the same hand-off areas.
    import torch
    import speculative_verify_router_amd as svr
    from gpu_common import desc_of

    cfg = synth.CONFIGS["step35_verify_m4"]
    M, H, k = cfg.n_tokens, cfg.hidden, cfg.top_k
    insts = []
    for i in range(4):
        log(f"[soak] drawing instance {i}")
        inp = synth.draw_layer(cfg, instance=i)
        x, _ = conditioned_tokens(inp, instance=i)
        insts.append((upload(inp), dev(x)))
        del inp
        gc.collect()
    desc = desc_of(cfg)
    ws = svr.workspace(desc, M, "cuda")
    y = torch.empty((M, H), dtype=torch.float32, device="cuda")
    ids = torch.empty((M, k), dtype=torch.int32, device="cuda")
    tw = torch.empty((M, k), dtype=torch.float32, device="cuda")
    first = []
    for w, x in insts:
        svr.moe_layer_forward(desc, w, x, y, ids, tw, ws=ws)
        first.append((y.clone(), ids.clone(), tw.clone()))
    torch.cuda.synchronize()
    n_calls, check_every = 2000, 50
    bad = torch.zeros((), dtype=torch.int64, device="cuda")
    for n in range(n_calls):
        i = n % 4
        w, x = insts[i]
        svr.moe_layer_forward(desc, w, x, y, ids, tw, ws=ws)
        y0, ids0, tw0 = first[i]
        bad += (y.view(torch.int32) != y0.view(torch.int32)).sum()
        bad += (ids != ids0).sum() + (tw.view(torch.int32) != tw0.view(torch.int32)).sum()
        if (n + 1) % check_every == 0:
            torch.cuda.synchronize()
            assert int(bad.item()) == 0, f"mismatch by call {n}"
            if (n + 1) % 500 == 0:
                log(f"[soak] {n + 1} calls equal")
    assert int(ws[:4].view(torch.int32).item()) == 0  # no routing wait gave up
