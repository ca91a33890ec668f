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
