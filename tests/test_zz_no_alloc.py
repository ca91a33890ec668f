"""moe_layer_forward_noalloc (the library's own per-GPU workspace) against
moe_layer_forward with a caller workspace: the same kernels on the same
inputs, so ids, weights and outputs agree bit for bit.  Each case makes two
calls in a row, the second on a smaller batch, so that the second call runs
on the scratch contents the first one left."""

import gc

import numpy as np
import pytest
import torch

import speculative_verify_router_amd as svr
import synth
from _support import conditioned_tokens, small_config
from gpu_common import desc_of, dev, log, upload

pytestmark = pytest.mark.gpu


def _call(cfg, w, x, noalloc: bool):
    M = x.shape[0]
    y = torch.full((M, cfg.hidden), float("nan"), dtype=torch.float32, device="cuda")
    ids = torch.full((M, cfg.top_k), -1, dtype=torch.int32, device="cuda")
    tw = torch.full((M, cfg.top_k), float("nan"), dtype=torch.float32, device="cuda")
    if noalloc:
        svr.moe_layer_forward_noalloc(desc_of(cfg), w, dev(x), y, ids, tw)
    else:
        svr.moe_layer_forward(desc_of(cfg), w, dev(x), y, ids, tw)
    torch.cuda.synchronize()
    return y.cpu().numpy(), ids.cpu().numpy(), tw.cpu().numpy()


CASES = [
    # Step-3.5-shaped verify batch (per-pair path), then a 2-token batch.
    ("step35_verify_m4", None, 4, 2),
    # 16 tokens (per-expert path of the small-batch kernels), then 5.
    ("custom", dict(hidden=512, n_experts=16, top_k=4, ffn=256, shared_ffn=256,
                    expert_type="q4_k", n_tokens=16), 16, 5),
    # Batched grouped-GEMM path: 40 tokens, then 20.
    ("custom", dict(hidden=512, n_experts=16, top_k=4, ffn=256, shared_ffn=256,
                    expert_type="q4_k", n_tokens=40), 40, 20),
]


@pytest.mark.parametrize("name,kw,m1,m2", CASES)
def test_noalloc_matches_workspace_forward(name, kw, m1, m2):
    cfg = synth.CONFIGS[name] if kw is None else small_config(**kw)
    cfg = cfg.replace(n_tokens=m1)
    log(f"[noalloc {name} M={m1},{m2}] drawing")
    inp = synth.draw_layer(cfg)
    x, _ = conditioned_tokens(inp)
    w = upload(inp)
    for M, rows in ((m1, x), (m2, x[1:1 + m2])):
        sub = cfg.replace(n_tokens=M)
        assert svr.moe_workspace_bytes(desc_of(sub), M) <= svr.NOALLOC_MAX_WORKSPACE
        ref = _call(sub, w, rows, noalloc=False)
        got = _call(sub, w, rows, noalloc=True)
        log(f"  M={M}: ids equal {np.array_equal(ref[1], got[1])}")
        assert np.array_equal(got[1], ref[1])
        assert np.array_equal(got[2].view(np.uint32), ref[2].view(np.uint32))
        assert np.array_equal(got[0].view(np.uint32), ref[0].view(np.uint32))
    del w, inp
    gc.collect()


def test_noalloc_refuses_a_batch_beyond_its_workspace():
    cfg = synth.CONFIGS["step5_prefill_m512"]
    desc = desc_of(cfg)
    assert svr.moe_workspace_bytes(desc, 512) > svr.NOALLOC_MAX_WORKSPACE
    x = torch.zeros((512, cfg.hidden), dtype=torch.float32, device="cuda")
    y = torch.zeros_like(x)
    dummy = torch.zeros(256, dtype=torch.uint8, device="cuda")
    w = svr.LayerWeights(torch.zeros(16, dtype=torch.float32, device="cuda"), dummy, dummy, dummy,
                         dummy, dummy, dummy)
    with pytest.raises(svr.MoeError) as e:
        svr.moe_layer_forward_noalloc(desc, w, x, y)
    assert e.value.status == 4
