"""Helpers for the GPU tests: device upload, calls through the C ABI, checks."""

from __future__ import annotations

import sys

import numpy as np
import torch

import speculative_verify_router_amd as svr

# Output tolerance: max |y - y_ref| <= 2e-3 * RMS(y_ref) over the whole
# [M][H] output (fp32-accumulated outputs against the fp64 oracle).
Y_TOL = 2e-3
# Routing weights: fp32 against fp64, absolute: 1e-6 for the fp32 softmax,
# plus what the fp32 logits carry.  A logit of magnitude L is a sum whose
# partial sums round at a few ulp(L) ~ 2^-23 L each; the renormalised
# softmax passes at most half of a logit error on to any weight.  Four such
# roundings of the token's largest logit: 2^-22 max|l|.
W_TOL = 1e-6


def w_tolerance(ref) -> np.ndarray:
    """Per-token tolerance of the routing weights, [M][1]."""
    lmax = np.max(np.abs(np.atleast_2d(ref["logits"])), axis=1, keepdims=True)
    return W_TOL + 2.0 ** -22 * lmax


def log(msg: str):
    print(msg, file=sys.stderr, flush=True)


def desc_of(cfg) -> svr.LayerDesc:
    return svr.LayerDesc(cfg.hidden, cfg.n_experts, cfg.top_k, cfg.ffn, cfg.shared_ffn,
                         cfg.expert_type, cfg.shared_type, down_type=cfg.down_type)


def dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda")


def upload(inp) -> svr.LayerWeights:
    c = inp.cfg
    w = svr.LayerWeights(dev(inp.router), dev(inp.gate), dev(inp.up), dev(inp.down))
    if c.shared_ffn > 0:
        w.shared_gate, w.shared_up, w.shared_down = (dev(inp.shared_gate), dev(inp.shared_up),
                                                     dev(inp.shared_down))
    return w


def gpu_forward(cfg, weights, x: np.ndarray, desc=None):
    M = x.shape[0]
    xd = dev(x.astype(np.float32))
    y = torch.empty((M, cfg.hidden), dtype=torch.float32, device="cuda")
    ids = torch.empty((M, cfg.top_k), dtype=torch.int32, device="cuda")
    tw = torch.empty((M, cfg.top_k), dtype=torch.float32, device="cuda")
    svr.moe_layer_forward(desc or desc_of(cfg), weights, xd, y, ids, tw)
    torch.cuda.synchronize()
    return y.cpu().numpy(), ids.cpu().numpy(), tw.cpu().numpy()


def gpu_route(cfg, router: torch.Tensor, x: np.ndarray):
    M, E, k = x.shape[0], cfg.n_experts, cfg.top_k
    i32 = dict(dtype=torch.int32, device="cuda")
    out = dict(ids=torch.empty((M, k), **i32),
               w=torch.empty((M, k), dtype=torch.float32, device="cuda"),
               counts=torch.empty(E, **i32), offsets=torch.empty(E + 1, **i32),
               slots=torch.empty(max(M * k, 1), **i32), active=torch.empty(E, **i32),
               n_active=torch.empty(1, **i32))
    svr.moe_route(desc_of(cfg), router, dev(x.astype(np.float32)), out["ids"], out["w"],
                  out["counts"], out["offsets"], out["slots"], out["active"], out["n_active"])
    torch.cuda.synchronize()
    return {k_: v.cpu().numpy() for k_, v in out.items()}


def check_y(y, y_ref, what=""):
    rms = float(np.sqrt(np.mean(np.asarray(y_ref, np.float64) ** 2)))
    err = float(np.max(np.abs(np.asarray(y, np.float64) - y_ref)))
    log(f"  {what} max|err| = {err:.3e}, rms = {rms:.3e}, ratio = {err / max(rms, 1e-300):.3e}")
    assert np.all(np.isfinite(y)), "non-finite output"
    assert err <= Y_TOL * rms, f"{what}: max|err| {err:.3e} > {Y_TOL} * rms {rms:.3e}"


def check_routing(ids, w, ref):
    assert np.array_equal(ids, ref["ids"]), f"ids differ:\n{ids}\nvs\n{ref['ids']}"
    err = np.abs(w - ref["w"])
    assert np.all(err <= w_tolerance(ref)), (np.max(err), np.max(w_tolerance(ref)))
