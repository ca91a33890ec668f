"""Shared helpers for the tests: fixtures, input conditioning, layout edits.

The conditioning predicates decide routing margins with the oracle's router
(tests may call the oracle); the generator only draws candidates.
"""

from __future__ import annotations

import os

import numpy as np

from oracle import moe_oracle as om
import synth

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def read_fixture(name: str):
    rows = cols = nbytes = None
    hexes, expects = [], []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            tok = line.split()
            if tok[0] == "rows":
                rows = int(tok[1])
            elif tok[0] == "cols":
                cols = int(tok[1])
            elif tok[0] == "bytes":
                nbytes = int(tok[1])
            elif tok[0] == "hex":
                hexes.append((int(tok[1]), bytes(int(b, 16) for b in tok[2:])))
            elif tok[0] == "expect":
                expects.append((int(tok[1]), int(tok[2]), float(tok[3])))
    buf = np.zeros(nbytes, dtype=np.uint8)
    for off, bs in hexes:
        buf[off:off + len(bs)] = np.frombuffer(bs, dtype=np.uint8)
    return rows, cols, buf, expects


def oracle_kwargs(inp) -> dict:
    c = inp.cfg
    kw = dict(top_k=c.top_k, ffn=c.ffn, expert_type=c.expert_type)
    if c.down_type:
        kw.update(down_type=c.down_type)
    if c.shared_ffn > 0:
        kw.update(shared=(inp.shared_gate, inp.shared_up, inp.shared_down),
                  shared_ffn=c.shared_ffn, shared_type=c.shared_type)
    return kw


def oracle_workers() -> int:
    """Threads for the oracle's per-expert loop: the host's cores, at most 16."""
    return max(1, min(16, os.cpu_count() or 1))


def run_oracle(inp, x, tokens=None, workers: int = 1) -> dict:
    if workers <= 1:
        return om.moe_layer(x, inp.router, inp.gate, inp.up, inp.down, tokens=tokens,
                            **oracle_kwargs(inp))
    # One BLAS thread per oracle thread: nested BLAS pools oversubscribe the host.
    from threadpoolctl import threadpool_limits
    with threadpool_limits(1):
        return om.moe_layer(x, inp.router, inp.gate, inp.up, inp.down, tokens=tokens,
                            workers=workers, **oracle_kwargs(inp))


def routing_predicate(router, k: int, margin: float = 1e-4, disjoint: bool = False):
    """accept(x_t, t, rows) for synth.draw_tokens.

    Accepts a candidate token when, in float64 router logits, every gap
    between consecutive entries of its top-(k+1) sorted logits is >= margin
    (so selection and order are decided with room to spare) and, if
    ``disjoint``, its top-k set shares no expert with earlier tokens.
    """
    R = np.asarray(router, dtype=np.float32)
    E = R.shape[0]
    used = set()

    def accept(xt, t, rows):
        if t == 0:
            used.clear()
        l = om.router_logits(R, xt[None, :])[0]
        top = np.sort(l)[::-1][: min(k + 1, E)]
        if top.size > 1 and np.min(top[:-1] - top[1:]) < margin:
            return False
        if disjoint:
            chosen = set(int(e) for e in om.select_experts(l[None, :], k)[0])
            if chosen & used:
                return False
            used.update(chosen)
        return True

    return accept


def conditioned_tokens(inp, instance: int = 0, n_tokens=None, margin: float = 1e-4):
    c = inp.cfg
    pred = routing_predicate(inp.router, c.top_k, margin, disjoint=(c.routing == "disjoint"))
    return synth.draw_tokens(c, instance, accept=pred, n_tokens=n_tokens)


# --------------------------------------------------------------------------
# Layout edits used by edge-case tests (they follow the documented layout).
# --------------------------------------------------------------------------

def scale_fields(dtype: str, buf: np.ndarray, rows: int, cols: int) -> np.ndarray:
    """uint16 view of every fp16 scale field (Q8_0 d; Q4_K and Q2_K d and dmin)."""
    if dtype == "q8_0":
        return buf[: 2 * rows * (cols // 32)].view(np.uint16)
    n = rows * (cols // 256)
    if dtype == "q2_k":
        return buf[: 4 * n].view(np.uint16).reshape(n, 2)
    if dtype in ("q3_k", "q6_k"):
        return buf[: 2 * n].view(np.uint16).reshape(n, 1)
    return buf[: 16 * n].view(np.uint16).reshape(n, 8)[:, 0:2]


def double_scales(dtype: str, buf: np.ndarray, rows: int, cols: int) -> np.ndarray:
    """Copy of ``buf`` with every fp16 scale multiplied by 2 (exponent + 1).

    Valid only for normal, finite scales below 32768.
    """
    out = buf.copy()
    f = scale_fields(dtype, out, rows, cols)
    v = f.astype(np.int64)
    e = (v >> 10) & 31
    assert np.all((e >= 1) & (e <= 29)), "scales must be normal and small"
    f[...] = (v + (1 << 10)).astype(np.uint16)
    return out


def copy_expert_rows(dtype: str, buf: np.ndarray, rows_per_expert: int, cols: int,
                     n_experts: int, src: int = 0) -> np.ndarray:
    """Copy of a stacked tensor in which every expert equals expert ``src``."""
    out = buf.copy()
    R = rows_per_expert * n_experts
    if dtype == "q8_0":
        nb = cols // 32
        sp = out[: 2 * R * nb].view(np.uint16).reshape(n_experts, rows_per_expert * nb)
        sp[:] = sp[src]
        qo = synth.q8_0_quant_offset(R, cols)
        qp = out[qo: qo + R * cols].reshape(n_experts, rows_per_expert * cols)
        qp[:] = qp[src]
    elif dtype in ("q2_k", "q3_k", "q6_k"):
        ns = cols // 256
        if dtype == "q2_k":
            planes = ((0, 4), (synth.q2_k_scale_offset(R, cols), 16),
                      (synth.q2_k_quant_offset(R, cols), 64))
        elif dtype == "q3_k":
            planes = ((0, 2), (synth.q3_k_scale_offset(R, cols), 16),
                      (synth.q3_k_low_offset(R, cols), 64), (synth.q3_k_high_offset(R, cols), 32))
        else:
            planes = ((0, 2), (synth.q6_k_scale_offset(R, cols), 16),
                      (synth.q6_k_low_offset(R, cols), 128), (synth.q6_k_high_offset(R, cols), 64))
        for start, width in planes:
            pl = out[start: start + R * ns * width].reshape(n_experts, rows_per_expert * ns * width)
            pl[:] = pl[src]
    else:
        ns = cols // 256
        hb = synth.q4_k_header_bytes(R, cols)
        hp = out[:hb].reshape(n_experts, rows_per_expert * ns * 16)
        hp[:] = hp[src]
        qp = out[hb:].reshape(n_experts, rows_per_expert * ns * 128)
        qp[:] = qp[src]
    return out


def small_config(**kw) -> "synth.LayerConfig":
    base = dict(name="custom", hidden=256, n_experts=8, top_k=2, ffn=128, shared_ffn=0,
                expert_type="q8_0", shared_type="q8_0", n_tokens=2, router_std=0.5,
                weight_std=0.02, routing="iid", seed_index=100)
    base.update(kw)
    return synth.LayerConfig(**base)
