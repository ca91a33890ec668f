"""Seeded generator for the routed-MoE layer's inputs.

Shapes follow the model cards the layer is taken from: Step-5 has hidden size
4096 and 352 routed experts with 8 selected per token ("Step-5 Preview GGUF",
Model background, configuration table); routers are kept in F32, shared
experts in Q8_0 and routed experts in Q4_K ("Step-5 Preview GGUF", Precision
distribution table; "Step 3.7 Flash Mixed-Quant GGUF", Tensor recipe); the
verify batch is the last accepted token plus three drafts ("Support
Step3.5/3.7 flash mtp3", Overview, data-flow trace, target batch step).

Byte layouts (planar block quantisation) are those documented in
``include/moe_layer.h``:

* Q8_0, R rows x K columns, K % 32 == 0, nb = K / 32: a scale plane of R*nb
  fp16 values (row-major) at byte 0, then, at ``q8_0_quant_offset(R, K)``
  (the scale plane size rounded up to 256 bytes), R*K int8 quants
  (row-major).  W[r][c] = d[r][c // 32] * q[r][c].
* Q4_K, R rows x K columns, K % 256 == 0, ns = K / 256: a header plane of
  R*ns 16-byte records (fp16 d, fp16 dmin, 12 bytes holding a 96-bit
  little-endian stream whose bits [6s, 6s+6) are the scale and bits
  [48+6s, 54+6s) the min of sub-block s), then R*ns 128-byte quant records;
  sub-block s of a record occupies bytes [16s, 16s+16) and weight i of the
  sub-block sits in byte i // 2, low nibble for even i.
  W = d * sc_s * q - dmin * m_s.
* Q2_K, R rows x K columns, K % 256 == 0, ns = K / 256: a plane of R*ns
  4-byte records (fp16 d, fp16 dmin) at byte 0; at ``q2_k_scale_offset``
  (that plane's size rounded up to 256 bytes) a plane of R*ns 16-byte scale
  records, byte s holding the scale of sub-block s in its low nibble and the
  min in its high nibble; at ``q2_k_quant_offset`` (scale plane end rounded
  up to 256) R*ns 64-byte quant records, sub-block s (16 weights) in bytes
  [4s, 4s+4) and weight i of it in byte i % 4, bits [2 (i // 4), 2 (i // 4) + 2).
  W = d * sc_s * q - dmin * m_s.
* Q3_K, R rows x K columns, K % 256 == 0, ns = K / 256: a plane of R*ns fp16
  d at byte 0; at ``q3_k_scale_offset`` (rounded up to 256) R*ns 16-byte
  scale records, byte s = S_s (6 bits); at ``q3_k_low_offset`` the low two
  bits of every quant, 64 bytes per record laid out as the Q2_K quants; at
  ``q3_k_high_offset`` the high bit of every quant, 32 bytes per record,
  weight i of sub-block s in byte 4 (s // 2) + i % 4, bit 4 (s % 2) + i // 4.
  W = d * (S_s - 32) * (Q - 4) with Q = low | high << 2.
* Q6_K, R rows x K columns, K % 256 == 0, ns = K / 256: a plane of R*ns fp16
  d at byte 0; at ``q6_k_scale_offset`` R*ns 16-byte records of int8
  scales; at ``q6_k_low_offset`` the low four bits of every quant, 128
  bytes per record laid out as the Q4_K quants; at ``q6_k_high_offset``
  the high two bits, 64 bytes per record, weight i of 32-weight group g at
  byte 8g + 4 (i // 16) + (i % 8) // 2, bit 4 ((i // 8) % 2) + 2 (i % 2).
  W = d * sc_s * (Q - 32) with Q = low | high << 4, s = 2g + i // 16.

Nothing here routes, dequantises or multiplies: those steps belong to the
oracle and to the HIP library.
"""

from __future__ import annotations

import concurrent.futures as _cf
import dataclasses
import os
from typing import Callable, Optional

import numpy as np

# Tensor identifiers used to key the seed tree.
_T_ROUTER, _T_GATE, _T_UP, _T_DOWN = 1, 2, 3, 4
_T_SH_GATE, _T_SH_UP, _T_SH_DOWN, _T_TOKENS = 5, 6, 7, 8

_MASTER_SEED = 20261202


@dataclasses.dataclass(frozen=True)
class LayerConfig:
    """One routed-MoE layer workload.

    ``routing`` is "iid" (tokens drawn independently) or "disjoint" (token t
    is redrawn until its top-k set avoids those of tokens < t; the predicate
    that decides this is supplied by the caller, see ``draw_tokens``).
    """

    name: str
    hidden: int
    n_experts: int
    top_k: int
    ffn: int
    shared_ffn: int
    expert_type: str  # "q8_0" | "q4_k" | "q2_k" | "q3_k" | "q6_k"
    shared_type: str  # "q8_0" | "q4_k" (ignored when shared_ffn == 0)
    n_tokens: int
    router_std: float
    weight_std: float  # std of the normal draw that Q8_0 tensors quantise
    routing: str = "iid"
    seed_index: int = 0
    down_type: Optional[str] = None  # routed down type; None: expert_type

    @property
    def routed_down_type(self) -> str:
        return self.down_type or self.expert_type

    @property
    def seed(self) -> int:
        return _MASTER_SEED + self.seed_index

    def replace(self, **kw) -> "LayerConfig":
        return dataclasses.replace(self, **kw)


# The workloads; the last positional index keys the seed.
CONFIGS = {
    # Tiny seed-generated layer (parity only): H 256, 8 experts, top-2, F 128.
    "tiny": LayerConfig("tiny", 256, 8, 2, 128, 0, "q8_0", "q8_0", 1, 0.5, 0.02, "iid", 1),
    # Step-3.5-Flash-shaped decode, one token, everything Q8_0.
    "step35_decode_m1": LayerConfig(
        "step35_decode_m1", 4096, 288, 8, 1280, 1280, "q8_0", "q8_0", 1, 0.02, 0.02, "iid", 2),
    # Same layer as the MTP verify batch: 1 accepted token + 3 drafts.
    "step35_verify_m4": LayerConfig(
        "step35_verify_m4", 4096, 288, 8, 1280, 1280, "q4_k", "q8_0", 4, 0.02, 0.02, "iid", 3),
    # Step-5-shaped verify batch with the four tokens on disjoint experts.
    "step5_verify_m4": LayerConfig(
        "step5_verify_m4", 4096, 352, 8, 1536, 1536, "q4_k", "q8_0", 4, 0.02, 0.02, "disjoint", 4),
    # Step-5-shaped prefill micro-batch of 512 tokens.
    "step5_prefill_m512": LayerConfig(
        "step5_prefill_m512", 4096, 352, 8, 1536, 1536, "q4_k", "q8_0", 512, 0.02, 0.02, "iid", 5),
    # The Step-5 verify batch with 2-bit routed experts (the Q2_K routed
    # matrices of the "Step-5 Preview GGUF" Q2 recipes, Tensor-type table).
    "step5_q2k_verify_m4": LayerConfig(
        "step5_q2k_verify_m4", 4096, 352, 8, 1536, 1536, "q2_k", "q8_0", 4, 0.02, 0.02, "disjoint", 6),
    # The same verify batch with the routed types of the Q2_K-Protected2
    # recipe: Q2_K gate/up, Q3_K down ("Step-5 Preview GGUF", Tensor-type
    # table), shared expert Q8_0.
    "step5_q2kp2_verify_m4": LayerConfig(
        "step5_q2kp2_verify_m4", 4096, 352, 8, 1536, 1536, "q2_k", "q8_0", 4, 0.02, 0.02, "disjoint",
        7, "q3_k"),
    # The Step-3.5 verify batch with 6-bit routed experts (Q6_K is the
    # recipes' type for the MTP heads' matrices, "Step-5 Preview GGUF",
    # Tensor-type table).
    "step35_q6k_verify_m4": LayerConfig(
        "step35_q6k_verify_m4", 4096, 288, 8, 1280, 1280, "q6_k", "q8_0", 4, 0.02, 0.02, "iid", 8),
    # The Step-5 prefill micro-batch with the Q2_K-Protected2 routed types
    # (Q2_K gate/up, Q3_K down) and with Q6_K routed experts.
    "step5_q2kp2_prefill_m512": LayerConfig(
        "step5_q2kp2_prefill_m512", 4096, 352, 8, 1536, 1536, "q2_k", "q8_0", 512, 0.02, 0.02, "iid",
        9, "q3_k"),
    "step5_q6k_prefill_m512": LayerConfig(
        "step5_q6k_prefill_m512", 4096, 352, 8, 1536, 1536, "q6_k", "q8_0", 512, 0.02, 0.02, "iid", 10),
}


# --------------------------------------------------------------------------
# Layout sizes
# --------------------------------------------------------------------------

def q8_0_quant_offset(rows: int, cols: int) -> int:
    """Byte offset of the int8 quant plane in a planar Q8_0 tensor."""
    scale_bytes = 2 * rows * (cols // 32)
    return (scale_bytes + 255) // 256 * 256


def q8_0_bytes(rows: int, cols: int) -> int:
    return q8_0_quant_offset(rows, cols) + rows * cols


def q4_k_header_bytes(rows: int, cols: int) -> int:
    return 16 * rows * (cols // 256)


def q4_k_bytes(rows: int, cols: int) -> int:
    return 144 * rows * (cols // 256)


def q2_k_scale_offset(rows: int, cols: int) -> int:
    """Byte offset of the scale plane in a planar Q2_K tensor."""
    return (4 * rows * (cols // 256) + 255) // 256 * 256


def q2_k_quant_offset(rows: int, cols: int) -> int:
    """Byte offset of the 2-bit quant plane in a planar Q2_K tensor."""
    return (q2_k_scale_offset(rows, cols) + 16 * rows * (cols // 256) + 255) // 256 * 256


def q2_k_bytes(rows: int, cols: int) -> int:
    return q2_k_quant_offset(rows, cols) + 64 * rows * (cols // 256)


def q3_k_scale_offset(rows: int, cols: int) -> int:
    return (2 * rows * (cols // 256) + 255) // 256 * 256


def q3_k_low_offset(rows: int, cols: int) -> int:
    return (q3_k_scale_offset(rows, cols) + 16 * rows * (cols // 256) + 255) // 256 * 256


def q3_k_high_offset(rows: int, cols: int) -> int:
    return (q3_k_low_offset(rows, cols) + 64 * rows * (cols // 256) + 255) // 256 * 256


def q3_k_bytes(rows: int, cols: int) -> int:
    return q3_k_high_offset(rows, cols) + 32 * rows * (cols // 256)


def q6_k_scale_offset(rows: int, cols: int) -> int:
    return (2 * rows * (cols // 256) + 255) // 256 * 256


def q6_k_low_offset(rows: int, cols: int) -> int:
    return (q6_k_scale_offset(rows, cols) + 16 * rows * (cols // 256) + 255) // 256 * 256


def q6_k_high_offset(rows: int, cols: int) -> int:
    return (q6_k_low_offset(rows, cols) + 128 * rows * (cols // 256) + 255) // 256 * 256


def q6_k_bytes(rows: int, cols: int) -> int:
    return q6_k_high_offset(rows, cols) + 64 * rows * (cols // 256)


def tensor_bytes(dtype: str, rows: int, cols: int) -> int:
    if dtype == "q8_0":
        if cols % 32:
            raise ValueError("Q8_0 needs cols % 32 == 0")
        return q8_0_bytes(rows, cols)
    if dtype == "q4_k":
        if cols % 256:
            raise ValueError("Q4_K needs cols % 256 == 0")
        return q4_k_bytes(rows, cols)
    if dtype == "q2_k":
        if cols % 256:
            raise ValueError("Q2_K needs cols % 256 == 0")
        return q2_k_bytes(rows, cols)
    if dtype == "q3_k":
        if cols % 256:
            raise ValueError("Q3_K needs cols % 256 == 0")
        return q3_k_bytes(rows, cols)
    if dtype == "q6_k":
        if cols % 256:
            raise ValueError("Q6_K needs cols % 256 == 0")
        return q6_k_bytes(rows, cols)
    if dtype == "f32":
        return 4 * rows * cols
    raise ValueError(f"unknown dtype {dtype!r}")


# --------------------------------------------------------------------------
# Encoders (the generator's side of the format)
# --------------------------------------------------------------------------

def quantize_q8_0(w: np.ndarray):
    """Quantise rows of ``w`` [R][K] to Q8_0 fields.

    Per 32-weight block: d = fp16(max|w| / 127) (round to nearest even),
    q = clamp(round_half_away(w / d), -127, 127), q = 0 where d == 0.
    Returns (d_bits uint16 [R][K/32], q int8 [R][K]).
    """
    w = np.asarray(w, dtype=np.float32)
    R, K = w.shape
    blk = w.reshape(R, K // 32, 32)
    amax = np.abs(blk).max(axis=2)
    d16 = (amax / np.float32(127.0)).astype(np.float16)
    d = d16.astype(np.float32)[..., None]
    safe = np.where(d > 0, d, np.float32(1.0))
    v = blk / safe
    q = np.sign(v) * np.floor(np.abs(v) + np.float32(0.5))
    q = np.where(d > 0, np.clip(q, -127, 127), 0).astype(np.int8)
    return d16.view(np.uint16), q.reshape(R, K)


def _fill_q8_0(buf: np.ndarray, rows_total: int, cols: int, row0: int, d_bits, q):
    nb = cols // 32
    R = q.shape[0]
    scales = buf[: 2 * rows_total * nb].view(np.uint16)
    scales[row0 * nb:(row0 + R) * nb] = d_bits.reshape(-1)
    qo = q8_0_quant_offset(rows_total, cols)
    buf[qo + row0 * cols: qo + (row0 + R) * cols] = q.reshape(-1).view(np.uint8)


def _draw_q8_0_rows(rng: np.random.Generator, rows: int, cols: int, std: float):
    w = rng.standard_normal((rows, cols), dtype=np.float32) * np.float32(std)
    return quantize_q8_0(w)


def _draw_q4_k_rows(rng: np.random.Generator, rows: int, cols: int):
    """Uniform-random Q4_K fields for ``rows`` rows.

    d ~ U[2^-14, 2^-12), dmin ~ U[2^-12, 2^-10), both rounded to fp16; the
    twelve scale/min bytes and the 128 quant bytes are uniform random bytes,
    which makes every 6-bit field uniform on 0..63 and every nibble uniform
    on 0..15.
    """
    ns = cols // 256
    n = rows * ns
    hdr = np.empty((n, 16), dtype=np.uint8)
    d = rng.uniform(2.0 ** -14, 2.0 ** -12, n).astype(np.float16)
    dmin = rng.uniform(2.0 ** -12, 2.0 ** -10, n).astype(np.float16)
    hdr[:, 0:2] = d.view(np.uint16).reshape(n, 1).view(np.uint8)
    hdr[:, 2:4] = dmin.view(np.uint16).reshape(n, 1).view(np.uint8)
    hdr[:, 4:16] = rng.integers(0, 256, (n, 12), dtype=np.uint8)
    qs = rng.integers(0, 256, (n, 128), dtype=np.uint8)
    return hdr, qs


def _fill_q4_k(buf: np.ndarray, rows_total: int, cols: int, row0: int, hdr, qs):
    ns = cols // 256
    hb = q4_k_header_bytes(rows_total, cols)
    n = hdr.shape[0]
    s0 = row0 * ns
    buf[16 * s0: 16 * (s0 + n)] = hdr.reshape(-1)
    buf[hb + 128 * s0: hb + 128 * (s0 + n)] = qs.reshape(-1)


def _draw_q2_k_rows(rng: np.random.Generator, rows: int, cols: int):
    """Uniform-random Q2_K fields for ``rows`` rows.

    d ~ U[2^-10, 2^-8), dmin ~ U[2^-10, 2^-8), both rounded to fp16 (weights
    of a few hundredths, as the Q4_K draw gives); the scale bytes and the
    quant bytes are uniform random bytes, so every 4-bit scale and min is
    uniform on 0..15 and every 2-bit quant on 0..3.
    """
    n = rows * (cols // 256)
    dd = np.empty((n, 4), dtype=np.uint8)
    d = rng.uniform(2.0 ** -10, 2.0 ** -8, n).astype(np.float16)
    dmin = rng.uniform(2.0 ** -10, 2.0 ** -8, n).astype(np.float16)
    dd[:, 0:2] = d.view(np.uint16).reshape(n, 1).view(np.uint8)
    dd[:, 2:4] = dmin.view(np.uint16).reshape(n, 1).view(np.uint8)
    sc = rng.integers(0, 256, (n, 16), dtype=np.uint8)
    qs = rng.integers(0, 256, (n, 64), dtype=np.uint8)
    return dd, sc, qs


def _fill_q2_k(buf: np.ndarray, rows_total: int, cols: int, row0: int, dd, sc, qs):
    ns = cols // 256
    so = q2_k_scale_offset(rows_total, cols)
    qo = q2_k_quant_offset(rows_total, cols)
    n = dd.shape[0]
    s0 = row0 * ns
    buf[4 * s0: 4 * (s0 + n)] = dd.reshape(-1)
    buf[so + 16 * s0: so + 16 * (s0 + n)] = sc.reshape(-1)
    buf[qo + 64 * s0: qo + 64 * (s0 + n)] = qs.reshape(-1)


def _draw_q3_k_rows(rng: np.random.Generator, rows: int, cols: int):
    """Uniform-random Q3_K fields for ``rows`` rows.

    d ~ U[2^-11, 2^-9) rounded to fp16 (weights of a few hundredths); every
    scale uniform on 0..63, every low and high quant byte uniform, so every
    3-bit quant is uniform on 0..7.
    """
    n = rows * (cols // 256)
    d = rng.uniform(2.0 ** -11, 2.0 ** -9, n).astype(np.float16)
    sc = rng.integers(0, 64, (n, 16), dtype=np.uint8)
    lo = rng.integers(0, 256, (n, 64), dtype=np.uint8)
    hi = rng.integers(0, 256, (n, 32), dtype=np.uint8)
    return d.view(np.uint16).reshape(n, 1).view(np.uint8), sc, lo, hi


def _fill_q3_k(buf: np.ndarray, rows_total: int, cols: int, row0: int, d, sc, lo, hi):
    ns = cols // 256
    n = d.shape[0]
    s0 = row0 * ns
    so = q3_k_scale_offset(rows_total, cols)
    lo_off = q3_k_low_offset(rows_total, cols)
    hi_off = q3_k_high_offset(rows_total, cols)
    buf[2 * s0: 2 * (s0 + n)] = d.reshape(-1)
    buf[so + 16 * s0: so + 16 * (s0 + n)] = sc.reshape(-1)
    buf[lo_off + 64 * s0: lo_off + 64 * (s0 + n)] = lo.reshape(-1)
    buf[hi_off + 32 * s0: hi_off + 32 * (s0 + n)] = hi.reshape(-1)


def _draw_q6_k_rows(rng: np.random.Generator, rows: int, cols: int):
    """Uniform-random Q6_K fields for ``rows`` rows.

    d ~ U[2^-14, 2^-12) rounded to fp16; every scale uniform on -128..127
    and every quant byte uniform, so every 6-bit quant is uniform on 0..63
    (weights of a few hundredths).
    """
    n = rows * (cols // 256)
    d = rng.uniform(2.0 ** -14, 2.0 ** -12, n).astype(np.float16)
    sc = rng.integers(0, 256, (n, 16), dtype=np.uint8)
    lo = rng.integers(0, 256, (n, 128), dtype=np.uint8)
    hi = rng.integers(0, 256, (n, 64), dtype=np.uint8)
    return d.view(np.uint16).reshape(n, 1).view(np.uint8), sc, lo, hi


def _fill_q6_k(buf: np.ndarray, rows_total: int, cols: int, row0: int, d, sc, lo, hi):
    ns = cols // 256
    n = d.shape[0]
    s0 = row0 * ns
    so = q6_k_scale_offset(rows_total, cols)
    lo_off = q6_k_low_offset(rows_total, cols)
    hi_off = q6_k_high_offset(rows_total, cols)
    buf[2 * s0: 2 * (s0 + n)] = d.reshape(-1)
    buf[so + 16 * s0: so + 16 * (s0 + n)] = sc.reshape(-1)
    buf[lo_off + 128 * s0: lo_off + 128 * (s0 + n)] = lo.reshape(-1)
    buf[hi_off + 64 * s0: hi_off + 64 * (s0 + n)] = hi.reshape(-1)


def _rng(cfg: LayerConfig, instance: int, *key: int) -> np.random.Generator:
    ss = np.random.SeedSequence([cfg.seed, instance, *key])
    return np.random.Generator(np.random.PCG64(ss))


# --------------------------------------------------------------------------
# Whole-layer inputs
# --------------------------------------------------------------------------

@dataclasses.dataclass
class LayerInputs:
    cfg: LayerConfig
    router: np.ndarray            # float32 [E][H]
    gate: np.ndarray              # uint8, E*F rows x H cols
    up: np.ndarray                # uint8, E*F rows x H cols
    down: np.ndarray              # uint8, E*H rows x F cols
    shared_gate: Optional[np.ndarray] = None   # Fs x H
    shared_up: Optional[np.ndarray] = None     # Fs x H
    shared_down: Optional[np.ndarray] = None   # H x Fs


def _stacked(cfg: LayerConfig, instance: int, tid: int, rows: int, cols: int,
             dtype: str, n_exp: int, pool) -> np.ndarray:
    total_rows = n_exp * rows
    buf = np.zeros(tensor_bytes(dtype, total_rows, cols), dtype=np.uint8)

    def one(e):
        rng = _rng(cfg, instance, tid, e)
        if dtype == "q8_0":
            d_bits, q = _draw_q8_0_rows(rng, rows, cols, cfg.weight_std)
            _fill_q8_0(buf, total_rows, cols, e * rows, d_bits, q)
        elif dtype == "q4_k":
            hdr, qs = _draw_q4_k_rows(rng, rows, cols)
            _fill_q4_k(buf, total_rows, cols, e * rows, hdr, qs)
        elif dtype == "q2_k":
            dd, sc, qs = _draw_q2_k_rows(rng, rows, cols)
            _fill_q2_k(buf, total_rows, cols, e * rows, dd, sc, qs)
        elif dtype == "q3_k":
            _fill_q3_k(buf, total_rows, cols, e * rows, *_draw_q3_k_rows(rng, rows, cols))
        elif dtype == "q6_k":
            _fill_q6_k(buf, total_rows, cols, e * rows, *_draw_q6_k_rows(rng, rows, cols))
        else:
            raise ValueError(f"unknown dtype {dtype!r}")

    if pool is None or n_exp == 1:
        for e in range(n_exp):
            one(e)
    else:
        list(pool.map(one, range(n_exp)))
    return buf


def draw_layer(cfg: LayerConfig, instance: int = 0, threads: Optional[int] = None) -> LayerInputs:
    """Draw router, routed experts and shared expert for ``cfg``.

    Every expert matrix has its own seed (config seed, instance, tensor,
    expert), so the result does not depend on ``threads``.
    """
    H, E, F, Fs = cfg.hidden, cfg.n_experts, cfg.ffn, cfg.shared_ffn
    router = (_rng(cfg, instance, _T_ROUTER, 0).standard_normal((E, H), dtype=np.float32)
              * np.float32(cfg.router_std))
    nthreads = threads if threads is not None else min(8, os.cpu_count() or 1)
    pool = _cf.ThreadPoolExecutor(nthreads) if nthreads > 1 else None
    try:
        et = cfg.expert_type
        gate = _stacked(cfg, instance, _T_GATE, F, H, et, E, pool)
        up = _stacked(cfg, instance, _T_UP, F, H, et, E, pool)
        down = _stacked(cfg, instance, _T_DOWN, H, F, cfg.routed_down_type, E, pool)
        sg = su = sd = None
        if Fs > 0:
            st = cfg.shared_type
            sg = _stacked(cfg, instance, _T_SH_GATE, Fs, H, st, 1, None)
            su = _stacked(cfg, instance, _T_SH_UP, Fs, H, st, 1, None)
            sd = _stacked(cfg, instance, _T_SH_DOWN, H, Fs, st, 1, None)
    finally:
        if pool is not None:
            pool.shutdown()
    return LayerInputs(cfg, router, gate, up, down, sg, su, sd)


def draw_tokens(cfg: LayerConfig, instance: int = 0,
                accept: Optional[Callable[[np.ndarray, int, list], bool]] = None,
                n_tokens: Optional[int] = None, max_attempts: int = 10000):
    """Draw activations x [M][H] ~ N(0, 1), float32.

    Token t, attempt a is drawn from its own seed (config seed, instance,
    tokens, t, a).  If ``accept`` is given, token t is redrawn until
    ``accept(x_t, t, accepted_rows)`` returns True; the predicate (e.g. a
    router-logit margin or a disjoint-experts rule) is supplied by the caller
    so that this module holds no routing arithmetic.

    Returns (x, attempts) where attempts[t] is the number of redraws.
    """
    M = cfg.n_tokens if n_tokens is None else n_tokens
    H = cfg.hidden
    x = np.empty((M, H), dtype=np.float32)
    attempts = []
    rows = []
    for t in range(M):
        for a in range(max_attempts):
            xt = _rng(cfg, instance, _T_TOKENS, t, a).standard_normal(H, dtype=np.float32)
            if accept is None or accept(xt, t, rows):
                break
        else:
            raise RuntimeError(f"token {t}: no acceptable draw in {max_attempts} attempts")
        x[t] = xt
        rows.append(xt)
        attempts.append(a)
    return x, attempts
