"""CPU oracle for the routed-MoE verify layer -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this module.  The HIP library never calls it and it
never calls the HIP library; the two share no code.

Everything is computed in float64 with plain NumPy: dequantise the touched
blocks exactly, then dense products.  What the layer computes:

* The layer is the routed mixture-of-experts FFN of a Step-3.5/3.7-Flash or
  Step-5 transformer block: 352 routed experts of which 8 are selected per
  token at hidden size 4096 for Step-5 ("Step-5 Preview GGUF", Model
  background, configuration table), an F32 router ("Step-5 Preview GGUF",
  Precision distribution table, routers row; "Step 3.7 Flash Mixed-Quant
  GGUF", Tensor recipe, router row), a Q8_0 shared expert beside the routed
  ones (same tables, shared-expert rows) and routed experts in Q4_K ("Step
  3.7 Flash Mixed-Quant GGUF", Tensor recipe, routed rows), or in Q2_K as
  the 2-bit recipes of "Step-5 Preview GGUF" store them (Tensor-type table,
  routed gate/up and down rows; the Q2_K-Protected2 recipe pairs Q2_K
  gate/up with Q3_K down).
* It is run on the verify batch of MTP speculative decoding: the last
  accepted token plus up to three drafts, all with logits ("Support
  Step3.5/3.7 flash mtp3", Overview, data-flow trace, target batch step).

The pages do not write down the router formula, the activation or the
block layouts.  Readings taken here:

* router: softmax over all experts of the F32 logits l = Wr x; the k largest
  logits are selected, ties to the lower expert index, in descending order;
  the selected probabilities are renormalised to sum to one;
* expert FFN: SwiGLU, h = silu(Wg x) * (Wu x), o = Wd h, silu(g) = g/(1+e^-g);
* shared expert: the same FFN, ungated, added with weight one;
* output y_t = s_t + sum_j w_tj o_tj, summed in slot order j = 0..k-1;
* block layouts: the planar Q8_0 / Q4_K / Q2_K / Q3_K / Q6_K layouts documented in
  include/moe_layer.h; Q2_K is read as the K-quant family's 2-bit member:
  256-weight super-blocks with fp16 d and dmin, sixteen 16-weight
  sub-blocks with a 4-bit scale and a 4-bit min, 2-bit quants,
  w = d*sc*q - dmin*m; Q3_K as the 3-bit member without mins: fp16 d,
  sixteen 16-weight sub-blocks with a 6-bit scale S stored with offset 32
  and 3-bit quants Q stored with offset 4, w = d*(S - 32)*(Q - 4); Q6_K as
  the 6-bit member: fp16 d, sixteen 16-weight sub-blocks with a signed
  8-bit scale and 6-bit quants stored with offset 32, w = d*sc*(Q - 32)
  (the recipes' type for the MTP heads' matrices, same table).
"""

from __future__ import annotations

from concurrent.futures import ThreadPoolExecutor

import numpy as np

# ---------------------------------------------------------------------------
# Scalar formats
# ---------------------------------------------------------------------------


def f16_to_f64(bits) -> np.ndarray:
    """IEEE 754 binary16 bit patterns -> float64, from the format definition.

    sign s = bit 15, exponent e = bits 14..10, fraction f = bits 9..0:
    e == 0: (-1)^s * f * 2^-24 (subnormal); e == 31: inf (f == 0) or NaN;
    else (-1)^s * (1024 + f) * 2^(e - 25).
    """
    b = np.asarray(bits).astype(np.int64) & 0xFFFF
    s = np.where(b >> 15, -1.0, 1.0)
    e = (b >> 10) & 31
    f = (b & 1023).astype(np.float64)
    normal = (1024.0 + f) * np.exp2((e - 25).astype(np.float64))
    sub = f * 2.0 ** -24
    special = np.where(f == 0, np.inf, np.nan)
    v = np.where(e == 0, sub, np.where(e == 31, special, normal))
    return s * v


# ---------------------------------------------------------------------------
# Dequantisation (planar layouts, exact in float64)
# ---------------------------------------------------------------------------


def _rows(rows, row_start, row_count):
    if row_count is None:
        row_count = rows - row_start
    if not (0 <= row_start and row_start + row_count <= rows):
        raise ValueError("row range out of bounds")
    return row_start, row_count


def q8_0_quant_offset(rows: int, cols: int) -> int:
    """Start of the int8 plane: the fp16 scale plane rounded up to 256 B."""
    return (2 * rows * (cols // 32) + 255) // 256 * 256


def dequant_q8_0(buf, rows: int, cols: int, row_start: int = 0, row_count=None) -> np.ndarray:
    """Planar Q8_0 -> float64 [row_count][cols].

    Block of 32 weights: w_i = d * q_i with fp16 d and int8 q_i.
    """
    if cols % 32:
        raise ValueError("Q8_0 needs cols % 32 == 0")
    r0, n = _rows(rows, row_start, row_count)
    buf = np.asarray(buf, dtype=np.uint8)
    nb = cols // 32
    sb = buf[2 * r0 * nb: 2 * (r0 + n) * nb].reshape(n * nb, 2).astype(np.int64)
    d = f16_to_f64(sb[:, 0] | (sb[:, 1] << 8)).reshape(n, nb, 1)
    qo = q8_0_quant_offset(rows, cols)
    q = buf[qo + r0 * cols: qo + (r0 + n) * cols].view(np.int8).astype(np.float64)
    return (d * q.reshape(n, nb, 32)).reshape(n, cols)


def _q4_k_field(sbytes: np.ndarray, bit: int) -> np.ndarray:
    """6-bit field starting at ``bit`` of the 96-bit little-endian stream."""
    lo = sbytes[:, bit // 8]
    hi = sbytes[:, bit // 8 + 1] if bit // 8 + 1 < 12 else 0
    return ((lo | (hi << 8)) >> (bit % 8)) & 63


def q4_k_fields(buf, rows: int, cols: int, row_start: int = 0, row_count=None):
    """Decode Q4_K records into (d, dmin, sc[8], m[8], q[8][32]) per record."""
    if cols % 256:
        raise ValueError("Q4_K needs cols % 256 == 0")
    r0, n = _rows(rows, row_start, row_count)
    buf = np.asarray(buf, dtype=np.uint8)
    ns = cols // 256
    a, b = r0 * ns, (r0 + n) * ns
    hdr = buf[16 * a: 16 * b].reshape(b - a, 16).astype(np.int64)
    d = f16_to_f64(hdr[:, 0] | (hdr[:, 1] << 8))
    dmin = f16_to_f64(hdr[:, 2] | (hdr[:, 3] << 8))
    sbytes = hdr[:, 4:16]
    sc = np.stack([_q4_k_field(sbytes, 6 * s) for s in range(8)], axis=1)
    m = np.stack([_q4_k_field(sbytes, 48 + 6 * s) for s in range(8)], axis=1)
    hb = 16 * rows * ns
    qs = buf[hb + 128 * a: hb + 128 * b].reshape(b - a, 8, 16).astype(np.int64)
    q = np.empty((b - a, 8, 32), dtype=np.int64)
    q[:, :, 0::2] = qs & 15   # even weight index: low nibble
    q[:, :, 1::2] = qs >> 4   # odd weight index: high nibble
    return d, dmin, sc, m, q


def dequant_q4_k(buf, rows: int, cols: int, row_start: int = 0, row_count=None) -> np.ndarray:
    """Planar Q4_K -> float64 [row_count][cols].

    256-weight super-block, 8 sub-blocks of 32: w = d*sc_s*q - dmin*m_s.
    """
    r0, n = _rows(rows, row_start, row_count)
    d, dmin, sc, m, q = q4_k_fields(buf, rows, cols, r0, n)
    w = (d[:, None, None] * sc[:, :, None].astype(np.float64) * q
         - dmin[:, None, None] * m[:, :, None].astype(np.float64))
    return w.reshape(n, cols)


def q2_k_offsets(rows: int, cols: int):
    """Plane starts of planar Q2_K: (scale plane, quant plane).

    The d/dmin plane (4 bytes per super-block) starts at 0; each later plane
    starts at the previous plane's end rounded up to 256 bytes.
    """
    ns = cols // 256
    so = (4 * rows * ns + 255) // 256 * 256
    qo = (so + 16 * rows * ns + 255) // 256 * 256
    return so, qo


def q2_k_fields(buf, rows: int, cols: int, row_start: int = 0, row_count=None):
    """Decode Q2_K records into (d, dmin, sc[16], m[16], q[16][16]) per record.

    Scale byte s of a record: sc_s in the low nibble, m_s in the high one.
    Sub-block s owns quant bytes [4s, 4s+4) of the record's 64; weight i of
    it is the 2-bit field at bits 2*(i // 4) of byte i % 4.
    """
    if cols % 256:
        raise ValueError("Q2_K needs cols % 256 == 0")
    r0, n = _rows(rows, row_start, row_count)
    buf = np.asarray(buf, dtype=np.uint8)
    ns = cols // 256
    a, b = r0 * ns, (r0 + n) * ns
    so, qo = q2_k_offsets(rows, cols)
    dd = buf[4 * a: 4 * b].reshape(b - a, 4).astype(np.int64)
    d = f16_to_f64(dd[:, 0] | (dd[:, 1] << 8))
    dmin = f16_to_f64(dd[:, 2] | (dd[:, 3] << 8))
    sb = buf[so + 16 * a: so + 16 * b].reshape(b - a, 16).astype(np.int64)
    sc = sb & 15
    m = sb >> 4
    qb = buf[qo + 64 * a: qo + 64 * b].reshape(b - a, 16, 4).astype(np.int64)
    q = np.empty((b - a, 16, 16), dtype=np.int64)
    for i in range(16):
        q[:, :, i] = (qb[:, :, i % 4] >> (2 * (i // 4))) & 3
    return d, dmin, sc, m, q


def dequant_q2_k(buf, rows: int, cols: int, row_start: int = 0, row_count=None) -> np.ndarray:
    """Planar Q2_K -> float64 [row_count][cols].

    256-weight super-block, 16 sub-blocks of 16: w = d*sc_s*q - dmin*m_s.
    """
    r0, n = _rows(rows, row_start, row_count)
    d, dmin, sc, m, q = q2_k_fields(buf, rows, cols, r0, n)
    w = (d[:, None, None] * sc[:, :, None].astype(np.float64) * q
         - dmin[:, None, None] * m[:, :, None].astype(np.float64))
    return w.reshape(n, cols)


def q3_k_offsets(rows: int, cols: int):
    """Plane starts of planar Q3_K: (scale plane, low-bit plane, high-bit plane).

    The fp16 d plane (2 bytes per super-block) starts at 0; each later plane
    starts at the previous plane's end rounded up to 256 bytes.
    """
    ns = cols // 256
    so = (2 * rows * ns + 255) // 256 * 256
    lo = (so + 16 * rows * ns + 255) // 256 * 256
    hi = (lo + 64 * rows * ns + 255) // 256 * 256
    return so, lo, hi


def q3_k_fields(buf, rows: int, cols: int, row_start: int = 0, row_count=None):
    """Decode Q3_K records into (d, S[16], Q[16][16]) per record.

    S_s is the low six bits of scale byte s.  Q = low | high << 2: the low
    two bits as in Q2_K (weight i of sub-block s at bits 2 (i // 4) of byte
    4s + i % 4 of the record's 64), the high bit at bit 4 (s % 2) + i // 4 of
    byte 4 (s // 2) + i % 4 of the record's 32.
    """
    if cols % 256:
        raise ValueError("Q3_K needs cols % 256 == 0")
    r0, n = _rows(rows, row_start, row_count)
    buf = np.asarray(buf, dtype=np.uint8)
    ns = cols // 256
    a, b = r0 * ns, (r0 + n) * ns
    so, lo, hi = q3_k_offsets(rows, cols)
    db = buf[2 * a: 2 * b].reshape(b - a, 2).astype(np.int64)
    d = f16_to_f64(db[:, 0] | (db[:, 1] << 8))
    S = buf[so + 16 * a: so + 16 * b].reshape(b - a, 16).astype(np.int64) & 63
    lb = buf[lo + 64 * a: lo + 64 * b].reshape(b - a, 16, 4).astype(np.int64)
    hb = buf[hi + 32 * a: hi + 32 * b].reshape(b - a, 8, 4).astype(np.int64)
    Q = np.empty((b - a, 16, 16), dtype=np.int64)
    for s in range(16):
        for i in range(16):
            low = (lb[:, s, i % 4] >> (2 * (i // 4))) & 3
            high = (hb[:, s // 2, i % 4] >> (4 * (s % 2) + i // 4)) & 1
            Q[:, s, i] = low | (high << 2)
    return d, S, Q


def dequant_q3_k(buf, rows: int, cols: int, row_start: int = 0, row_count=None) -> np.ndarray:
    """Planar Q3_K -> float64 [row_count][cols].

    256-weight super-block, 16 sub-blocks of 16: w = d*(S_s - 32)*(Q - 4).
    """
    r0, n = _rows(rows, row_start, row_count)
    d, S, Q = q3_k_fields(buf, rows, cols, r0, n)
    w = d[:, None, None] * (S[:, :, None] - 32).astype(np.float64) * (Q - 4).astype(np.float64)
    return w.reshape(n, cols)


def q6_k_offsets(rows: int, cols: int):
    """Plane starts of planar Q6_K: (scale plane, low-bit plane, high-bit plane)."""
    ns = cols // 256
    so = (2 * rows * ns + 255) // 256 * 256
    lo = (so + 16 * rows * ns + 255) // 256 * 256
    hi = (lo + 128 * rows * ns + 255) // 256 * 256
    return so, lo, hi


def q6_k_fields(buf, rows: int, cols: int, row_start: int = 0, row_count=None):
    """Decode Q6_K records into (d, sc[16], Q[16][16]) per record.

    sc is the signed byte of scale s.  Q = low | high << 4: weight i of
    32-weight group g (sub-block 2g + i // 16, position i % 16) has its low
    four bits in byte 16g + i // 2 of the record's 128 (low nibble for even
    i) and its high two bits at bit 4 ((i // 8) % 2) + 2 (i % 2) of byte
    8g + 4 (i // 16) + (i % 8) // 2 of the record's 64.
    """
    if cols % 256:
        raise ValueError("Q6_K needs cols % 256 == 0")
    r0, n = _rows(rows, row_start, row_count)
    buf = np.asarray(buf, dtype=np.uint8)
    ns = cols // 256
    a, b = r0 * ns, (r0 + n) * ns
    so, lo, hi = q6_k_offsets(rows, cols)
    db = buf[2 * a: 2 * b].reshape(b - a, 2).astype(np.int64)
    d = f16_to_f64(db[:, 0] | (db[:, 1] << 8))
    sc = buf[so + 16 * a: so + 16 * b].view(np.int8).reshape(b - a, 16).astype(np.int64)
    lb = buf[lo + 128 * a: lo + 128 * b].reshape(b - a, 8, 16).astype(np.int64)
    hb = buf[hi + 64 * a: hi + 64 * b].reshape(b - a, 8, 8).astype(np.int64)
    Q = np.empty((b - a, 16, 16), dtype=np.int64)
    for g in range(8):
        for i in range(32):
            low = (lb[:, g, i // 2] >> (4 * (i % 2))) & 15
            high = (hb[:, g, 4 * (i // 16) + (i % 8) // 2] >> (4 * ((i // 8) % 2) + 2 * (i % 2))) & 3
            Q[:, 2 * g + i // 16, i % 16] = low | (high << 4)
    return d, sc, Q


def dequant_q6_k(buf, rows: int, cols: int, row_start: int = 0, row_count=None) -> np.ndarray:
    """Planar Q6_K -> float64 [row_count][cols].

    256-weight super-block, 16 sub-blocks of 16: w = d*sc_s*(Q - 32).
    """
    r0, n = _rows(rows, row_start, row_count)
    d, sc, Q = q6_k_fields(buf, rows, cols, r0, n)
    w = d[:, None, None] * sc[:, :, None].astype(np.float64) * (Q - 32).astype(np.float64)
    return w.reshape(n, cols)


def dequant(dtype: str, buf, rows: int, cols: int, row_start: int = 0, row_count=None) -> np.ndarray:
    if dtype == "q8_0":
        return dequant_q8_0(buf, rows, cols, row_start, row_count)
    if dtype == "q4_k":
        return dequant_q4_k(buf, rows, cols, row_start, row_count)
    if dtype == "q2_k":
        return dequant_q2_k(buf, rows, cols, row_start, row_count)
    if dtype == "q3_k":
        return dequant_q3_k(buf, rows, cols, row_start, row_count)
    if dtype == "q6_k":
        return dequant_q6_k(buf, rows, cols, row_start, row_count)
    if dtype == "f32":
        r0, n = _rows(rows, row_start, row_count)
        a = np.asarray(buf).view(np.float32).reshape(rows, cols)
        return a[r0:r0 + n].astype(np.float64)
    raise ValueError(f"unknown dtype {dtype!r}")


# ---------------------------------------------------------------------------
# Router
# ---------------------------------------------------------------------------


def router_logits(router, x) -> np.ndarray:
    """l[t][e] = sum_h Wr[e][h] * x[t][h] in float64 (F32 inputs)."""
    W = np.asarray(router, dtype=np.float32).astype(np.float64)
    X = np.atleast_2d(np.asarray(x, dtype=np.float32)).astype(np.float64)
    return X @ W.T


def select_experts(logits, k: int) -> np.ndarray:
    """Top-k expert ids per token, sorted by the key (-logit, expert id)."""
    L = np.atleast_2d(np.asarray(logits, dtype=np.float64))
    M, E = L.shape
    if not 1 <= k <= E:
        raise ValueError("need 1 <= k <= n_experts")
    idx = np.arange(E)
    ids = np.empty((M, k), dtype=np.int64)
    for t in range(M):
        order = np.lexsort((idx, -L[t]))
        ids[t] = order[:k]
    return ids


def softmax(logits) -> np.ndarray:
    L = np.atleast_2d(np.asarray(logits, dtype=np.float64))
    z = np.exp(L - L.max(axis=1, keepdims=True))
    return z / z.sum(axis=1, keepdims=True)


def routing_weights(logits, ids) -> np.ndarray:
    """w_tj = p_t[ids_tj] / sum_j p_t[ids_tj] with p_t = softmax(l_t) over all experts."""
    p = softmax(logits)
    sel = np.take_along_axis(p, np.asarray(ids), axis=1)
    return sel / sel.sum(axis=1, keepdims=True)


def bucket(ids, n_experts: int):
    """Per-expert lists of (token, slot) pairs.

    Pair index p = t*k + j.  Returns counts[E], offsets[E+1] (exclusive
    prefix sums), slots[M*k] (for each expert in ascending order, its pair
    indices with t ascending) and the ascending list of active experts.
    """
    ids = np.asarray(ids, dtype=np.int64)
    flat = ids.reshape(-1)
    counts = np.bincount(flat, minlength=n_experts).astype(np.int64)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    slots = np.argsort(flat, kind="stable").astype(np.int64)
    active = np.nonzero(counts)[0].astype(np.int64)
    return counts, offsets, slots, active


def route(router, x, k: int) -> dict:
    logits = router_logits(router, x)
    ids = select_experts(logits, k)
    w = routing_weights(logits, ids)
    counts, offsets, slots, active = bucket(ids, np.asarray(router).shape[0])
    return dict(logits=logits, ids=ids, w=w, counts=counts, offsets=offsets,
                slots=slots, active=active)


# ---------------------------------------------------------------------------
# Expert FFN and the whole layer
# ---------------------------------------------------------------------------


def silu(g):
    g = np.asarray(g, dtype=np.float64)
    with np.errstate(over="ignore"):
        return g / (1.0 + np.exp(-g))


def swiglu_ffn(Wg, Wu, Wd, xs) -> np.ndarray:
    """o = Wd (silu(Wg x) * (Wu x)) for each row x of ``xs``."""
    xs = np.atleast_2d(np.asarray(xs, dtype=np.float64))
    g = xs @ Wg.T
    u = xs @ Wu.T
    h = silu(g) * u
    return h @ Wd.T


def moe_layer(x, router, gate, up, down, *, top_k: int, ffn: int, expert_type: str,
              shared=None, shared_ffn: int = 0, shared_type: str = "q8_0",
              tokens=None, down_type=None, workers: int = 1) -> dict:
    """The routed-MoE layer on x [M][H] (float32 input), in float64.

    ``gate``/``up`` are stacked E*F x H tensors in the planar layout of
    ``expert_type``, ``down`` E*H x F in that of ``down_type`` (None: the
    same); ``shared`` is (gate, up, down) of the
    shared expert (Fs x H, Fs x H, H x Fs) or None.  ``tokens`` restricts
    the FFN part to a subset of tokens (routing is always computed for all).
    Returns the routing of ``route`` plus y [len(tokens)][H].

    ``workers`` > 1 evaluates the selected experts' FFNs on that many
    threads (NumPy releases the interpreter lock inside its array
    operations).  Each expert's arithmetic and the final slot-order sum are
    the same either way, so the result does not depend on it.
    """
    X = np.atleast_2d(np.asarray(x, dtype=np.float32)).astype(np.float64)
    M, H = X.shape
    R = np.asarray(router, dtype=np.float32)
    E = R.shape[0]
    F = ffn
    r = route(R, X.astype(np.float32), top_k)
    toks = list(range(M)) if tokens is None else [int(t) for t in tokens]
    y = np.zeros((len(toks), H), dtype=np.float64)

    if shared is not None and shared_ffn > 0:
        Fs = shared_ffn
        Wsg = dequant(shared_type, shared[0], Fs, H)
        Wsu = dequant(shared_type, shared[1], Fs, H)
        Wsd = dequant(shared_type, shared[2], H, Fs)
        y += swiglu_ffn(Wsg, Wsu, Wsd, X[toks])

    ids, w = r["ids"], r["w"]
    need = {}
    for ti, t in enumerate(toks):
        for j in range(top_k):
            need.setdefault(int(ids[t, j]), []).append((ti, j))
    o = np.zeros((len(toks), top_k, H), dtype=np.float64)

    def expert_out(e):
        Wg = dequant(expert_type, gate, E * F, H, e * F, F)
        Wu = dequant(expert_type, up, E * F, H, e * F, F)
        Wd = dequant(down_type or expert_type, down, E * H, F, e * H, H)
        return swiglu_ffn(Wg, Wu, Wd, X[[toks[ti] for ti, _ in need[e]]])

    experts = sorted(need)
    if workers > 1 and len(experts) > 1:
        with ThreadPoolExecutor(max_workers=workers) as pool:
            outs = list(pool.map(expert_out, experts))
    else:
        outs = [expert_out(e) for e in experts]
    for e, out in zip(experts, outs):
        for (ti, j), row in zip(need[e], out):
            o[ti, j] = row
    for ti, t in enumerate(toks):
        for j in range(top_k):
            y[ti] += w[t, j] * o[ti, j]
    r["y"] = y
    r["tokens"] = toks
    return r
