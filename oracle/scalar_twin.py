"""Scalar-loop twin of the oracle -- TEST INFRASTRUCTURE ONLY.

A second, deliberately naive CPU implementation of the same layer used to pin
the vectorised oracle on tiny shapes.  It shares no code with
``moe_oracle.py``: fp16 is decoded with Python's ``struct`` half-precision
codec, the Q4_K scale/min fields are cut from one Python integer holding the
96-bit stream, a Q2_K quant is cut from the little-endian integer of its
sub-block's four bytes (weight i at bit 8 (i % 4) + 2 (i // 4)), a Q3_K
high bit from the integer of its sub-block pair's four bytes (bit
8 (i % 4) + 4 (s % 2) + i // 4), a Q6_K quant from the integers of its
group's 16 low bytes and 8 high bytes, and every product is an explicit
loop over Python floats.
Meant for hidden sizes of a few hundred and a handful of experts.
"""

from __future__ import annotations

import math
import struct


def _f16(lo: int, hi: int) -> float:
    return struct.unpack("<e", bytes([lo, hi]))[0]


def weight_q8_0(buf, rows: int, cols: int, r: int, c: int) -> float:
    nb = cols // 32
    b = c // 32
    so = 2 * (r * nb + b)
    d = _f16(int(buf[so]), int(buf[so + 1]))
    qo = -(-2 * rows * nb // 256) * 256
    q = int(buf[qo + r * cols + c])
    if q >= 128:
        q -= 256
    return d * q


def weight_q4_k(buf, rows: int, cols: int, r: int, c: int) -> float:
    ns = cols // 256
    rec = r * ns + c // 256
    within = c % 256
    s, i = within // 32, within % 32
    h = [int(v) for v in buf[16 * rec: 16 * rec + 16]]
    d = _f16(h[0], h[1])
    dmin = _f16(h[2], h[3])
    stream = int.from_bytes(bytes(h[4:16]), "little")
    sc = (stream >> (6 * s)) & 0x3F
    mn = (stream >> (48 + 6 * s)) & 0x3F
    qbyte = int(buf[16 * rows * ns + 128 * rec + 16 * s + i // 2])
    q = (qbyte >> 4) if (i % 2) else (qbyte & 0xF)
    return d * sc * q - dmin * mn


def weight_q2_k(buf, rows: int, cols: int, r: int, c: int) -> float:
    ns = cols // 256
    rec = r * ns + c // 256
    s, i = (c % 256) // 16, c % 16
    d = _f16(int(buf[4 * rec]), int(buf[4 * rec + 1]))
    dmin = _f16(int(buf[4 * rec + 2]), int(buf[4 * rec + 3]))
    sbase = -(-4 * rows * ns // 256) * 256
    qbase = -(-(sbase + 16 * rows * ns) // 256) * 256
    sbyte = int(buf[sbase + 16 * rec + s])
    word = int.from_bytes(bytes(int(v) for v in buf[qbase + 64 * rec + 4 * s: qbase + 64 * rec + 4 * s + 4]),
                          "little")
    q = (word >> (8 * (i % 4) + 2 * (i // 4))) & 3
    return d * (sbyte % 16) * q - dmin * (sbyte // 16)


def weight_q3_k(buf, rows: int, cols: int, r: int, c: int) -> float:
    ns = cols // 256
    rec = r * ns + c // 256
    s, i = (c % 256) // 16, c % 16
    d = _f16(int(buf[2 * rec]), int(buf[2 * rec + 1]))
    sbase = -(-2 * rows * ns // 256) * 256
    lbase = -(-(sbase + 16 * rows * ns) // 256) * 256
    hbase = -(-(lbase + 64 * rows * ns) // 256) * 256
    scale = int(buf[sbase + 16 * rec + s]) % 64 - 32
    lw = int.from_bytes(bytes(int(v) for v in buf[lbase + 64 * rec + 4 * s: lbase + 64 * rec + 4 * s + 4]),
                        "little")
    hw = int.from_bytes(bytes(int(v) for v in buf[hbase + 32 * rec + 4 * (s // 2):
                                                   hbase + 32 * rec + 4 * (s // 2) + 4]), "little")
    q = ((lw >> (8 * (i % 4) + 2 * (i // 4))) & 3) + 4 * ((hw >> (8 * (i % 4) + 4 * (s % 2) + i // 4)) & 1)
    return d * scale * (q - 4)


def weight_q6_k(buf, rows: int, cols: int, r: int, c: int) -> float:
    ns = cols // 256
    rec = r * ns + c // 256
    g, i = (c % 256) // 32, c % 32
    d = _f16(int(buf[2 * rec]), int(buf[2 * rec + 1]))
    sbase = -(-2 * rows * ns // 256) * 256
    lbase = -(-(sbase + 16 * rows * ns) // 256) * 256
    hbase = -(-(lbase + 128 * rows * ns) // 256) * 256
    sc = struct.unpack("<b", bytes([int(buf[sbase + 16 * rec + 2 * g + i // 16])]))[0]
    lw = int.from_bytes(bytes(int(v) for v in buf[lbase + 128 * rec + 16 * g: lbase + 128 * rec + 16 * g + 16]),
                        "little")
    hw = int.from_bytes(bytes(int(v) for v in buf[hbase + 64 * rec + 8 * g: hbase + 64 * rec + 8 * g + 8]),
                        "little")
    low = (lw >> (4 * i)) & 15
    high = (hw >> (32 * (i // 16) + 8 * ((i % 8) // 2) + 4 * ((i // 8) % 2) + 2 * (i % 2))) & 3
    return d * sc * ((low | (high << 4)) - 32)


_WEIGHT = {"q8_0": weight_q8_0, "q4_k": weight_q4_k, "q2_k": weight_q2_k, "q3_k": weight_q3_k,
           "q6_k": weight_q6_k}


def weight(dtype: str, buf, rows: int, cols: int, r: int, c: int) -> float:
    return _WEIGHT[dtype](buf, rows, cols, r, c)


def _matvec(dtype, buf, rows, cols, row0, nrows, v):
    out = []
    for r in range(row0, row0 + nrows):
        acc = 0.0
        for c in range(cols):
            acc += weight(dtype, buf, rows, cols, r, c) * v[c]
        out.append(acc)
    return out


def _ffn(dtype, g_buf, u_buf, d_buf, rows_gu, rows_d, g_row0, d_row0, F, H, x, ddtype=None):
    g = _matvec(dtype, g_buf, rows_gu, H, g_row0, F, x)
    u = _matvec(dtype, u_buf, rows_gu, H, g_row0, F, x)
    h = [gi / (1.0 + math.exp(-gi)) * ui for gi, ui in zip(g, u)]
    return _matvec(ddtype or dtype, d_buf, rows_d, F, d_row0, H, h)


def moe_layer(x, router, gate, up, down, *, top_k, ffn, expert_type,
              shared=None, shared_ffn=0, shared_type="q8_0", down_type=None):
    """Returns (y, ids, w) with y a list of lists of floats."""
    E = len(router)
    H = len(router[0])
    F = ffn
    ys, all_ids, all_w = [], [], []
    for xt in x:
        xt = [float(v) for v in xt]
        logits = []
        for e in range(E):
            acc = 0.0
            for h in range(H):
                acc += float(router[e][h]) * xt[h]
            logits.append(acc)
        # selection sort on (-logit, index)
        chosen = []
        for _ in range(top_k):
            best = None
            for e in range(E):
                if e in chosen:
                    continue
                if best is None or logits[e] > logits[best]:
                    best = e
            chosen.append(best)
        mx = max(logits)
        p = [math.exp(v - mx) for v in logits]
        tot = sum(p)
        p = [v / tot for v in p]
        ssum = sum(p[e] for e in chosen)
        w = [p[e] / ssum for e in chosen]
        y = [0.0] * H
        if shared is not None and shared_ffn > 0:
            s = _ffn(shared_type, shared[0], shared[1], shared[2], shared_ffn, H,
                     0, 0, shared_ffn, H, xt)
            y = [a + b for a, b in zip(y, s)]
        for j, e in enumerate(chosen):
            o = _ffn(expert_type, gate, up, down, E * F, E * H, e * F, e * H, F, H, xt, down_type)
            y = [a + w[j] * b for a, b in zip(y, o)]
        ys.append(y)
        all_ids.append(chosen)
        all_w.append(w)
    return ys, all_ids, all_w
