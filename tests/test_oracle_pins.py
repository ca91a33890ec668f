"""Pins of the CPU oracle against facts outside itself (no GPU).

Each test fixes one part of the oracle to something independent: hand-derived
byte fixtures, the IEEE half-precision codec of NumPy, the generator's own
quantiser run backwards, textbook softmax, brute-force loops and the
scalar-loop twin, plus invariants of the layer (sum of routing weights,
one-expert reduction, token independence, exact power-of-two scaling).
"""

import numpy as np
import pytest
import scipy.special

from oracle import moe_oracle as om
from oracle import scalar_twin as tw
import synth
from _support import (copy_expert_rows, double_scales, oracle_kwargs, read_fixture,
                      routing_predicate, run_oracle, small_config)


# --------------------------------------------------------------------------- formats

def test_f16_decode_all_bit_patterns_match_numpy():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    got = om.f16_to_f64(bits)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))


FIXTURES = [("q8_0_planar.txt", "q8_0"), ("q4_k_planar.txt", "q4_k"), ("q2_k_planar.txt", "q2_k"),
            ("q3_k_planar.txt", "q3_k"), ("q6_k_planar.txt", "q6_k")]


@pytest.mark.parametrize("fixture,dtype", FIXTURES)
def test_dequant_matches_hand_derived_fixture(fixture, dtype):
    rows, cols, buf, expects = read_fixture(fixture)
    assert synth.tensor_bytes(dtype, rows, cols) == buf.size
    W = om.dequant(dtype, buf, rows, cols)
    assert W.shape == (rows, cols)
    for r, c, v in expects:
        assert W[r, c] == v, (r, c, W[r, c], v)


def test_dequant_fixture_twin_agrees():
    for fixture, dtype in FIXTURES:
        rows, cols, buf, _ = read_fixture(fixture)
        W = om.dequant(dtype, buf, rows, cols)
        for r in range(rows):
            for c in range(cols):
                assert tw.weight(dtype, buf, rows, cols, r, c) == W[r, c]


def test_q8_0_requantise_roundtrip_is_byte_exact():
    rng = np.random.default_rng(7)
    R, K = 64, 512
    w = (rng.standard_normal((R, K)) * 0.02).astype(np.float32)
    w[3, 32:64] = 0.0                        # an all-zero block: d = 0, q = 0
    d_bits, q = synth.quantize_q8_0(w)
    buf = np.zeros(synth.q8_0_bytes(R, K), dtype=np.uint8)
    buf[: 2 * R * (K // 32)].view(np.uint16)[:] = d_bits.reshape(-1)
    qo = synth.q8_0_quant_offset(R, K)
    buf[qo:qo + R * K] = q.reshape(-1).view(np.uint8)
    W = om.dequant_q8_0(buf, R, K)
    d2, q2 = synth.quantize_q8_0(W)
    assert np.array_equal(d2, d_bits)
    assert np.array_equal(q2, q)
    assert np.all(W[3, 32:64] == 0.0)
    # |q| reaches 127 in every non-zero block (d = max|w| / 127)
    qb = np.abs(q.reshape(R, K // 32, 32).astype(np.int64)).max(axis=2)
    assert np.all((qb == 127) | (d_bits == 0))


def _q4k_record(d_bits=0x3C00, dmin_bits=0x3C00, sc=None, m=None, nib=None):
    """One Q4_K record built field by field (test-side encoder)."""
    sc = sc or [0] * 8
    m = m or [0] * 8
    stream = 0
    for s in range(8):
        stream |= (sc[s] & 63) << (6 * s)
        stream |= (m[s] & 63) << (48 + 6 * s)
    hdr = (int(d_bits).to_bytes(2, "little") + int(dmin_bits).to_bytes(2, "little")
           + stream.to_bytes(12, "little"))
    qs = bytearray(128)
    if nib is not None:
        for s in range(8):
            for i in range(32):
                v = nib[s][i] & 15
                qs[16 * s + i // 2] |= v << (4 * (i % 2))
    return np.frombuffer(hdr + bytes(qs), dtype=np.uint8).copy()


@pytest.mark.parametrize("s", range(8))
def test_q4_k_single_field_positions(s):
    # Only sub-block s gets a scale, and only one weight a quant: exactly one
    # non-zero weight must appear, at column 32*s + i, with value sc * q.
    for i in (0, 1, 17, 30, 31):
        nib = [[0] * 32 for _ in range(8)]
        nib[s][i] = 5
        sc = [0] * 8
        sc[s] = 3 + s
        W = om.dequant_q4_k(_q4k_record(sc=sc, nib=nib), 1, 256)[0]
        nz = np.nonzero(W)[0]
        assert list(nz) == [32 * s + i]
        assert W[32 * s + i] == 5.0 * (3 + s)
    # Only min m_s set: the whole sub-block s equals -dmin * m_s.
    m = [0] * 8
    m[s] = 1 + 7 * s
    W = om.dequant_q4_k(_q4k_record(m=m, dmin_bits=0x3800), 1, 256)[0]
    exp = np.zeros(256)
    exp[32 * s:32 * s + 32] = -0.5 * (1 + 7 * s)
    assert np.array_equal(W, exp)


def test_q4_k_multi_row_record_order():
    # Two rows x 512 cols: record (r, b) is at r*ns + b in both planes.
    recs = []
    for r in range(2):
        for b in range(2):
            nib = [[(r * 2 + b + 1)] * 32 for _ in range(8)]
            recs.append(_q4k_record(sc=[1] * 8, nib=nib))
    hdr = np.concatenate([x[:16] for x in recs])
    qs = np.concatenate([x[16:] for x in recs])
    buf = np.concatenate([hdr, qs])
    W = om.dequant_q4_k(buf, 2, 512)
    for r in range(2):
        for b in range(2):
            assert np.all(W[r, 256 * b:256 * (b + 1)] == r * 2 + b + 1)
    assert np.array_equal(om.dequant_q4_k(buf, 2, 512, row_start=1, row_count=1), W[1:2])


def _q2k_tensor(recs, rows, cols):
    """Planar Q2_K bytes from records (d_bits, dmin_bits, sc[16], m[16],
    q[16][16]) in row-major super-block order (test-side encoder, written
    from the layout: plane starts rounded up to 256 bytes, scale byte
    m << 4 | sc, weight i of a sub-block at bits 2 (i // 4) of its byte i % 4).
    """
    n = len(recs)
    so = -(-4 * n // 256) * 256
    qo = -(-(so + 16 * n) // 256) * 256
    out = bytearray(qo + 64 * n)
    for k, (db, mb, sc, m, q) in enumerate(recs):
        out[4 * k: 4 * k + 4] = int(db).to_bytes(2, "little") + int(mb).to_bytes(2, "little")
        for s in range(16):
            out[so + 16 * k + s] = (m[s] & 15) << 4 | (sc[s] & 15)
            for i in range(16):
                out[qo + 64 * k + 4 * s + i % 4] |= (q[s][i] & 3) << (2 * (i // 4))
    assert len(out) == synth.tensor_bytes("q2_k", rows, cols)
    return np.frombuffer(bytes(out), dtype=np.uint8).copy()


@pytest.mark.parametrize("s", [0, 1, 5, 10, 15])
def test_q2_k_single_field_positions(s):
    # Only sub-block s gets a scale, and only one weight a quant: exactly one
    # non-zero weight must appear, at column 16*s + i, with value sc * q.
    for i in (0, 1, 3, 4, 6, 11, 15):
        q = [[0] * 16 for _ in range(16)]
        q[s][i] = 3 - (i % 2)
        sc = [0] * 16
        sc[s] = 15 - (s % 7)
        buf = _q2k_tensor([(0x3C00, 0x3C00, sc, [0] * 16, q)], 1, 256)
        W = om.dequant_q2_k(buf, 1, 256)[0]
        assert list(np.nonzero(W)[0]) == [16 * s + i]
        assert W[16 * s + i] == (3 - (i % 2)) * (15 - (s % 7))
    # Only min m_s set: the whole sub-block s equals -dmin * m_s.
    m = [0] * 16
    m[s] = 1 + (s % 15)
    buf = _q2k_tensor([(0x3C00, 0x3800, [0] * 16, m, [[3] * 16 for _ in range(16)])], 1, 256)
    W = om.dequant_q2_k(buf, 1, 256)[0]
    exp = np.zeros(256)
    exp[16 * s:16 * s + 16] = -0.5 * (1 + (s % 15))
    assert np.array_equal(W, exp)


def test_q2_k_multi_row_record_order():
    # Three rows x 512 cols: record (r, b) is at r*ns + b in all three planes,
    # and the planes start at the rounded offsets of a 6-record tensor.
    recs = []
    for r in range(3):
        for b in range(2):
            v = r * 2 + b + 1          # 1..6
            recs.append((0x3C00, 0x3C00, [v] * 16, [0] * 16, [[1] * 16 for _ in range(16)]))
    buf = _q2k_tensor(recs, 3, 512)
    W = om.dequant_q2_k(buf, 3, 512)
    for r in range(3):
        for b in range(2):
            assert np.all(W[r, 256 * b:256 * (b + 1)] == r * 2 + b + 1)
    assert np.array_equal(om.dequant_q2_k(buf, 3, 512, row_start=1, row_count=2), W[1:3])


def _q3k_tensor(recs, rows, cols):
    """Planar Q3_K bytes from records (d_bits, S[16], Q[16][16]) (test-side
    encoder, written from the layout: plane starts rounded up to 256 bytes,
    low two bits as in Q2_K, high bit of weight i of sub-block s at byte
    4 (s // 2) + i % 4, bit 4 (s % 2) + i // 4 of the record's 32).
    """
    n = len(recs)
    so = -(-2 * n // 256) * 256
    lo = -(-(so + 16 * n) // 256) * 256
    hi = -(-(lo + 64 * n) // 256) * 256
    out = bytearray(hi + 32 * n)
    for k, (db, S, Q) in enumerate(recs):
        out[2 * k: 2 * k + 2] = int(db).to_bytes(2, "little")
        for s in range(16):
            out[so + 16 * k + s] = S[s] & 63
            for i in range(16):
                out[lo + 64 * k + 4 * s + i % 4] |= (Q[s][i] & 3) << (2 * (i // 4))
                out[hi + 32 * k + 4 * (s // 2) + i % 4] |= ((Q[s][i] >> 2) & 1) << (4 * (s % 2) + i // 4)
    assert len(out) == synth.tensor_bytes("q3_k", rows, cols)
    return np.frombuffer(bytes(out), dtype=np.uint8).copy()


@pytest.mark.parametrize("s", [0, 1, 6, 11, 15])
def test_q3_k_single_field_positions(s):
    # Every quant at the zero point Q = 4 except one: exactly one non-zero
    # weight must appear, at column 16*s + i, with value (S - 32) * (Q - 4).
    for i in (0, 1, 3, 4, 9, 14, 15):
        for q in (0, 3, 5, 7):                   # high bit clear and set
            Q = [[4] * 16 for _ in range(16)]
            Q[s][i] = q
            S = [32 + (s % 5) - 2 * (s % 3) + 1 for _ in range(16)]
            S[s] = 32 - 7 + s
            buf = _q3k_tensor([(0x3C00, S, Q)], 1, 256)
            W = om.dequant_q3_k(buf, 1, 256)[0]
            assert list(np.nonzero(W)[0]) == [16 * s + i]
            assert W[16 * s + i] == (s - 7) * (q - 4)
    # All quants zero (Q = 0): sub-block s is -4 * (S_s - 32) * d throughout.
    S = [32] * 16
    S[s] = 0 if s % 2 else 63
    buf = _q3k_tensor([(0x3800, S, [[0] * 16 for _ in range(16)])], 1, 256)
    W = om.dequant_q3_k(buf, 1, 256)[0]
    exp = np.zeros(256)
    exp[16 * s:16 * s + 16] = 0.5 * (S[s] - 32) * -4
    assert np.array_equal(W, exp)


def test_q3_k_multi_row_record_order():
    recs = []
    for r in range(3):
        for b in range(2):
            v = r * 2 + b + 1          # 1..6
            recs.append((0x3C00, [32 + v] * 16, [[5] * 16 for _ in range(16)]))
    buf = _q3k_tensor(recs, 3, 512)
    W = om.dequant_q3_k(buf, 3, 512)
    for r in range(3):
        for b in range(2):
            assert np.all(W[r, 256 * b:256 * (b + 1)] == r * 2 + b + 1)
    assert np.array_equal(om.dequant_q3_k(buf, 3, 512, row_start=2, row_count=1), W[2:3])


def _q6k_tensor(recs, rows, cols):
    """Planar Q6_K bytes from records (d_bits, sc[16] signed, Q[16][16])
    (test-side encoder, from the layout: plane starts rounded up to 256
    bytes; weight i of 32-weight group g: low nibble in byte 16g + i // 2,
    high two bits at byte 8g + 4 (i // 16) + (i % 8) // 2, bit
    4 ((i // 8) % 2) + 2 (i % 2); sub-block s = 2g + i // 16).
    """
    n = len(recs)
    so = -(-2 * n // 256) * 256
    lo = -(-(so + 16 * n) // 256) * 256
    hi = -(-(lo + 128 * n) // 256) * 256
    out = bytearray(hi + 64 * n)
    for k, (db, sc, Q) in enumerate(recs):
        out[2 * k: 2 * k + 2] = int(db).to_bytes(2, "little")
        for s in range(16):
            out[so + 16 * k + s] = sc[s] & 255
        for g in range(8):
            for i in range(32):
                q = Q[2 * g + i // 16][i % 16]
                out[lo + 128 * k + 16 * g + i // 2] |= (q & 15) << (4 * (i % 2))
                out[hi + 64 * k + 8 * g + 4 * (i // 16) + (i % 8) // 2] |= \
                    ((q >> 4) & 3) << (4 * ((i // 8) % 2) + 2 * (i % 2))
    assert len(out) == synth.tensor_bytes("q6_k", rows, cols)
    return np.frombuffer(bytes(out), dtype=np.uint8).copy()


@pytest.mark.parametrize("s", [0, 1, 7, 10, 15])
def test_q6_k_single_field_positions(s):
    # Every quant at the zero point Q = 32 except one: exactly one non-zero
    # weight, at column 16*s + i, with value sc * (Q - 32).
    for i in (0, 1, 2, 7, 8, 9, 14, 15):
        for q in (0, 17, 31, 33, 48, 63):         # every high-bit value
            Q = [[32] * 16 for _ in range(16)]
            Q[s][i] = q
            sc = [3] * 16
            sc[s] = -5 - s
            buf = _q6k_tensor([(0x3C00, sc, Q)], 1, 256)
            W = om.dequant_q6_k(buf, 1, 256)[0]
            assert list(np.nonzero(W)[0]) == [16 * s + i]
            assert W[16 * s + i] == (-5 - s) * (q - 32)
    # All quants zero: sub-block s is -32 * sc_s * d throughout.
    sc = [0] * 16
    sc[s] = 127 if s % 2 else -128
    buf = _q6k_tensor([(0x3800, sc, [[0] * 16 for _ in range(16)])], 1, 256)
    W = om.dequant_q6_k(buf, 1, 256)[0]
    exp = np.zeros(256)
    exp[16 * s:16 * s + 16] = 0.5 * sc[s] * -32
    assert np.array_equal(W, exp)


def test_q6_k_multi_row_record_order():
    recs = []
    for r in range(3):
        for b in range(2):
            v = r * 2 + b + 1          # 1..6
            recs.append((0x3C00, [v] * 16, [[33] * 16 for _ in range(16)]))
    buf = _q6k_tensor(recs, 3, 512)
    W = om.dequant_q6_k(buf, 3, 512)
    for r in range(3):
        for b in range(2):
            assert np.all(W[r, 256 * b:256 * (b + 1)] == r * 2 + b + 1)
    assert np.array_equal(om.dequant_q6_k(buf, 3, 512, row_start=1, row_count=1), W[1:2])


def test_q8_0_row_slice_matches_full():
    cfg = small_config(n_experts=3, ffn=64)
    inp = synth.draw_layer(cfg, threads=1)
    R = cfg.n_experts * cfg.ffn
    full = om.dequant_q8_0(inp.gate, R, cfg.hidden)
    part = om.dequant_q8_0(inp.gate, R, cfg.hidden, row_start=64, row_count=64)
    assert np.array_equal(part, full[64:128])


# --------------------------------------------------------------------------- router

def test_router_logits_unit_vectors_pick_columns():
    rng = np.random.default_rng(1)
    R = rng.standard_normal((6, 40)).astype(np.float32)
    X = np.eye(40, dtype=np.float32)[[0, 7, 39]]
    L = om.router_logits(R, X)
    assert np.array_equal(L, R[:, [0, 7, 39]].T.astype(np.float64))


def test_select_ties_go_to_lower_index():
    L = np.array([[1.0, 3.0, 3.0, 2.0, 3.0, -1.0]])
    assert om.select_experts(L, 4).tolist() == [[1, 2, 4, 3]]
    L2 = np.zeros((1, 5))
    assert om.select_experts(L2, 3).tolist() == [[0, 1, 2]]


def test_select_matches_brute_force_sort():
    rng = np.random.default_rng(2)
    L = np.round(rng.standard_normal((20, 17)), 1)  # many exact ties
    ids = om.select_experts(L, 5)
    for t in range(20):
        ref = sorted(range(17), key=lambda e: (-L[t, e], e))[:5]
        assert ids[t].tolist() == ref


def test_routing_weights_sum_to_one_and_k1_is_one():
    rng = np.random.default_rng(3)
    L = rng.standard_normal((50, 64)) * 3
    for k in (1, 2, 8, 64):
        ids = om.select_experts(L, k)
        w = om.routing_weights(L, ids)
        assert np.max(np.abs(w.sum(axis=1) - 1.0)) <= 1e-12
        assert np.all(w > 0)
        assert np.all(np.diff(w, axis=1) <= 0)   # descending logits -> descending weights
        if k == 1:
            assert np.all(w == 1.0)


def test_k_equals_E_is_the_textbook_softmax():
    rng = np.random.default_rng(4)
    L = rng.standard_normal((10, 12)) * 2
    ids = om.select_experts(L, 12)
    w = om.routing_weights(L, ids)
    ref = scipy.special.softmax(L, axis=1)
    assert np.allclose(w, np.take_along_axis(ref, ids, axis=1), rtol=1e-13, atol=0)


def test_renormalised_weights_equal_softmax_over_selected():
    rng = np.random.default_rng(5)
    L = rng.standard_normal((10, 30)) * 2
    ids = om.select_experts(L, 4)
    w = om.routing_weights(L, ids)
    ref = scipy.special.softmax(np.take_along_axis(L, ids, axis=1), axis=1)
    assert np.allclose(w, ref, rtol=1e-13, atol=0)


def test_bucket_matches_brute_force():
    rng = np.random.default_rng(6)
    E, M, k = 11, 9, 3
    ids = np.stack([rng.choice(E, k, replace=False) for _ in range(M)])
    counts, offsets, slots, active = om.bucket(ids, E)
    ref_slots = []
    for e in range(E):
        lst = [t * k + j for t in range(M) for j in range(k) if ids[t, j] == e]
        assert counts[e] == len(lst)
        assert offsets[e] == len(ref_slots)
        ref_slots += lst
    assert offsets[E] == M * k
    assert slots.tolist() == ref_slots
    assert active.tolist() == [e for e in range(E) if counts[e] > 0]


def test_permuting_experts_permutes_ids():
    cfg = small_config(n_experts=6, top_k=3, n_tokens=3)
    inp = synth.draw_layer(cfg, threads=1)
    x, _ = synth.draw_tokens(cfg)
    perm = np.array([4, 0, 5, 2, 1, 3])        # new expert i = old expert perm[i]
    r0 = om.route(inp.router, x, 3)
    r1 = om.route(inp.router[perm], x, 3)
    inv = np.argsort(perm)
    assert np.array_equal(r1["ids"], inv[r0["ids"]])
    assert np.allclose(r1["w"], r0["w"], rtol=1e-14, atol=0)


# --------------------------------------------------------------------------- FFN / layer

def test_silu_is_g_times_logistic():
    g = np.linspace(-40, 40, 2001)
    assert np.allclose(om.silu(g), g * scipy.special.expit(g), rtol=1e-14, atol=1e-300)
    assert om.silu(np.array([0.0]))[0] == 0.0


@pytest.mark.parametrize("etype,H,F,Fs,E", [("q8_0", 256, 128, 0, 8), ("q8_0", 256, 64, 96, 4),
                                             ("q4_k", 256, 256, 64, 4), ("q2_k", 256, 256, 64, 4),
                                             ("q2_k/q3_k", 256, 256, 64, 4),
                                             ("q6_k", 256, 256, 64, 4)])
def test_oracle_matches_scalar_twin(etype, H, F, Fs, E):
    etype, _, dtype = etype.partition("/")
    cfg = small_config(hidden=H, ffn=F, shared_ffn=Fs, n_experts=E, expert_type=etype,
                       down_type=dtype or None, n_tokens=2, seed_index=200 + F)
    inp = synth.draw_layer(cfg, threads=1)
    x, _ = synth.draw_tokens(cfg)
    ref = run_oracle(inp, x)
    kw = oracle_kwargs(inp)
    y, ids, w = tw.moe_layer(x, inp.router.tolist(), inp.gate, inp.up, inp.down, **kw)
    assert np.array_equal(ref["ids"], np.array(ids))
    assert np.allclose(ref["w"], np.array(w), rtol=1e-12, atol=0)
    yt = np.array(y)
    scale = np.sqrt(np.mean(yt ** 2))
    assert np.max(np.abs(ref["y"] - yt)) <= 1e-12 * scale


def test_one_expert_top1_layer_is_dense_swiglu_ffn():
    cfg = small_config(n_experts=1, top_k=1, n_tokens=3, ffn=96)
    inp = synth.draw_layer(cfg, threads=1)
    x, _ = synth.draw_tokens(cfg)
    ref = run_oracle(inp, x)
    assert np.all(ref["w"] == 1.0)
    Wg = om.dequant_q8_0(inp.gate, 96, 256)
    Wu = om.dequant_q8_0(inp.up, 96, 256)
    Wd = om.dequant_q8_0(inp.down, 256, 96)
    dense = om.swiglu_ffn(Wg, Wu, Wd, x.astype(np.float64))
    assert np.array_equal(ref["y"], dense)


def test_identical_experts_make_routing_irrelevant():
    cfg = small_config(n_experts=5, top_k=3, n_tokens=3)
    inp = synth.draw_layer(cfg, threads=1)
    x, _ = synth.draw_tokens(cfg)
    E, F, H = 5, cfg.ffn, cfg.hidden
    inp.gate = copy_expert_rows("q8_0", inp.gate, F, H, E)
    inp.up = copy_expert_rows("q8_0", inp.up, F, H, E)
    inp.down = copy_expert_rows("q8_0", inp.down, H, F, E)
    ref = run_oracle(inp, x)
    one = om.swiglu_ffn(om.dequant_q8_0(inp.gate, E * F, H, 0, F),
                        om.dequant_q8_0(inp.up, E * F, H, 0, F),
                        om.dequant_q8_0(inp.down, E * H, F, 0, H), x.astype(np.float64))
    assert np.allclose(ref["y"], one, rtol=1e-12, atol=1e-12 * np.abs(one).max())


@pytest.mark.parametrize("etype", ["q8_0", "q4_k", "q2_k", "q3_k", "q6_k"])
def test_doubling_down_scales_doubles_routed_part_exactly(etype):
    F = 128 if etype == "q8_0" else 256
    cfg = small_config(n_experts=4, ffn=F, shared_ffn=64, expert_type=etype, n_tokens=2)
    inp = synth.draw_layer(cfg, threads=1)
    x, _ = synth.draw_tokens(cfg)
    y1 = run_oracle(inp, x)["y"]
    base = om.moe_layer(x, inp.router, inp.gate, inp.up, inp.down, top_k=2, ffn=F,
                        expert_type=etype)["y"]
    inp.down = double_scales(etype, inp.down, cfg.n_experts * cfg.hidden, F)
    y2 = run_oracle(inp, x)["y"]
    routed1 = base
    routed2 = om.moe_layer(x, inp.router, inp.gate, inp.up, inp.down, top_k=2, ffn=F,
                           expert_type=etype)["y"]
    assert np.array_equal(routed2, 2.0 * routed1)
    shared = y1 - routed1
    assert np.allclose(y2 - routed2, shared, rtol=1e-12, atol=1e-12)


def test_rows_are_independent_of_batch():
    cfg = small_config(n_experts=6, top_k=2, n_tokens=4, shared_ffn=64)
    inp = synth.draw_layer(cfg, threads=1)
    x, _ = synth.draw_tokens(cfg)
    full = run_oracle(inp, x)
    for t in range(4):
        one = run_oracle(inp, x[t:t + 1])
        assert np.array_equal(one["ids"][0], full["ids"][t])
        assert np.allclose(one["y"][0], full["y"][t], rtol=1e-12, atol=1e-13)
    sub = run_oracle(inp, x, tokens=[2, 0])
    assert np.allclose(sub["y"], full["y"][[2, 0]], rtol=1e-12, atol=1e-13)


# --------------------------------------------------------------------------- generator

def test_generator_is_deterministic_and_thread_independent():
    cfg = small_config(n_experts=5, shared_ffn=64, expert_type="q4_k", ffn=256)
    a = synth.draw_layer(cfg, threads=1)
    b = synth.draw_layer(cfg, threads=4)
    c = synth.draw_layer(cfg, instance=1, threads=1)
    for name in ("router", "gate", "up", "down", "shared_gate", "shared_up", "shared_down"):
        assert np.array_equal(getattr(a, name), getattr(b, name)), name
        assert not np.array_equal(getattr(a, name), getattr(c, name)), name
    assert a.gate.size == synth.tensor_bytes("q4_k", 5 * 256, 256)
    assert a.down.size == synth.tensor_bytes("q4_k", 5 * 256, 256)
    assert a.shared_down.size == synth.tensor_bytes("q8_0", 256, 64)


def test_q4_k_generated_fields_cover_their_ranges():
    cfg = small_config(n_experts=4, expert_type="q4_k", ffn=256)
    inp = synth.draw_layer(cfg, threads=1)
    d, dmin, sc, m, q = om.q4_k_fields(inp.gate, 4 * 256, 256)
    assert d.min() >= 2.0 ** -14 and d.max() <= 2.0 ** -12
    assert dmin.min() >= 2.0 ** -12 and dmin.max() <= 2.0 ** -10
    assert sc.min() == 0 and sc.max() == 63 and m.min() == 0 and m.max() == 63
    assert q.min() == 0 and q.max() == 15


def test_q2_k_generated_fields_cover_their_ranges():
    cfg = small_config(n_experts=4, expert_type="q2_k", ffn=256)
    inp = synth.draw_layer(cfg, threads=1)
    assert inp.gate.size == synth.tensor_bytes("q2_k", 4 * 256, 256)
    d, dmin, sc, m, q = om.q2_k_fields(inp.gate, 4 * 256, 256)
    assert d.min() >= 2.0 ** -10 and d.max() <= 2.0 ** -8
    assert dmin.min() >= 2.0 ** -10 and dmin.max() <= 2.0 ** -8
    assert sc.min() == 0 and sc.max() == 15 and m.min() == 0 and m.max() == 15
    assert q.min() == 0 and q.max() == 3
    # every quant value is about equally frequent (uniform random bytes)
    counts = np.bincount(q.reshape(-1), minlength=4) / q.size
    assert np.all(np.abs(counts - 0.25) < 0.01)


def test_q3_k_generated_fields_cover_their_ranges():
    cfg = small_config(n_experts=4, expert_type="q2_k", down_type="q3_k", ffn=256)
    inp = synth.draw_layer(cfg, threads=1)
    assert inp.gate.size == synth.tensor_bytes("q2_k", 4 * 256, 256)
    assert inp.down.size == synth.tensor_bytes("q3_k", 4 * 256, 256)
    d, S, Q = om.q3_k_fields(inp.down, 4 * 256, 256)
    assert d.min() >= 2.0 ** -11 and d.max() <= 2.0 ** -9
    assert S.min() == 0 and S.max() == 63
    assert Q.min() == 0 and Q.max() == 7
    counts = np.bincount(Q.reshape(-1), minlength=8) / Q.size
    assert np.all(np.abs(counts - 0.125) < 0.01)


def test_q6_k_generated_fields_cover_their_ranges():
    cfg = small_config(n_experts=4, expert_type="q6_k", ffn=256)
    inp = synth.draw_layer(cfg, threads=1)
    assert inp.gate.size == synth.tensor_bytes("q6_k", 4 * 256, 256)
    d, sc, Q = om.q6_k_fields(inp.gate, 4 * 256, 256)
    assert d.min() >= 2.0 ** -14 and d.max() <= 2.0 ** -12
    assert sc.min() == -128 and sc.max() == 127
    assert Q.min() == 0 and Q.max() == 63
    counts = np.bincount(Q.reshape(-1), minlength=64) / Q.size
    assert np.all(np.abs(counts - 1 / 64) < 0.004)


def test_margin_predicate_enforces_gaps():
    cfg = small_config(n_experts=8, top_k=2, n_tokens=16)
    inp = synth.draw_layer(cfg, threads=1)
    pred = routing_predicate(inp.router, 2, margin=1.0)
    x, attempts = synth.draw_tokens(cfg, accept=pred)
    L = om.router_logits(inp.router, x)
    top = -np.sort(-L, axis=1)[:, :3]
    assert np.all(top[:, :-1] - top[:, 1:] >= 1.0)
    assert sum(attempts) > 0       # a margin of 1 at logit sigma ~ 8 rejects some draws


def test_disjoint_predicate_gives_disjoint_sets():
    cfg = small_config(n_experts=120, top_k=8, n_tokens=4, routing="disjoint")
    inp = synth.draw_layer(cfg, threads=1)
    pred = routing_predicate(inp.router, 8, disjoint=True)
    x, _ = synth.draw_tokens(cfg, accept=pred)
    ids = om.route(inp.router, x, 8)["ids"]
    assert len(set(ids.reshape(-1).tolist())) == 32


@pytest.mark.parametrize("expert_type", ["q8_0", "q4_k"])
def test_threaded_expert_loop_gives_the_same_layer(expert_type):
    # The oracle's optional thread pool only changes where each expert's FFN
    # runs: outputs, ids and weights equal the one-thread evaluation bit for bit.
    cfg = small_config(n_experts=12, top_k=3, n_tokens=9, expert_type=expert_type,
                       ffn=256, shared_ffn=64)
    inp = synth.draw_layer(cfg, threads=1)
    x, _ = synth.draw_tokens(cfg)
    kw = oracle_kwargs(inp)
    one = om.moe_layer(x, inp.router, inp.gate, inp.up, inp.down, **kw)
    many = om.moe_layer(x, inp.router, inp.gate, inp.up, inp.down, workers=4, **kw)
    assert np.array_equal(one["ids"], many["ids"])
    assert np.array_equal(one["w"], many["w"])
    assert np.array_equal(one["y"], many["y"])
    assert len(one["active"]) > 3
