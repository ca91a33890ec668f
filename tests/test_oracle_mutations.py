"""Planted mistakes in the oracle must be caught by its pins (CPU only).

Each case patches one oracle function with a plausible slip (a wrong bias, a
swapped nibble, a flipped sign, a wrong tie-break, a dropped term) and runs
the pin tests of ``test_oracle_pins``; at least one pin must fail.
"""

import contextlib

import numpy as np
import pytest

from oracle import moe_oracle as om
import test_oracle_pins as P

_orig = {name: getattr(om, name) for name in dir(om) if callable(getattr(om, name))}


def _pins():
    yield P.test_f16_decode_all_bit_patterns_match_numpy
    for fx, dt in P.FIXTURES:
        yield lambda fx=fx, dt=dt: P.test_dequant_matches_hand_derived_fixture(fx, dt)
    yield P.test_dequant_fixture_twin_agrees
    yield P.test_q8_0_requantise_roundtrip_is_byte_exact
    for s in (0, 3, 7):
        yield lambda s=s: P.test_q4_k_single_field_positions(s)
    yield P.test_q4_k_multi_row_record_order
    for s in (0, 5, 15):
        yield lambda s=s: P.test_q2_k_single_field_positions(s)
    yield P.test_q2_k_multi_row_record_order
    for s in (0, 1, 11):
        yield lambda s=s: P.test_q3_k_single_field_positions(s)
    yield P.test_q3_k_multi_row_record_order
    for s in (0, 7, 15):
        yield lambda s=s: P.test_q6_k_single_field_positions(s)
    yield P.test_q6_k_multi_row_record_order
    yield P.test_router_logits_unit_vectors_pick_columns
    yield P.test_select_ties_go_to_lower_index
    yield P.test_select_matches_brute_force_sort
    yield P.test_routing_weights_sum_to_one_and_k1_is_one
    yield P.test_k_equals_E_is_the_textbook_softmax
    yield P.test_renormalised_weights_equal_softmax_over_selected
    yield P.test_bucket_matches_brute_force
    yield P.test_silu_is_g_times_logistic
    for args in [("q8_0", 256, 128, 0, 8), ("q8_0", 256, 64, 96, 4)]:
        yield lambda a=args: P.test_oracle_matches_scalar_twin(*a)
    yield P.test_one_expert_top1_layer_is_dense_swiglu_ffn
    for et in ("q8_0", "q4_k", "q2_k", "q3_k", "q6_k"):
        yield lambda et=et: P.test_doubling_down_scales_doubles_routed_part_exactly(et)
    yield P.test_rows_are_independent_of_batch


# --- the planted mistakes -------------------------------------------------

def _f16_bias(bits):
    return _orig["f16_to_f64"](bits) * 2.0


def _f16_no_subnormal(bits):
    b = np.asarray(bits).astype(np.int64) & 0xFFFF
    v = _orig["f16_to_f64"](bits)
    return np.where(((b >> 10) & 31) == 0, 0.0, v)


def _q4k_fields_swapped_nibbles(*a, **k):
    d, dmin, sc, m, q = _orig["q4_k_fields"](*a, **k)
    q2 = q.copy()
    q2[:, :, 0::2], q2[:, :, 1::2] = q[:, :, 1::2], q[:, :, 0::2]
    return d, dmin, sc, m, q2


def _q4k_field_shifted(sbytes, bit):
    return _orig["_q4_k_field"](sbytes, bit - 6 if bit >= 48 else bit)


def _q4k_plus_min(buf, rows, cols, row_start=0, row_count=None):
    r0, n = om._rows(rows, row_start, row_count)
    d, dmin, sc, m, q = om.q4_k_fields(buf, rows, cols, r0, n)
    w = d[:, None, None] * sc[:, :, None] * q + dmin[:, None, None] * m[:, :, None]
    return w.reshape(n, cols)


def _q2k_fields_transposed(buf, rows, cols, row_start=0, row_count=None):
    # weight i read from byte i // 4, bits 2 (i % 4): the field order transposed
    d, dmin, sc, m, q = _orig["q2_k_fields"](buf, rows, cols, row_start, row_count)
    return d, dmin, sc, m, q.reshape(q.shape[0], 16, 4, 4).transpose(0, 1, 3, 2).reshape(q.shape)


def _q2k_fields_scale_nibbles_swapped(*a, **k):
    d, dmin, sc, m, q = _orig["q2_k_fields"](*a, **k)
    return d, dmin, m, sc, q


def _q2k_offsets_unpadded(rows, cols):
    ns = cols // 256
    return 4 * rows * ns, 20 * rows * ns


def _q2k_plus_min(buf, rows, cols, row_start=0, row_count=None):
    r0, n = om._rows(rows, row_start, row_count)
    d, dmin, sc, m, q = om.q2_k_fields(buf, rows, cols, r0, n)
    w = d[:, None, None] * sc[:, :, None] * q + dmin[:, None, None] * m[:, :, None]
    return w.reshape(n, cols)


def _q3k_fields_high_nibbles_swapped(buf, rows, cols, row_start=0, row_count=None):
    # high bits of sub-blocks 2p and 2p+1 read from each other's nibble
    d, S, Q = _orig["q3_k_fields"](buf, rows, cols, row_start, row_count)
    low, high = Q & 3, Q >> 2
    high = high.reshape(high.shape[0], 8, 2, 16)[:, :, ::-1, :].reshape(Q.shape)
    return d, S, low | (high << 2)


def _q3k_fields_high_bit_dropped(*a, **k):
    d, S, Q = _orig["q3_k_fields"](*a, **k)
    return d, S, Q & 3


def _q3k_no_scale_offset(buf, rows, cols, row_start=0, row_count=None):
    r0, n = om._rows(rows, row_start, row_count)
    d, S, Q = om.q3_k_fields(buf, rows, cols, r0, n)
    return (d[:, None, None] * S[:, :, None] * (Q - 4)).reshape(n, cols)


def _q3k_quant_offset_sign(buf, rows, cols, row_start=0, row_count=None):
    r0, n = om._rows(rows, row_start, row_count)
    d, S, Q = om.q3_k_fields(buf, rows, cols, r0, n)
    return (d[:, None, None] * (S[:, :, None] - 32) * (Q + 4)).reshape(n, cols)


def _q3k_offsets_unpadded(rows, cols):
    ns = cols // 256
    return 2 * rows * ns, 18 * rows * ns, 82 * rows * ns


def _q6k_fields_high_pairs_swapped(buf, rows, cols, row_start=0, row_count=None):
    # high bits of even and odd weights read from each other's bit pair
    d, sc, Q = _orig["q6_k_fields"](buf, rows, cols, row_start, row_count)
    low, high = Q & 15, Q >> 4
    high = high.reshape(high.shape[0], 16, 8, 2)[:, :, :, ::-1].reshape(Q.shape)
    return d, sc, low | (high << 4)


def _q6k_fields_unsigned_scales(*a, **k):
    d, sc, Q = _orig["q6_k_fields"](*a, **k)
    return d, sc & 255, Q


def _q6k_offset_sign(buf, rows, cols, row_start=0, row_count=None):
    r0, n = om._rows(rows, row_start, row_count)
    d, sc, Q = om.q6_k_fields(buf, rows, cols, r0, n)
    return (d[:, None, None] * sc[:, :, None] * (Q + 32)).reshape(n, cols)


def _q6k_offsets_unpadded(rows, cols):
    ns = cols // 256
    return 2 * rows * ns, 18 * rows * ns, 146 * rows * ns


def _q8_offset_unpadded(rows, cols):
    return 2 * rows * (cols // 32)


def _select_high_tie(logits, k):
    L = np.atleast_2d(np.asarray(logits, dtype=np.float64))
    E = L.shape[1]
    ids = np.empty((L.shape[0], k), dtype=np.int64)
    for t in range(L.shape[0]):
        ids[t] = np.lexsort((-np.arange(E), -L[t]))[:k]
    return ids


def _weights_unnormalised(logits, ids):
    return np.take_along_axis(om.softmax(logits), np.asarray(ids), axis=1)


def _sigmoid_only(g):
    g = np.asarray(g, dtype=np.float64)
    return 1.0 / (1.0 + np.exp(-g))


def _bucket_unstable(ids, n_experts):
    counts, offsets, slots, active = _orig["bucket"](ids, n_experts)
    return counts, offsets, np.argsort(np.asarray(ids).reshape(-1)[::-1], kind="stable")[::-1].copy(), active


def _ffn_no_up(Wg, Wu, Wd, xs):
    xs = np.atleast_2d(np.asarray(xs, dtype=np.float64))
    return om.silu(xs @ Wg.T) @ Wd.T


MUTATIONS = {
    "f16_scale": ("f16_to_f64", _f16_bias),
    "f16_subnormal_flush": ("f16_to_f64", _f16_no_subnormal),
    "q4k_nibble_order": ("q4_k_fields", _q4k_fields_swapped_nibbles),
    "q4k_min_offset": ("_q4_k_field", _q4k_field_shifted),
    "q4k_min_sign": ("dequant_q4_k", _q4k_plus_min),
    "q8_plane_offset": ("q8_0_quant_offset", _q8_offset_unpadded),
    "q2k_field_order": ("q2_k_fields", _q2k_fields_transposed),
    "q2k_scale_nibbles": ("q2_k_fields", _q2k_fields_scale_nibbles_swapped),
    "q2k_plane_offsets": ("q2_k_offsets", _q2k_offsets_unpadded),
    "q2k_min_sign": ("dequant_q2_k", _q2k_plus_min),
    "q3k_high_nibbles": ("q3_k_fields", _q3k_fields_high_nibbles_swapped),
    "q3k_high_bit_dropped": ("q3_k_fields", _q3k_fields_high_bit_dropped),
    "q3k_scale_offset": ("dequant_q3_k", _q3k_no_scale_offset),
    "q3k_quant_offset_sign": ("dequant_q3_k", _q3k_quant_offset_sign),
    "q3k_plane_offsets": ("q3_k_offsets", _q3k_offsets_unpadded),
    "q6k_high_pairs": ("q6_k_fields", _q6k_fields_high_pairs_swapped),
    "q6k_unsigned_scales": ("q6_k_fields", _q6k_fields_unsigned_scales),
    "q6k_offset_sign": ("dequant_q6_k", _q6k_offset_sign),
    "q6k_plane_offsets": ("q6_k_offsets", _q6k_offsets_unpadded),
    "tie_to_higher": ("select_experts", _select_high_tie),
    "no_renormalise": ("routing_weights", _weights_unnormalised),
    "silu_is_sigmoid": ("silu", _sigmoid_only),
    "bucket_order": ("bucket", _bucket_unstable),
    "ffn_drops_up": ("swiglu_ffn", _ffn_no_up),
}


@contextlib.contextmanager
def _patched(name, fn):
    setattr(om, name, fn)
    try:
        yield
    finally:
        setattr(om, name, _orig[name])


@pytest.mark.parametrize("case", sorted(MUTATIONS))
def test_planted_mistake_is_caught(case):
    name, fn = MUTATIONS[case]
    caught = []
    with _patched(name, fn):
        for pin in _pins():
            try:
                with np.errstate(all="ignore"):
                    pin()
            except (AssertionError, ValueError, IndexError):
                caught.append(getattr(pin, "__name__", "pin"))
    assert caught, f"no pin caught the planted mistake {case!r}"


def test_unpatched_pins_pass():
    for pin in _pins():
        pin()
