"""C-ABI checks that need no GPU: the library loads, exports every entry
point the header declares, sizes its tensors and workspace, and rejects bad
arguments with the documented status before enqueueing anything."""

import ctypes
import os
import re

import pytest

import speculative_verify_router_amd as svr
from speculative_verify_router_amd import _binding as B
import synth

INCLUDE = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include")


def _declared():
    names = set()
    for h in sorted(os.listdir(INCLUDE)):
        if h.endswith(".h"):
            text = re.sub(r"/\*.*?\*/", "", open(os.path.join(INCLUDE, h)).read(), flags=re.S)
            names |= set(re.findall(r"\b(moe_[a-z_]+)\s*\(", text))
    return sorted(names)


def test_header_declares_the_binding_symbols():
    assert _declared() == sorted(B.C_SYMBOLS)


def test_library_loads_and_exports_every_declared_symbol():
    L = svr.lib()
    for name in _declared():
        assert hasattr(L, name), name
    assert svr.moe_version() >= 100
    assert svr.moe_strerror(0) == "ok"
    assert svr.moe_strerror(12345) == "unknown status"



def _stage_names(desc, M):
    return [svr.moe_stage_name(desc, M, i) for i in range(svr.moe_stage_count(desc, M))]


def test_stage_lists_follow_the_launch_path():
    # Step-3.5-shaped verify layer: three stages up to 16 tokens.
    d = svr.LayerDesc(4096, 288, 8, 1280, 1280, "q4_k", "q8_0")
    for M in (1, 2, 3, 4, 5, 16):
        assert _stage_names(d, M) == ["route_shared_gateup", "gateup", "down_combine"]
        assert _stage_names(svr.LayerDesc(4096, 288, 8, 1280, 0, "q4_k", "q8_0"), M) == [
            "route_shared_gateup", "gateup", "down_combine"]
    # Batches above 16 tokens: the grouped-GEMM path.
    for M in (17, 512):
        assert _stage_names(d, M) == ["route", "shared_gateup", "gateup", "shared_down",
                                      "down_combine"]
    # Shapes without a fused instantiation take the same three stages.
    odd = svr.LayerDesc(640, 5, 2, 96, 160, "q8_0", "q8_0")
    assert _stage_names(odd, 2) == ["route_shared_gateup", "gateup", "down_combine"]
    assert svr.moe_stage_name(d, 4, -1) is None and svr.moe_stage_name(d, 4, 3) is None
    with pytest.raises(svr.MoeError):
        svr.moe_stage_count(svr.LayerDesc(4096, 288, 8, 1000, 0, "q4_k", "q8_0"), 4)


def test_missing_library_fails_loudly(monkeypatch):
    monkeypatch.setattr(B, "LIB_PATH", "/nonexistent/libsvr_moe.so")
    monkeypatch.setattr(B, "_lib", None)
    with pytest.raises(RuntimeError, match="not found"):
        B.lib()


@pytest.mark.parametrize("dtype,rows,cols", [("q8_0", 1, 32), ("q8_0", 1280, 4096), ("q8_0", 7, 96),
                                             ("q4_k", 5, 256), ("q4_k", 352 * 1536, 4096),
                                             ("q2_k", 1, 256), ("q2_k", 3, 512),
                                             ("q2_k", 352 * 4096, 1536), ("q3_k", 1, 256),
                                             ("q3_k", 5, 768), ("q3_k", 352 * 4096, 1536),
                                             ("q6_k", 1, 256), ("q6_k", 3, 1280),
                                             ("q6_k", 288 * 1280, 4096),
                                             ("f32", 3, 5)])
def test_tensor_bytes_match_the_generator(dtype, rows, cols):
    assert svr.moe_tensor_bytes(dtype, rows, cols) == synth.tensor_bytes(dtype, rows, cols)


def test_tensor_bytes_rejects_bad_shapes():
    with pytest.raises(svr.MoeError) as e:
        svr.moe_tensor_bytes("q4_k", 4, 100)
    assert e.value.status == B.ERR_SHAPE
    out = ctypes.c_int64()
    assert svr.lib().moe_tensor_bytes(9, 1, 32, ctypes.byref(out)) == B.ERR_DTYPE
    assert svr.lib().moe_tensor_bytes(1, 1, 32, None) == B.ERR_NULL


def _desc(**kw):
    base = dict(hidden=4096, n_experts=288, top_k=8, ffn=1280, shared_ffn=1280,
                expert_type="q4_k", shared_type="q8_0")
    base.update(kw)
    return svr.LayerDesc(**base)


def test_workspace_grows_with_tokens():
    a = svr.moe_workspace_bytes(_desc(), 1)
    b = svr.moe_workspace_bytes(_desc(), 4)
    c = svr.moe_workspace_bytes(_desc(), 512)
    assert 0 < a < b < c
    assert a % 256 == 0


@pytest.mark.parametrize("kw,status", [
    (dict(hidden=4000), B.ERR_SHAPE),            # not a multiple of 256 for Q4_K
    (dict(ffn=1000), B.ERR_SHAPE),
    (dict(shared_ffn=100), B.ERR_SHAPE),
    (dict(n_experts=0), B.ERR_SHAPE),
    (dict(n_experts=2000), B.ERR_SHAPE),
    (dict(top_k=0), B.ERR_SHAPE),
    (dict(top_k=300), B.ERR_SHAPE),
    (dict(top_k=65, n_experts=100), B.ERR_SHAPE),
        (dict(hidden=100, expert_type="q8_0", shared_type="q8_0"), B.ERR_SHAPE),  # not k*32
    (dict(expert_type="f32"), B.ERR_DTYPE),
    (dict(shared_type="f32"), B.ERR_DTYPE),
    (dict(shared_type="q2_k"), B.ERR_DTYPE),           # 2-bit: routed experts only
    (dict(expert_type="q2_k", ffn=1000), B.ERR_SHAPE),
    (dict(expert_type="q2_k", hidden=65536, shared_ffn=0), B.ERR_SHAPE),  # > 512 chunks a row
    (dict(shared_type="q3_k"), B.ERR_DTYPE),
    (dict(shared_type="q6_k"), B.ERR_DTYPE),
    (dict(expert_type="q6_k", hidden=32768, shared_ffn=0), B.ERR_SHAPE),  # > 512 chunks a row
    (dict(expert_type="q2_k", down_type="q3_k", ffn=1000), B.ERR_SHAPE),
    (dict(expert_type="q8_0", down_type="q4_k", ffn=96), B.ERR_SHAPE),  # Q8_0 F fits, Q4_K does not
])
def test_bad_descriptors_are_rejected(kw, status):
    d = _desc(**kw).c()
    out = ctypes.c_size_t()
    assert svr.lib().moe_workspace_bytes(ctypes.byref(d), 4, ctypes.byref(out)) == status


def test_q2_k_routed_experts_are_accepted():
    for M in (1, 4, 16, 512):
        assert svr.moe_workspace_bytes(_desc(expert_type="q2_k"), M) > 0
    # 2-bit experts have a matrix-core decoder: large batches take the five stages
    d = _desc(expert_type="q2_k").c()
    assert svr.lib().moe_stage_count(ctypes.byref(d), 512) == 5
    assert svr.lib().moe_stage_count(ctypes.byref(_desc().c()), 512) == 5


def test_routed_down_type_selects_the_path():
    mixed = _desc(expert_type="q2_k", down_type="q3_k")
    for M in (1, 4, 16, 512):
        assert svr.moe_workspace_bytes(mixed, M) > 0
    L = svr.lib()
    # matrix-core path for every routed type, gate/up and down types apart
    assert L.moe_stage_count(ctypes.byref(mixed.c()), 512) == 5
    assert L.moe_stage_count(ctypes.byref(_desc(expert_type="q6_k").c()), 512) == 5
    assert L.moe_stage_count(ctypes.byref(_desc(down_type="q6_k").c()), 512) == 5
    assert L.moe_stage_count(ctypes.byref(_desc(expert_type="q6_k").c()), 16) == 3
    assert L.moe_stage_count(ctypes.byref(_desc(down_type="q4_k").c()), 512) == 5
    assert L.moe_stage_count(ctypes.byref(_desc(down_type="q8_0").c()), 512) == 5
    # verify batches: the staged path, gate/up and down types apart
    assert L.moe_stage_count(ctypes.byref(_desc(down_type="q8_0").c()), 4) == 3
    assert L.moe_stage_count(ctypes.byref(mixed.c()), 4) == 3
    out = ctypes.c_size_t()
    bad = _desc().c()
    bad.down_type = 9
    assert L.moe_workspace_bytes(ctypes.byref(bad), 4, ctypes.byref(out)) == B.ERR_DTYPE


def test_shared_type_ignored_without_shared_expert():
    d = _desc(shared_ffn=0, shared_type="f32").c()
    out = ctypes.c_size_t()
    assert svr.lib().moe_workspace_bytes(ctypes.byref(d), 4, ctypes.byref(out)) == B.OK


FAKE = 1 << 20  # never dereferenced: every call below fails validation first


def _fake_weights(**kw):
    w = B._Weights(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE)
    for k, v in kw.items():
        setattr(w, k, v)
    return w


def _forward(desc=None, weights=None, x=FAKE, M=4, y=FAKE, ws=FAKE, ws_bytes=1 << 40):
    L = svr.lib()
    d = desc if desc is not None else _desc().c()
    w = weights if weights is not None else _fake_weights()
    return L.moe_layer_forward(ctypes.byref(d) if d else None, ctypes.byref(w) if w else None,
                               x, M, y, None, None, ws, ws_bytes, None)


def test_forward_error_paths():
    need = svr.moe_workspace_bytes(_desc(), 4)
    assert _forward(ws_bytes=need - 1) == B.ERR_WORKSPACE
    assert _forward(x=None) == B.ERR_NULL
    assert _forward(y=None) == B.ERR_NULL
    assert _forward(ws=None) == B.ERR_NULL
    assert _forward(weights=_fake_weights(gate=None)) == B.ERR_NULL
    assert _forward(weights=_fake_weights(shared_down=None)) == B.ERR_NULL
    assert _forward(M=-1) == B.ERR_NULL
    assert _forward(desc=_desc(ffn=100).c()) == B.ERR_SHAPE
    assert _forward(x=FAKE + 4) == B.ERR_ARG          # misaligned activations
    assert _forward(ws=FAKE + 16) == B.ERR_ARG        # misaligned workspace
    L = svr.lib()
    assert L.moe_layer_forward(None, None, FAKE, 4, FAKE, None, None, FAKE, 1 << 40, None) == B.ERR_NULL


def test_forward_timed_checks_the_event_count():
    L = svr.lib()
    d, w = _desc().c(), _fake_weights()
    # One event more than the stage count + 1: rejected before anything runs.
    n = svr.moe_stage_count(_desc(), 4) + 2
    evs = (ctypes.c_void_p * n)(*range(1, n + 1))
    st = L.moe_layer_forward_timed(ctypes.byref(d), ctypes.byref(w), FAKE, 4, FAKE, None, None,
                                   FAKE, 1 << 40, None, evs, n)
    assert st == B.ERR_ARG
    st = L.moe_layer_forward_timed(ctypes.byref(d), ctypes.byref(w), FAKE, 4, FAKE, None, None,
                                   FAKE, 1 << 40, None, None, 0)
    assert st == B.ERR_NULL


def test_route_and_dequant_error_paths():
    L = svr.lib()
    d = _desc().c()
    st = L.moe_route(ctypes.byref(d), FAKE, FAKE, 4, None, FAKE, None, None, None, None, None,
                     FAKE, 1 << 40, None)
    assert st == B.ERR_NULL
    st = L.moe_route(ctypes.byref(d), FAKE, FAKE, 4, FAKE, FAKE, None, None, None, None, None,
                     FAKE, 10, None)
    assert st == B.ERR_WORKSPACE
    assert L.moe_dequant_rows(7, FAKE, 10, 256, 0, 10, FAKE, None) == B.ERR_DTYPE
    assert L.moe_dequant_rows(2, FAKE, 10, 100, 0, 10, FAKE, None) == B.ERR_SHAPE
    assert L.moe_dequant_rows(1, FAKE, 10, 64, 5, 6, FAKE, None) == B.ERR_SHAPE
    assert L.moe_dequant_rows(1, None, 10, 64, 0, 5, FAKE, None) == B.ERR_NULL
    assert L.moe_dequant_rows(1, None, 10, 64, 0, 0, None, None) == B.OK    # empty range


def test_reserved_flags_must_be_zero():
    d = _desc().c()
    out = ctypes.c_size_t()
    assert svr.lib().moe_workspace_bytes(ctypes.byref(d), 4, ctypes.byref(out)) == B.OK
    for bad in (1, 2, -1):
        d.flags = bad
        assert svr.lib().moe_workspace_bytes(ctypes.byref(d), 4, ctypes.byref(out)) == B.ERR_ARG


# --- include/moe_accept.h ---------------------------------------------------


def test_accept_workspace_sizes():
    small = svr.moe_accept_workspace_bytes(4, 1000)
    big = svr.moe_accept_workspace_bytes(4, 131072)
    assert 256 < small <= big and big % 256 == 0
    assert svr.moe_accept_workspace_bytes(64, 1 << 30) >= svr.moe_accept_workspace_bytes(4, 1 << 30)
    L = svr.lib()
    out = ctypes.c_size_t()
    assert L.moe_accept_workspace_bytes(0, 10, ctypes.byref(out)) == B.ERR_SHAPE
    assert L.moe_accept_workspace_bytes(65, 10, ctypes.byref(out)) == B.ERR_SHAPE
    assert L.moe_accept_workspace_bytes(4, 0, ctypes.byref(out)) == B.ERR_SHAPE
    assert L.moe_accept_workspace_bytes(4, (1 << 30) + 1, ctypes.byref(out)) == B.ERR_SHAPE
    assert L.moe_accept_workspace_bytes(4, 10, None) == B.ERR_NULL


def _accept(logits=FAKE, M=4, V=131072, drafts=FAKE, vh=FAKE, hd=4096, tokens=FAKE, acc=FAKE,
            n=FAKE, pend=FAKE, ws=FAKE, ws_bytes=1 << 40):
    return svr.lib().moe_verify_accept(logits, M, V, drafts, vh, hd, tokens, acc, n, pend, ws,
                                       ws_bytes, None)


def test_accept_error_paths():
    need = svr.moe_accept_workspace_bytes(4, 131072)
    assert _accept(ws_bytes=need - 1) == B.ERR_WORKSPACE
    assert _accept(logits=None) == B.ERR_NULL
    assert _accept(tokens=None) == B.ERR_NULL
    assert _accept(acc=None) == B.ERR_NULL
    assert _accept(n=None) == B.ERR_NULL
    assert _accept(ws=None) == B.ERR_NULL
    assert _accept(drafts=None) == B.ERR_NULL            # drafts needed with more than one row
    assert _accept(pend=None) == B.ERR_NULL              # verify_h without pending_h
    assert _accept(vh=None, hd=16) == B.ERR_NULL         # pending_h without verify_h
    assert _accept(vh=None, pend=None, hd=16) == B.ERR_SHAPE
    assert _accept(M=-1) == B.ERR_SHAPE
    assert _accept(M=65) == B.ERR_SHAPE
    assert _accept(V=0) == B.ERR_SHAPE
    assert _accept(V=(1 << 30) + 1) == B.ERR_SHAPE
    assert _accept(hd=-1) == B.ERR_SHAPE
    assert _accept(ws=FAKE + 16) == B.ERR_ARG            # misaligned workspace
    assert _accept(logits=FAKE + 2) == B.ERR_ARG         # logits not 4-byte aligned
    assert _accept(M=0, logits=None, ws=None) == B.OK    # empty batch: nothing enqueued


def test_noalloc_limit_matches_header_and_rejects_large_batches():
    text = open(os.path.join(INCLUDE, "moe_layer.h")).read()
    m = re.search(r"#define MOE_NOALLOC_MAX_WORKSPACE \((\d+)u << (\d+)\)", text)
    assert m and int(m.group(1)) << int(m.group(2)) == svr.NOALLOC_MAX_WORKSPACE
    L = svr.lib()
    step5 = svr.LayerDesc(4096, 352, 8, 1536, 1536, "q4_k", "q8_0")
    # A 16-token verify batch fits the library's workspace; a 512-token
    # prefill batch does not, and is refused before anything is enqueued.
    assert svr.moe_workspace_bytes(step5, 16) <= svr.NOALLOC_MAX_WORKSPACE
    assert svr.moe_workspace_bytes(step5, 512) > svr.NOALLOC_MAX_WORKSPACE
    w = B._Weights()
    assert L.moe_layer_forward_noalloc(ctypes.byref(step5.c()), ctypes.byref(w), None, 512, None,
                                       None, None, None) == B.ERR_WORKSPACE
    assert L.moe_layer_forward_noalloc(None, ctypes.byref(w), None, 4, None, None, None,
                                       None) == B.ERR_NULL
    bad = step5.c()
    bad.flags = 1
    assert L.moe_layer_forward_noalloc(ctypes.byref(bad), ctypes.byref(w), None, 4, None, None,
                                       None, None) == B.ERR_ARG
