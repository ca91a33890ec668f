"""ctypes binding of the C ABI in include/moe_layer.h.

Argument marshalling only: torch tensors are checked for device, dtype and
contiguity and passed as raw device pointers; the HIP stream is torch's
current stream.  Every step of the layer runs in the HIP library; there is
no fallback, so a missing library raises.
"""

from __future__ import annotations

import ctypes
import dataclasses
import os
from typing import Optional, Sequence

import torch  # load torch first: the library then binds to torch's HIP runtime

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "lib", "libsvr_moe.so")

F32, Q8_0, Q4_K, Q2_K, Q3_K, Q6_K = 0, 1, 2, 3, 4, 5
_DTYPES = {"f32": F32, "q8_0": Q8_0, "q4_k": Q4_K, "q2_k": Q2_K, "q3_k": Q3_K, "q6_k": Q6_K}

OK, ERR_NULL, ERR_SHAPE, ERR_DTYPE, ERR_WORKSPACE, ERR_LAUNCH, ERR_ARG = range(7)


class MoeError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: status {status} ({strerror(status)})")
        self.status = status


class _Desc(ctypes.Structure):
    _fields_ = [("hidden", ctypes.c_int32), ("n_experts", ctypes.c_int32),
                ("top_k", ctypes.c_int32), ("ffn", ctypes.c_int32),
                ("shared_ffn", ctypes.c_int32), ("expert_type", ctypes.c_int32),
                ("shared_type", ctypes.c_int32), ("flags", ctypes.c_int32),
                ("down_type", ctypes.c_int32)]


class _Weights(ctypes.Structure):
    _fields_ = [("router", ctypes.c_void_p), ("gate", ctypes.c_void_p), ("up", ctypes.c_void_p),
                ("down", ctypes.c_void_p), ("shared_gate", ctypes.c_void_p),
                ("shared_up", ctypes.c_void_p), ("shared_down", ctypes.c_void_p)]


@dataclasses.dataclass(frozen=True)
class LayerDesc:
    hidden: int
    n_experts: int
    top_k: int
    ffn: int
    shared_ffn: int = 0
    expert_type: str = "q4_k"
    shared_type: str = "q8_0"
    down_type: Optional[str] = None  # routed down; None: expert_type

    def c(self) -> _Desc:
        return _Desc(self.hidden, self.n_experts, self.top_k, self.ffn, self.shared_ffn,
                     _DTYPES[self.expert_type], _DTYPES[self.shared_type], 0,
                     _DTYPES[self.down_type] if self.down_type else 0)


@dataclasses.dataclass
class LayerWeights:
    """Device tensors of one layer (uint8 for quantised tensors)."""
    router: torch.Tensor
    gate: torch.Tensor
    up: torch.Tensor
    down: torch.Tensor
    shared_gate: Optional[torch.Tensor] = None
    shared_up: Optional[torch.Tensor] = None
    shared_down: Optional[torch.Tensor] = None

    def c(self) -> _Weights:
        p = lambda t: None if t is None else _ptr(t, None)  # noqa: E731
        return _Weights(_ptr(self.router, torch.float32), p(self.gate), p(self.up), p(self.down),
                        p(self.shared_gate), p(self.shared_up), p(self.shared_down))


_lib = None


def lib():
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"HIP library not found at {LIB_PATH}; build it with "
                               "`python -m speculative_verify_router_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        i32, i64, vp, sz = ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p, ctypes.c_size_t
        D, W = ctypes.POINTER(_Desc), ctypes.POINTER(_Weights)
        sig = {
            "moe_version": (i32, []),
            "moe_strerror": (ctypes.c_char_p, [i32]),
            "moe_tensor_bytes": (i32, [i32, i64, i64, ctypes.POINTER(i64)]),
            "moe_workspace_bytes": (i32, [D, i32, ctypes.POINTER(sz)]),
            "moe_route": (i32, [D, vp, vp, i32, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]),
            "moe_layer_forward": (i32, [D, W, vp, i32, vp, vp, vp, vp, sz, vp]),
            "moe_layer_forward_timed": (i32, [D, W, vp, i32, vp, vp, vp, vp, sz, vp,
                                              ctypes.POINTER(vp), i32]),
            "moe_layer_forward_noalloc": (i32, [D, W, vp, i32, vp, vp, vp, vp]),
            "moe_stage_count": (i32, [D, i32]),
            "moe_stage_name": (ctypes.c_char_p, [D, i32, i32]),
            "moe_dequant_rows": (i32, [i32, vp, i64, i32, i64, i64, vp, vp]),
            "moe_accept_workspace_bytes": (i32, [i32, i64, ctypes.POINTER(sz)]),
            "moe_verify_accept": (i32, [vp, i32, i64, vp, vp, i32, vp, vp, vp, vp, vp, sz, vp]),
        }
        for name, (res, args) in sig.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


# Exported names of the C ABI (the header declares exactly these).
C_SYMBOLS = ("moe_version", "moe_strerror", "moe_tensor_bytes", "moe_workspace_bytes",
             "moe_route", "moe_layer_forward", "moe_layer_forward_timed",
             "moe_layer_forward_noalloc", "moe_stage_count",
             "moe_stage_name", "moe_dequant_rows", "moe_accept_workspace_bytes",
             "moe_verify_accept")


def _ptr(t: Optional[torch.Tensor], dtype) -> Optional[int]:
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("expected a device tensor")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"expected {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError("expected a contiguous tensor")
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def _check(status: int, what: str):
    if status != OK:
        raise MoeError(status, what)


def moe_version() -> int:
    return lib().moe_version()


def strerror(status: int) -> str:
    return lib().moe_strerror(status).decode()


def moe_strerror(status: int) -> str:
    return strerror(status)


def moe_tensor_bytes(dtype: str, rows: int, cols: int) -> int:
    out = ctypes.c_int64()
    _check(lib().moe_tensor_bytes(_DTYPES[dtype], rows, cols, ctypes.byref(out)), "moe_tensor_bytes")
    return out.value


def moe_workspace_bytes(desc: LayerDesc, max_tokens: int) -> int:
    out = ctypes.c_size_t()
    d = desc.c()
    _check(lib().moe_workspace_bytes(ctypes.byref(d), max_tokens, ctypes.byref(out)),
           "moe_workspace_bytes")
    return out.value


def moe_stage_count(desc: LayerDesc, n_tokens: int) -> int:
    d = desc.c()
    n = lib().moe_stage_count(ctypes.byref(d), n_tokens)
    if n <= 0:
        raise MoeError(-n, "moe_stage_count")
    return n


def moe_stage_name(desc: LayerDesc, n_tokens: int, i: int) -> Optional[str]:
    d = desc.c()
    s = lib().moe_stage_name(ctypes.byref(d), n_tokens, i)
    return None if s is None else s.decode()


# Leading workspace bytes that hold hand-off counters (zero between calls).
COUNTER_BYTES = 16384


def workspace(desc: LayerDesc, max_tokens: int, device="cuda") -> torch.Tensor:
    """A zero-filled device workspace of moe_workspace_bytes(desc, max_tokens)
    bytes (its counter page must start at zero; calls keep it so)."""
    n = max(moe_workspace_bytes(desc, max_tokens), COUNTER_BYTES)
    return torch.zeros(n, dtype=torch.uint8, device=device)


def moe_route(desc: LayerDesc, router: torch.Tensor, x: torch.Tensor, topk_ids: torch.Tensor,
              topk_w: torch.Tensor, expert_counts=None, expert_offsets=None, token_slots=None,
              active_experts=None, n_active=None, ws: torch.Tensor = None, stream=None):
    M = x.shape[0] if x.dim() == 2 else 0
    d = desc.c()
    if ws is None:
        ws = workspace(desc, M, x.device)
    i32 = torch.int32
    st = lib().moe_route(ctypes.byref(d), _ptr(router, torch.float32), _ptr(x, torch.float32), M,
                         _ptr(topk_ids, i32), _ptr(topk_w, torch.float32),
                         _ptr(expert_counts, i32), _ptr(expert_offsets, i32),
                         _ptr(token_slots, i32), _ptr(active_experts, i32), _ptr(n_active, i32),
                         _ptr(ws, torch.uint8), ws.numel(), _stream(stream))
    _check(st, "moe_route")


def moe_layer_forward(desc: LayerDesc, weights: LayerWeights, x: torch.Tensor, y: torch.Tensor,
                      topk_ids=None, topk_w=None, ws: torch.Tensor = None, stream=None):
    M = x.shape[0]
    d, w = desc.c(), weights.c()
    if ws is None:
        ws = workspace(desc, M, x.device)
    st = lib().moe_layer_forward(ctypes.byref(d), ctypes.byref(w), _ptr(x, torch.float32), M,
                                 _ptr(y, torch.float32), _ptr(topk_ids, torch.int32),
                                 _ptr(topk_w, torch.float32), _ptr(ws, torch.uint8), ws.numel(),
                                 _stream(stream))
    _check(st, "moe_layer_forward")


def moe_layer_forward_timed(desc: LayerDesc, weights: LayerWeights, x: torch.Tensor,
                            y: torch.Tensor, events: Sequence, topk_ids=None, topk_w=None,
                            ws: torch.Tensor = None, stream=None):
    """``events``: moe_stage_count(desc, M) + 1 raw hipEvent_t handles (ints)."""
    M = x.shape[0]
    d, w = desc.c(), weights.c()
    if ws is None:
        ws = workspace(desc, M, x.device)
    arr = (ctypes.c_void_p * len(events))(*events)
    st = lib().moe_layer_forward_timed(ctypes.byref(d), ctypes.byref(w), _ptr(x, torch.float32), M,
                                       _ptr(y, torch.float32), _ptr(topk_ids, torch.int32),
                                       _ptr(topk_w, torch.float32), _ptr(ws, torch.uint8),
                                       ws.numel(), _stream(stream), arr, len(events))
    _check(st, "moe_layer_forward_timed")


# Workspace bytes that moe_layer_forward_noalloc holds per GPU (MOE_NOALLOC_MAX_WORKSPACE).
NOALLOC_MAX_WORKSPACE = 8 << 20


def moe_layer_forward_noalloc(desc: LayerDesc, weights: LayerWeights, x: torch.Tensor,
                              y: torch.Tensor, topk_ids=None, topk_w=None, stream=None):
    """moe_layer_forward with the library's own per-GPU workspace (no allocation)."""
    M = x.shape[0]
    d, w = desc.c(), weights.c()
    st = lib().moe_layer_forward_noalloc(ctypes.byref(d), ctypes.byref(w), _ptr(x, torch.float32),
                                         M, _ptr(y, torch.float32), _ptr(topk_ids, torch.int32),
                                         _ptr(topk_w, torch.float32), _stream(stream))
    _check(st, "moe_layer_forward_noalloc")


class PreparedForward:
    """A moe_layer_forward call with its arguments marshalled once.

    The tensors are captured by reference (their device pointers are fixed);
    calling the object enqueues the layer again on the captured stream.
    ``events`` (raw hipEvent_t handles), if given per call, selects
    moe_layer_forward_timed.
    """

    def __init__(self, desc: LayerDesc, weights: LayerWeights, x: torch.Tensor, y: torch.Tensor,
                 topk_ids=None, topk_w=None, ws: torch.Tensor = None, stream=None):
        self._keep = (weights, x, y, topk_ids, topk_w)
        if ws is None:
            ws = workspace(desc, x.shape[0], x.device)
        self._ws = ws
        self._d = desc.c()
        self._w = weights.c()
        vp = ctypes.c_void_p
        self._args = (ctypes.byref(self._d), ctypes.byref(self._w), vp(_ptr(x, torch.float32)),
                      ctypes.c_int32(x.shape[0]), vp(_ptr(y, torch.float32)),
                      vp(_ptr(topk_ids, torch.int32)), vp(_ptr(topk_w, torch.float32)),
                      vp(_ptr(ws, torch.uint8)), ctypes.c_size_t(ws.numel()),
                      vp(_stream(stream)))
        self._f = lib().moe_layer_forward
        self._ft = lib().moe_layer_forward_timed

    def __call__(self, events=None):
        if events is None:
            st = self._f(*self._args)
        else:
            st = self._ft(*self._args, events, len(events))
        if st != OK:
            raise MoeError(st, "moe_layer_forward")


def moe_dequant_rows(dtype: str, tensor: torch.Tensor, rows: int, cols: int, row_start: int,
                     row_count: int, out: torch.Tensor, stream=None):
    st = lib().moe_dequant_rows(_DTYPES[dtype], _ptr(tensor, None), rows, cols, row_start,
                                row_count, _ptr(out, torch.float32), _stream(stream))
    _check(st, "moe_dequant_rows")


# include/moe_accept.h: greedy verify/accept of an MTP verify batch.
ACCEPT_MAX_ROWS = 64


def moe_accept_workspace_bytes(max_rows: int, vocab: int) -> int:
    out = ctypes.c_size_t()
    _check(lib().moe_accept_workspace_bytes(max_rows, vocab, ctypes.byref(out)),
           "moe_accept_workspace_bytes")
    return out.value


def accept_workspace(max_rows: int, vocab: int, device="cuda") -> torch.Tensor:
    """A zero-filled device workspace for moe_verify_accept (its counter line
    must start at zero; calls keep it so)."""
    return torch.zeros(moe_accept_workspace_bytes(max_rows, vocab), dtype=torch.uint8,
                       device=device)


def moe_verify_accept(logits: torch.Tensor, drafts: Optional[torch.Tensor], tokens: torch.Tensor,
                      accepted: torch.Tensor, n_accepted: torch.Tensor,
                      verify_h: Optional[torch.Tensor] = None,
                      pending_h: Optional[torch.Tensor] = None, ws: torch.Tensor = None,
                      stream=None, n_rows: Optional[int] = None, vocab: Optional[int] = None):
    """logits [M][V] float32; drafts [M-1] int32 (None for M == 1); tokens,
    accepted [M] and n_accepted [1] int32 outputs; verify_h [M][h] and
    pending_h [h] float32, both or neither.  ``n_rows``/``vocab`` override
    the shape read from ``logits`` (for error-path tests)."""
    M = logits.shape[0] if n_rows is None else n_rows
    V = logits.shape[-1] if vocab is None else vocab
    if ws is None:
        ws = accept_workspace(max(M, 1), max(V, 1), logits.device)
    h_dim = 0 if verify_h is None else verify_h.shape[-1]
    i32 = torch.int32
    st = lib().moe_verify_accept(_ptr(logits, torch.float32), M, V, _ptr(drafts, i32),
                                 _ptr(verify_h, torch.float32), h_dim, _ptr(tokens, i32),
                                 _ptr(accepted, i32), _ptr(n_accepted, i32),
                                 _ptr(pending_h, torch.float32), _ptr(ws, torch.uint8), ws.numel(),
                                 _stream(stream))
    _check(st, "moe_verify_accept")
