"""Routed mixture-of-experts verify layer for AMD Instinct MI355X (gfx950).

One routed-MoE FFN block (F32 softmax top-k router, Q8_0 / Q4_K / Q2_K / Q3_K / Q6_K experts,
SwiGLU, a shared expert and a weighted combine) applied to the verify batch
of MTP speculative decoding, implemented as hand-written HIP kernels behind
the C ABI of ``include/moe_layer.h``, plus greedy MTP verify/accept
(``include/moe_accept.h``).  This package is the thin Python
binding of that ABI (``_binding``) and the build helper (``build``).
"""

from ._binding import (  # noqa: F401
    ACCEPT_MAX_ROWS,
    C_SYMBOLS,
    LIB_PATH,
    LayerDesc,
    LayerWeights,
    NOALLOC_MAX_WORKSPACE,
    MoeError,
    PreparedForward,
    accept_workspace,
    lib,
    moe_accept_workspace_bytes,
    moe_dequant_rows,
    moe_layer_forward,
    moe_layer_forward_noalloc,
    moe_layer_forward_timed,
    moe_route,
    moe_stage_count,
    moe_stage_name,
    moe_strerror,
    moe_tensor_bytes,
    moe_verify_accept,
    moe_version,
    moe_workspace_bytes,
    workspace,
)
