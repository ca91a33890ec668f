"""Seeded synthetic inputs for the routed-MoE verify layer.

This package draws router weights, activations and block-quantised expert
tensors from fixed seeds and packs them into the byte layouts that
``include/moe_layer.h`` documents.  It holds none of the layer's arithmetic
(no routing, no dequantisation, no matrix products); the CPU oracle and the
HIP library both read the bytes it writes.  ``verify`` draws the seeded
verify batches (logits, drafts, hidden-state rows) of greedy verify/accept.
"""

from .layers import (  # noqa: F401
    CONFIGS,
    LayerConfig,
    LayerInputs,
    draw_layer,
    draw_tokens,
    q2_k_bytes,
    q2_k_quant_offset,
    q2_k_scale_offset,
    q3_k_bytes,
    q3_k_high_offset,
    q3_k_low_offset,
    q3_k_scale_offset,
    q4_k_bytes,
    q6_k_bytes,
    q6_k_high_offset,
    q6_k_low_offset,
    q6_k_scale_offset,
    q4_k_header_bytes,
    q8_0_bytes,
    q8_0_quant_offset,
    quantize_q8_0,
    tensor_bytes,
)
from .verify import ACCEPT_WORKLOADS, VerifyBatch, draw_verify_batch  # noqa: F401,E402
