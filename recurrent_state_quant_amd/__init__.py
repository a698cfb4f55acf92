"""LeapQuant decode hot path for AMD Instinct MI355X (gfx950).

Per-window int8 recurrent-state decode for Gated DeltaNet and Kimi Delta
Attention layers, with fp32 compensator rows and per-column residual
smoothing, as hand-written HIP kernels behind the C ABI of
include/leapquant.h.  This package is the thin Python binding: it marshals
torch device tensors and streams into the C calls and runs nothing itself.
"""
from ._lib import (LQ_DENSE_BF16, LQ_DENSE_COMP, LQ_DENSE_FP32, LQ_GATE_GDN, LQ_GATE_KDA, LQ_NO_DELTA, LQ_NO_SMOOTH,
                   LeapQuantError, LIB_PATH, load)
from .api import (LeapQuantState, code_offsets, codes_from_matrix, codes_to_matrix,
                  leapquant_abi_version, leapquant_bf16w_decode_step, leapquant_bf16w_window_close,
                  leapquant_decode_close, leapquant_decode_step,
                  leapquant_decode_close_slots, leapquant_decode_step_slots, leapquant_dense_step,
                  leapquant_window_close_slots, leapquant_decode_close_list, leapquant_window_close_list,
                  leapquant_decode_step_close_list, leapquant_dequantize_state, leapquant_quantize_state,
                  leapquant_stream_reference, leapquant_status_string, leapquant_window_close)

__all__ = [
    "LQ_DENSE_BF16", "LQ_DENSE_COMP", "LQ_DENSE_FP32", "LQ_GATE_GDN", "LQ_GATE_KDA", "LQ_NO_DELTA", "LQ_NO_SMOOTH",
    "LeapQuantError", "LIB_PATH", "load",
    "LeapQuantState", "code_offsets", "codes_from_matrix", "codes_to_matrix",
    "leapquant_abi_version", "leapquant_bf16w_decode_step", "leapquant_bf16w_window_close",
    "leapquant_decode_close", "leapquant_decode_step",
    "leapquant_decode_close_slots", "leapquant_decode_step_slots", "leapquant_dense_step",
    "leapquant_window_close_slots", "leapquant_decode_close_list", "leapquant_window_close_list",
    "leapquant_decode_step_close_list", "leapquant_dequantize_state", "leapquant_quantize_state",
    "leapquant_stream_reference", "leapquant_status_string", "leapquant_window_close",
]
