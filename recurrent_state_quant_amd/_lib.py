"""ctypes loader for libleapquant.so (the C ABI in include/leapquant.h).

Loading fails loudly when the library has not been built: there is no
fallback implementation.
"""
import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libleapquant.so")

ABI_VERSION = 6  # the lq_params / lq_state layout and entry points this binding mirrors

LQ_OK = 0
LQ_ERR_NULL = -1
LQ_ERR_SHAPE = -2
LQ_ERR_UNSUPPORTED = -3
LQ_ERR_ALIGN = -4
LQ_ERR_ALIAS = -5
LQ_ERR_HIP = -6

LQ_GATE_GDN = 0
LQ_GATE_KDA = 1
LQ_NO_SMOOTH = 1
LQ_NO_DELTA = 2
LQ_DENSE_COMP = 4
LQ_DENSE_FP32 = 0
LQ_DENSE_BF16 = 1

EXPORTED = (
    "leapquant_quantize_state",
    "leapquant_decode_step",
    "leapquant_window_close",
    "leapquant_decode_close",
    "leapquant_dense_step",
    "leapquant_decode_step_slots",
    "leapquant_decode_close_slots",
    "leapquant_window_close_slots",
    "leapquant_decode_close_list",
    "leapquant_window_close_list",
    "leapquant_decode_step_close_list",
    "leapquant_dequantize_state",
    "leapquant_bf16w_decode_step",
    "leapquant_bf16w_window_close",
    "leapquant_stream_reference",
    "leapquant_status_string",
    "leapquant_abi_version",
)


class LqParams(ctypes.Structure):
    _fields_ = [("n", ctypes.c_int32), ("dk", ctypes.c_int32), ("dv", ctypes.c_int32),
                ("p", ctypes.c_int32), ("r", ctypes.c_int32), ("gate", ctypes.c_int32),
                ("flags", ctypes.c_uint32), ("comp_iters", ctypes.c_int32)]


class LqState(ctypes.Structure):
    _fields_ = [("codes", ctypes.c_void_p), ("row_scale", ctypes.c_void_p),
                ("col_scale", ctypes.c_void_p), ("comp_idx", ctypes.c_void_p),
                ("comp_val", ctypes.c_void_p), ("buf_gate", ctypes.c_void_p),
                ("buf_k", ctypes.c_void_p), ("buf_u", ctypes.c_void_p),
                ("comp_key", ctypes.c_void_p)]


class LeapQuantError(RuntimeError):
    def __init__(self, status, message):
        super().__init__(f"leapquant error {status}: {message}")
        self.status = status


_lib = None


def load():
    """Return the loaded library, loading it on first use."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is not built; build it with recurrent_state_quant_amd.build.build()")
    lib = ctypes.CDLL(LIB_PATH)
    P, S, vp, i32 = ctypes.POINTER(LqParams), ctypes.POINTER(LqState), ctypes.c_void_p, ctypes.c_int32
    lib.leapquant_quantize_state.argtypes = [P, vp, S, vp]
    lib.leapquant_decode_step.argtypes = [P, S, i32, vp, vp, vp, vp, vp, vp, vp]
    lib.leapquant_window_close.argtypes = [P, S, i32, vp]
    lib.leapquant_decode_close.argtypes = [P, S, i32, vp, vp, vp, vp, vp, vp, vp]
    lib.leapquant_dense_step.argtypes = [P, vp, i32, vp, vp, vp, vp, vp, vp, vp]
    lib.leapquant_decode_step_slots.argtypes = [P, S, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.leapquant_decode_close_slots.argtypes = [P, S, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.leapquant_window_close_slots.argtypes = [P, S, vp, vp]
    lib.leapquant_decode_close_list.argtypes = [P, S, vp, vp, i32, vp, vp, vp, vp, vp, vp, vp]
    lib.leapquant_window_close_list.argtypes = [P, S, vp, vp, i32, vp]
    lib.leapquant_decode_step_close_list.argtypes = [P, S, vp, vp, i32, vp, vp, vp, vp, vp, vp, vp]
    lib.leapquant_dequantize_state.argtypes = [P, S, vp, vp]
    lib.leapquant_bf16w_decode_step.argtypes = [P, vp, S, i32, vp, vp, vp, vp, vp, vp, vp]
    lib.leapquant_bf16w_window_close.argtypes = [P, vp, S, i32, vp]
    lib.leapquant_stream_reference.argtypes = [vp, ctypes.c_int64, vp, ctypes.c_int64, i32, i32, vp, vp]
    for f in ("leapquant_quantize_state", "leapquant_decode_step", "leapquant_window_close",
              "leapquant_decode_close", "leapquant_dense_step", "leapquant_decode_step_slots",
              "leapquant_decode_close_slots", "leapquant_window_close_slots",
              "leapquant_decode_close_list", "leapquant_window_close_list", "leapquant_decode_step_close_list",
              "leapquant_dequantize_state", "leapquant_bf16w_decode_step",
              "leapquant_bf16w_window_close", "leapquant_stream_reference"):
        getattr(lib, f).restype = ctypes.c_int
    lib.leapquant_status_string.argtypes = [ctypes.c_int]
    lib.leapquant_status_string.restype = ctypes.c_char_p
    lib.leapquant_abi_version.argtypes = []
    lib.leapquant_abi_version.restype = ctypes.c_int
    if lib.leapquant_abi_version() != ABI_VERSION:
        raise ImportError(f"{LIB_PATH} has ABI version {lib.leapquant_abi_version()}, "
                          f"this binding needs {ABI_VERSION}; rebuild it")
    _lib = lib
    return lib


def check(status):
    if status != LQ_OK:
        raise LeapQuantError(status, load().leapquant_status_string(status).decode())
