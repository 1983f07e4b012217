"""ctypes declarations of the C ABI in include/gdn_cpr.h.

Loading fails loudly (RuntimeError) when the shared library has not been
built: there is no fallback implementation anywhere in this package.
"""

from __future__ import annotations

import ctypes
import os

LIB_NAME = "libgdn_cpr.so"
LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), LIB_NAME)

GDN_OK = 0
GDN_ERR_INVALID_ARG = 1
GDN_ERR_UNSUPPORTED = 2
GDN_ERR_WORKSPACE = 3
GDN_ERR_HIP = 4

GDN_DTYPE_F32 = 0
GDN_DTYPE_BF16 = 1

GDN_OP_PREFILL = 0
GDN_OP_DECODE = 1
GDN_OP_FWD_BWD = 2
GDN_OP_PREFILL_CONTINUE = 3

GDN_CMP_RECURRENT = 0
GDN_CMP_CHUNKWISE = 1

# every symbol the header declares
EXPORTED = (
    "gdn_cpr_workspace_size",
    "gdn_cpr_prefill",
    "gdn_cpr_decode_step",
    "gdn_cpr_decode_step_noalloc",
    "gdn_cpr_prefill_continue",
    "gdn_cpr_fwd_bwd",
    "gdn_cpr_cache_state",
    "gdn_cpr_wait_status",
    "gdn_cpr_debug_set_wait_polls",
    "gdn_cpr_set_stage_events",
    "gdn_cpr_last_error",
    "gdn_cpr_numerics_id",
    "gdn_cmp_workspace_size",
    "gdn_cmp_prefill",
    "gdn_cmp_decode_step",
    "gdn_cmp_chunk_decode_step",
)


class Shape(ctypes.Structure):
    _fields_ = [
        ("num_heads", ctypes.c_int32),
        ("head_dim_k", ctypes.c_int32),
        ("head_dim_v", ctypes.c_int32),
        ("chunk", ctypes.c_int32),
        ("dtype", ctypes.c_int32),
        ("num_key_heads", ctypes.c_int32),
    ]


class Cache(ctypes.Structure):
    _fields_ = [
        ("s_bnd", ctypes.c_void_p),
        ("s_run", ctypes.c_void_p),
        ("tail_k", ctypes.c_void_p),
        ("tail_v", ctypes.c_void_p),
        ("tail_g", ctypes.c_void_p),
        ("tail_beta", ctypes.c_void_p),
        ("tail_len", ctypes.c_void_p),
        ("slot_index", ctypes.c_void_p),
        ("run_log_scale", ctypes.c_void_p),
    ]


_vp = ctypes.c_void_p
_lib = None


def load() -> ctypes.CDLL:
    """The loaded library (RuntimeError if it is not built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"{LIB_NAME} is not built (expected at {LIB_PATH}); run python -m bitwise_invariant_gated_amd.build")
    lib = ctypes.CDLL(LIB_PATH)
    lib.gdn_cpr_workspace_size.restype = ctypes.c_size_t
    lib.gdn_cpr_workspace_size.argtypes = [ctypes.POINTER(Shape), ctypes.c_int32, ctypes.c_int64,
                                           ctypes.c_int32]
    lib.gdn_cpr_prefill.restype = ctypes.c_int
    lib.gdn_cpr_prefill.argtypes = [ctypes.POINTER(Shape), ctypes.c_int32, ctypes.c_int64,
                                    _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, ctypes.POINTER(Cache), _vp,
                                    _vp, ctypes.c_size_t, _vp]
    lib.gdn_cpr_decode_step.restype = ctypes.c_int
    lib.gdn_cpr_decode_step.argtypes = [ctypes.POINTER(Shape), ctypes.c_int32, _vp, _vp, _vp, _vp,
                                        _vp, ctypes.POINTER(Cache), _vp, _vp, _vp, ctypes.c_size_t, _vp]
    lib.gdn_cpr_decode_step_noalloc.restype = ctypes.c_int
    lib.gdn_cpr_decode_step_noalloc.argtypes = [ctypes.POINTER(Shape), ctypes.c_int32, _vp, _vp, _vp, _vp,
                                                _vp, ctypes.POINTER(Cache), _vp, _vp, _vp]
    lib.gdn_cpr_prefill_continue.restype = ctypes.c_int
    lib.gdn_cpr_prefill_continue.argtypes = [ctypes.POINTER(Shape), ctypes.c_int32, ctypes.c_int64,
                                             _vp, _vp, _vp, _vp, _vp, _vp, ctypes.POINTER(Cache), _vp, _vp,
                                             _vp, ctypes.c_size_t, _vp]
    lib.gdn_cpr_fwd_bwd.restype = ctypes.c_int
    lib.gdn_cpr_fwd_bwd.argtypes = [ctypes.POINTER(Shape), ctypes.c_int32, ctypes.c_int64,
                                    _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                    _vp, _vp, _vp, _vp, _vp, _vp, ctypes.c_size_t, _vp]
    lib.gdn_cpr_debug_set_wait_polls.restype = ctypes.c_int
    lib.gdn_cpr_debug_set_wait_polls.argtypes = [ctypes.c_int32]
    lib.gdn_cpr_wait_status.restype = ctypes.c_int
    lib.gdn_cpr_wait_status.argtypes = [ctypes.POINTER(Shape), ctypes.c_int32, ctypes.c_int64, _vp,
                                        ctypes.c_size_t, _vp, _vp]
    lib.gdn_cpr_cache_state.restype = ctypes.c_int
    lib.gdn_cpr_cache_state.argtypes = [ctypes.POINTER(Shape), ctypes.c_int32, ctypes.POINTER(Cache), _vp, _vp]
    lib.gdn_cmp_workspace_size.restype = ctypes.c_size_t
    lib.gdn_cmp_workspace_size.argtypes = [ctypes.POINTER(Shape), ctypes.c_int32, ctypes.c_int32, ctypes.c_int64]
    lib.gdn_cmp_prefill.restype = ctypes.c_int
    lib.gdn_cmp_prefill.argtypes = [ctypes.POINTER(Shape), ctypes.c_int32, ctypes.c_int32, ctypes.c_int64,
                                    _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, ctypes.c_size_t, _vp]
    lib.gdn_cmp_decode_step.restype = ctypes.c_int
    lib.gdn_cmp_decode_step.argtypes = [ctypes.POINTER(Shape), ctypes.c_int32, _vp, _vp, _vp, _vp, _vp, _vp,
                                        _vp, _vp]
    lib.gdn_cmp_chunk_decode_step.restype = ctypes.c_int
    lib.gdn_cmp_chunk_decode_step.argtypes = [ctypes.POINTER(Shape), ctypes.c_int32, _vp, _vp, _vp, _vp,
                                              _vp, ctypes.POINTER(Cache), _vp, _vp, ctypes.c_size_t, _vp]
    lib.gdn_cpr_set_stage_events.restype = None
    lib.gdn_cpr_set_stage_events.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_int32]
    lib.gdn_cpr_last_error.restype = ctypes.c_char_p
    lib.gdn_cpr_last_error.argtypes = []
    lib.gdn_cpr_numerics_id.restype = ctypes.c_char_p
    lib.gdn_cpr_numerics_id.argtypes = []
    _lib = lib
    return lib


class GdnError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"status {status}: {message}")
        self.status = status


def check(status: int) -> None:
    if status != GDN_OK:
        raise GdnError(status, load().gdn_cpr_last_error().decode())
