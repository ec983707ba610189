"""ctypes view of libgma.so (declared in include/gma.h).  Argument marshalling only."""
from __future__ import annotations

import ctypes
import os
import threading

from .build import LIB_PATH

GMA_DTYPE_F32 = 0
GMA_DTYPE_BF16 = 1
GMA_OP_RESPONSIBILITIES = 0
GMA_OP_FORWARD_BIDIR = 1
GMA_OP_FORWARD_CAUSAL = 2
GMA_OP_FORWARD_CAUSAL_STATE = 3
GMA_OP_RESPONSIBILITY_STATS = 4
GMA_OP_BACKWARD_BIDIR = 5
GMA_OP_BACKWARD_CAUSAL = 6
NOALLOC_SCRATCH_BYTES = 64 << 20   # GMA_NOALLOC_SCRATCH_BYTES in gma.h
STATUS = {0: "GMA_SUCCESS", 1: "GMA_ERROR_INVALID_VALUE", 2: "GMA_ERROR_NOT_SUPPORTED",
          3: "GMA_ERROR_WORKSPACE_TOO_SMALL", 4: "GMA_ERROR_LAUNCH"}


class Problem(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int64), ("heads", ctypes.c_int64), ("seq_len", ctypes.c_int64),
                ("d_route", ctypes.c_int32), ("n_comp", ctypes.c_int32), ("d_value", ctypes.c_int32),
                ("dtype", ctypes.c_int32), ("eps", ctypes.c_float)]


class GmaError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__("%s: %s" % (STATUS.get(status, status), message))
        self.status = status


_lock = threading.Lock()
_lib = None

# (name, restype, argtypes)
_VP = ctypes.c_void_p
_SIGS = [
    ("gma_workspace_size", ctypes.c_size_t, [ctypes.POINTER(Problem), ctypes.c_int]),
    ("gma_responsibilities", ctypes.c_int, [ctypes.POINTER(Problem), _VP, _VP, _VP, _VP, _VP, _VP, ctypes.c_size_t, _VP]),
    ("gma_forward_bidir", ctypes.c_int, [ctypes.POINTER(Problem), _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, ctypes.c_size_t, _VP]),
    ("gma_forward_causal", ctypes.c_int, [ctypes.POINTER(Problem), _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, ctypes.c_size_t, _VP]),
    ("gma_forward_causal_noalloc", ctypes.c_int, [ctypes.POINTER(Problem), _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP]),
    ("gma_forward_bidir_kv", ctypes.c_int, [ctypes.POINTER(Problem), ctypes.c_int64, _VP, _VP, _VP, _VP, _VP, _VP, _VP,
                                            _VP, ctypes.c_size_t, _VP]),
    ("gma_responsibility_stats", ctypes.c_int, [ctypes.POINTER(Problem), _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP,
                                                ctypes.c_size_t, _VP]),
    ("gma_decode_step", ctypes.c_int, [ctypes.POINTER(Problem), _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP]),
    ("gma_decode_params_size", ctypes.c_size_t, [ctypes.POINTER(Problem)]),
    ("gma_decode_prepare", ctypes.c_int, [ctypes.POINTER(Problem), _VP, _VP, _VP, ctypes.c_size_t, _VP]),
    ("gma_decode_step_prepared", ctypes.c_int, [ctypes.POINTER(Problem), _VP, _VP, _VP, _VP, _VP, ctypes.c_size_t, _VP,
                                                _VP, _VP, _VP]),
    ("gma_forward_causal_state", ctypes.c_int, [ctypes.POINTER(Problem), _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP,
                                                ctypes.c_size_t, _VP]),
    ("gma_backward_bidir", ctypes.c_int, [ctypes.POINTER(Problem)] + [_VP] * 14 + [ctypes.c_size_t, _VP]),
    ("gma_backward_causal", ctypes.c_int, [ctypes.POINTER(Problem)] + [_VP] * 14 + [ctypes.c_size_t, _VP]),
    ("gma_status_string", ctypes.c_char_p, [ctypes.c_int]),
    ("gma_last_error", ctypes.c_char_p, []),
    ("gma_timing_enable", ctypes.c_int, [ctypes.c_int]),
    ("gma_timing_read", ctypes.c_int, [ctypes.c_int, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_int64)]),
    ("gma_kernel_count", ctypes.c_int, []),
    ("gma_kernel_name", ctypes.c_char_p, [ctypes.c_int]),
    ("gma_probe_exp2_rate", ctypes.c_int, [ctypes.POINTER(ctypes.c_double), ctypes.c_void_p]),
    ("gma_probe_read_rate", ctypes.c_int,
     [ctypes.c_void_p, ctypes.c_size_t, ctypes.POINTER(ctypes.c_double), ctypes.c_void_p]),
]


def lib_path() -> str:
    return LIB_PATH


def load():
    """Load libgma.so; raises if it has not been built (the product path has no fallback)."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                raise RuntimeError("libgma.so is not built at %s: run __graft_entry__.build() or "
                                   "python -m gaussian_mixture_token_amd.build" % LIB_PATH)
            lib = ctypes.CDLL(LIB_PATH)
            for name, res, args in _SIGS:
                fn = getattr(lib, name)
                fn.restype = res
                fn.argtypes = args
            _lib = lib
    return _lib


def check(status: int) -> None:
    if status != 0:
        msg = load().gma_last_error().decode(errors="replace")
        raise GmaError(status, msg)
