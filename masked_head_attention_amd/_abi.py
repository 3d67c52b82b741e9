"""ctypes view of libmha's C ABI (include/mha.h). No torch, no computation.

The library is built in-tree (``libmha.so`` next to this file). If it is
missing, loading raises: there is no fallback path of any kind.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmha.so")

F32, F16, BF16 = 0, 1, 2
MASK_NONE, CAUSAL, PADDING, ADDITIVE, KEEP, PER_HEAD = 0, 1, 2, 4, 8, 16
FLAG_FULLY_MASKED_ROW, FLAG_NONFINITE, FLAG_BAD_LENGTH = 1, 2, 4
STATUS = {0: "MHA_OK", 1: "MHA_E_NULL", 2: "MHA_E_SHAPE", 3: "MHA_E_DTYPE", 4: "MHA_E_MASK",
          5: "MHA_E_UNSUPPORTED", 6: "MHA_E_ALIGN", 7: "MHA_E_OVERFLOW", 8: "MHA_E_NO_DEVICE",
          9: "MHA_E_LAUNCH", 10: "MHA_E_ARG", 11: "MHA_E_WORKSPACE", 12: "MHA_E_NOT_INITIALIZED",
          13: "MHA_E_SCRATCH"}
STATUS_CODE = {v: k for k, v in STATUS.items()}

_vp, _i, _u, _f = ctypes.c_void_p, ctypes.c_int, ctypes.c_uint, ctypes.c_float
SIGNATURES = {
    "mha_init": ([], _i),
    "mha_fwd": ([_vp, _vp, _vp, _vp, _u, _i, _i, _i, _i, _i, _f, _i, _vp, _vp], _i),
    "mha_prenorm_cross_fwd": ([_vp, _vp, _vp, _vp, _u, _vp, _vp, _f, _vp, _i, _i, _i, _i, _i, _f,
                               _i, _vp, _vp], _i),
    "mha_prenorm_cross_fwd_ws": ([_vp, _vp, _vp, _vp, _u, _vp, _vp, _f, _vp, _i, _i, _i, _i, _i,
                                  _f, _i, _vp, ctypes.c_size_t, _vp, _vp], _i),
    "mha_prenorm_cross_workspace_size": ([_i, _i, _i, _i, _i, _i, ctypes.POINTER(ctypes.c_size_t)],
                                         _i),
    "mha_get_flags": ([_vp, ctypes.POINTER(ctypes.c_uint32), _i], _i),
    "mha_set_debug_counters": ([_vp], _i),
    "mha_tile_config": ([_i, _i, _u, ctypes.POINTER(_i), ctypes.POINTER(_i)], _i),
    "mha_status_str": ([_i], ctypes.c_char_p),
    "mha_softmax_rows": ([_vp, _vp, ctypes.c_int64, _i, _f, _i, _vp], _i),
    "mha_decode_fwd": ([_vp, _vp, _vp, _vp, _i, _i, _i, _i, _f, _i, _vp, ctypes.c_size_t, _vp,
                        _vp, _vp], _i),
    "mha_decode_workspace_size": ([_i, _i, _i, _i, _i, ctypes.POINTER(ctypes.c_size_t)], _i),
    "mha_decode_fwd_noalloc": ([_vp, _vp, _vp, _vp, _i, _i, _i, _i, _f, _i, _vp, _vp, _vp], _i),
    "mha_noalloc_scratch_bytes": ([ctypes.POINTER(ctypes.c_size_t)], _i),
    "mha_bwd": ([_vp, _vp, _vp, _vp, _vp, _u, _i, _i, _i, _i, _i, _f, _i, _vp, ctypes.c_size_t,
                 _vp, _vp, _vp, _vp], _i),
    "mha_bwd_workspace_size": ([_i, _i, _i, _i, ctypes.POINTER(ctypes.c_size_t)], _i),
}

_lib = None


class MhaError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {STATUS.get(status, status)}")


def lib() -> ctypes.CDLL:
    """Load libmha.so (once). Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(
                f"{LIB_PATH} is missing: build it first (python -m masked_head_attention_amd.build "
                "or __graft_entry__.build())")
        l = ctypes.CDLL(LIB_PATH)
        for name, (args, res) in SIGNATURES.items():
            fn = getattr(l, name)
            fn.argtypes = args
            fn.restype = res
        _lib = l
    return _lib


def check(status: int, where: str) -> None:
    if status != 0:
        raise MhaError(status, where)
