"""ctypes loader for libattn_mi355x.so (argument marshalling only).

There is no fallback: if the HIP library is not built, or cannot be loaded,
importing the binding's compute entry points raises.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libattn_mi355x.so")

# Status codes, mirroring include/attn.h.
ATTN_OK = 0
ATTN_ERR_NULL_PTR = 1
ATTN_ERR_BAD_SHAPE = 2
ATTN_ERR_UNSUPPORTED_HEAD_DIM = 3
ATTN_ERR_BAD_SCALE = 4
ATTN_ERR_MISALIGNED = 5
ATTN_ERR_ALIAS = 6
ATTN_ERR_WORKSPACE = 7
ATTN_ERR_HIP = 8
ATTN_ERR_TOO_LARGE = 9
ATTN_ERR_BAD_STRIDE = 10
ATTN_ERR_BAD_MASK = 11
ATTN_ERR_SCRATCH_TOO_SMALL = 12

ATTN_NOALLOC_SCRATCH_BYTES = 128 << 20

ATTN_MASK_NONE = 0
ATTN_MASK_CAUSAL = 1
ATTN_MASK_COMPRESSED_CAUSAL = 2

ATTN_PATH_NONE = -1
ATTN_PATH_ONLINE = 0
ATTN_PATH_TWO_PASS = 1

KERNEL_NAMES = ("online", "scores", "values", "values_reduce", "online_combine")

# Every symbol include/attn.h declares, with its ctypes signature.
SIGNATURES = {
    "attn_forward": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                    ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                                    ctypes.c_float, ctypes.c_int, ctypes.c_void_p]),
    "attn_forward_noalloc": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                            ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64,
                                            ctypes.c_int64, ctypes.c_int64, ctypes.c_float,
                                            ctypes.c_int, ctypes.c_void_p]),
    "attn_forward_ex": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                       ctypes.c_void_p, ctypes.c_void_p,
                                       ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                                       ctypes.c_int64, ctypes.c_int64,
                                       ctypes.POINTER(ctypes.c_int64), ctypes.POINTER(ctypes.c_int64),
                                       ctypes.POINTER(ctypes.c_int64), ctypes.POINTER(ctypes.c_int64),
                                       ctypes.c_float, ctypes.c_int, ctypes.c_int64, ctypes.c_int64,
                                       ctypes.c_void_p]),
    "attn_forward_varlen": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                           ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                           ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                                           ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64,
                                           ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                                           ctypes.POINTER(ctypes.c_int64), ctypes.POINTER(ctypes.c_int64),
                                           ctypes.POINTER(ctypes.c_int64), ctypes.POINTER(ctypes.c_int64),
                                           ctypes.c_float, ctypes.c_int, ctypes.c_int64, ctypes.c_int64,
                                           ctypes.c_void_p]),
    "attn_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "attn_path_for_head_dim": (ctypes.c_int, [ctypes.c_int64]),
    "attn_workspace_bytes": (ctypes.c_int64, [ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                                              ctypes.c_int64, ctypes.c_int]),
    "attn_timing_enable": (ctypes.c_int, [ctypes.c_int]),
    "attn_timing_collect": (ctypes.c_int, [ctypes.POINTER(ctypes.c_double),
                                           ctypes.POINTER(ctypes.c_int64), ctypes.c_int]),
}

_lib = None


class AttnError(RuntimeError):
    def __init__(self, status: int, where: str = "attn_forward"):
        self.status = status
        super().__init__(f"{where}: {status_string(status)} (status {status})")


def load() -> ctypes.CDLL:
    """Load the in-tree HIP library once; raise if it is not built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"HIP library not built: {LIB_PATH} is missing. Build it with "
            "`python -c 'import __graft_entry__ as g; g.build()'` or "
            "`python exact_softmax_attention_bf16_amd/build.py`.")
    lib = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def status_string(status: int) -> str:
    return load().attn_status_string(int(status)).decode()
