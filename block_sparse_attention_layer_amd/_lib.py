"""ctypes view of libvmoba.so (the C ABI in include/vmoba.h).

Loading fails loudly when the library has not been built: there is no other
implementation of these calls in this package.
"""

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libvmoba.so")

VMOBA_OK = 0
STATUS_NAMES = {
    0: "VMOBA_OK", 1: "VMOBA_ERR_NULL", 2: "VMOBA_ERR_SHAPE", 3: "VMOBA_ERR_MODE",
    4: "VMOBA_ERR_TAU", 5: "VMOBA_ERR_DTYPE", 6: "VMOBA_ERR_HEAD_DIM",
    7: "VMOBA_ERR_WORKSPACE", 8: "VMOBA_ERR_OVERFLOW", 9: "VMOBA_ERR_HIP",
    10: "VMOBA_ERR_OP", 11: "VMOBA_ERR_SELECT", 12: "VMOBA_ERR_SCRATCH",
}
NOALLOC_SCRATCH_BYTES = 16 << 20   # VMOBA_NOALLOC_SCRATCH_BYTES
VMOBA_BF16, VMOBA_FP32 = 0, 1
OPS = {"pool": 0, "select": 1, "sparse_fwd": 2, "sparse_bwd": 3, "dense_fwd": 4,
       "dense_bwd": 5, "select_tokens": 6, "token_fwd": 7, "token_bwd": 8}


class CProblem(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "batch", "heads", "head_dim", "T", "H", "W", "layer_idx", "bt", "bh", "bw",
        "dtype", "grad_dtype")]


_P = ctypes.c_void_p
_I32P = ctypes.POINTER(ctypes.c_int32)
_SIG = {
    "vmoba_version": (ctypes.c_char_p, []),
    "vmoba_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "vmoba_validate": (ctypes.c_int, [ctypes.POINTER(CProblem)]),
    "vmoba_num_blocks": (ctypes.c_int, [ctypes.POINTER(CProblem), _I32P]),
    "vmoba_workspace_size": (ctypes.c_int, [ctypes.POINTER(CProblem), ctypes.c_int,
                                            ctypes.POINTER(ctypes.c_size_t)]),
    "vmoba_partition_pool": (ctypes.c_int, [ctypes.POINTER(CProblem), _P, _P, _P, _P, _P]),
    "vmoba_select": (ctypes.c_int, [ctypes.POINTER(CProblem), _P, _P, ctypes.c_float, _P, _P,
                                    _P, _P, _P, _P, _P, ctypes.c_size_t, _P]),
    "vmoba_select_mode": (ctypes.c_int, [ctypes.POINTER(CProblem), _P, _P, ctypes.c_int,
                                         ctypes.c_float, ctypes.c_int32, _P, _P, _P, _P, _P,
                                         _P, _P, ctypes.c_size_t, _P]),
    "vmoba_sparse_attn_fwd": (ctypes.c_int, [ctypes.POINTER(CProblem), _P, _P, _P, _P, _P,
                                             _P, _P, _P, ctypes.c_size_t, _P]),
    "vmoba_sparse_attn_bwd": (ctypes.c_int, [ctypes.POINTER(CProblem)] + [_P] * 14 +
                              [ctypes.c_size_t, _P]),
    "vmoba_sparse_attn_bwd_noalloc": (ctypes.c_int, [ctypes.POINTER(CProblem)] + [_P] * 14),
    "vmoba_sparse_attn_bwd_delta": (ctypes.c_int, [ctypes.POINTER(CProblem), _P, _P, _P, _P]),
    "vmoba_sparse_attn_bwd_dkdv": (ctypes.c_int, [ctypes.POINTER(CProblem)] + [_P] * 11),
    "vmoba_sparse_attn_bwd_dq": (ctypes.c_int, [ctypes.POINTER(CProblem)] + [_P] * 10),
    "vmoba_dense_attn_fwd": (ctypes.c_int, [ctypes.POINTER(CProblem), _P, _P, _P, _P, _P, _P,
                                            ctypes.c_size_t, _P]),
    "vmoba_dense_attn_bwd": (ctypes.c_int, [ctypes.POINTER(CProblem)] + [_P] * 10 +
                             [ctypes.c_size_t, _P]),
    "vmoba_select_tokens": (ctypes.c_int, [ctypes.POINTER(CProblem), _P, _P, ctypes.c_float] +
                            [_P] * 7 + [ctypes.c_size_t, _P]),
    "vmoba_token_attn_fwd": (ctypes.c_int, [ctypes.POINTER(CProblem)] + [_P] * 9 +
                             [ctypes.c_size_t, _P]),
    "vmoba_token_attn_bwd": (ctypes.c_int, [ctypes.POINTER(CProblem)] + [_P] * 15 +
                             [ctypes.c_size_t, _P]),
}

_lib = None


def lib():
    """The loaded library (loaded on first use)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(
                f"{LIB_PATH} is missing: build it with "
                "`python -m block_sparse_attention_layer_amd.build`")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIG.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


class VMoBAError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        msg = lib().vmoba_status_string(status).decode()
        super().__init__(f"{where}: {STATUS_NAMES.get(status, status)} ({msg})")


def check(status, where):
    if status != VMOBA_OK:
        raise VMoBAError(status, where)
