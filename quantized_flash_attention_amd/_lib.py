"""ctypes view of libqfa.so (the C ABI declared in include/qfa.h).

The library must have been built (``quantized_flash_attention_amd.build`` or
``__graft_entry__.build()``); there is no fallback implementation, so a
missing library raises at first use.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
# QFA_LIB_PATH names another build of the same library (the sanitizer test loads one whose host
# code is built with ASan/UBSan); there is no other implementation to fall back to
LIB_PATH = os.environ.get("QFA_LIB_PATH") or os.path.join(_HERE, "libqfa.so")

QFA_OK, QFA_ERR_INVALID_ARG, QFA_ERR_UNSUPPORTED, QFA_ERR_HIP = 0, 1, 2, 3
QFA_BF16, QFA_FP16, QFA_FP32, QFA_BOOL = 1, 2, 3, 4

EXPORTS = (
    "qfa_version",
    "qfa_status_string",
    "qfa_last_error",
    "qfa_quantize_workspace_bytes",
    "qfa_quantize_qk",
    "qfa_quantize_qk_noalloc",
    "qfa_blockmask_to_index",
    "qfa_attn_fwd",
    "qfa_attn_fwd_splitk",
    "qfa_attn_fwd_unquant",
    "qfa_attn_split_workspace_bytes",
    "qfa_attn_splits_auto",
    "qfa_lse_merge",
    "qfa_qk_scores_i32",
)

_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_I = ctypes.c_int

_lib = None


class QFAError(RuntimeError):
    pass


def _declare(L: ctypes.CDLL) -> None:
    L.qfa_version.argtypes = []
    L.qfa_version.restype = _I
    L.qfa_status_string.argtypes = [_I]
    L.qfa_status_string.restype = ctypes.c_char_p
    L.qfa_last_error.argtypes = []
    L.qfa_last_error.restype = ctypes.c_char_p
    L.qfa_quantize_workspace_bytes.argtypes = [_I64, _I64, _I64, _I64, ctypes.POINTER(ctypes.c_size_t)]
    L.qfa_quantize_workspace_bytes.restype = _I
    L.qfa_quantize_qk.argtypes = ([_I64] * 6 + [_I] + [_P, _I64, _I64, _I64] * 2
                                  + [_P, _I] + [_P] * 6 + [_P, ctypes.c_size_t, _P])
    L.qfa_quantize_qk.restype = _I
    L.qfa_quantize_qk_noalloc.argtypes = L.qfa_quantize_qk.argtypes[:-3] + [_P]
    L.qfa_quantize_qk_noalloc.restype = _I
    L.qfa_blockmask_to_index.argtypes = [_P, _I64, _I64, _I64, _I64, _P, _P, _P]
    L.qfa_blockmask_to_index.restype = _I
    # sm_scale, bias, block-sparse lists, v_scale, segments, causal, out, lse
    masks_out = ([ctypes.c_float] + [_P, _I, _I64, _I64, _I64] + [_P] * 3 + [_P, _I, _P, _I]
                 + [_P, _I, _I64, _I64, _I64] + [_P])
    v_view = [_P, _I, _I64, _I64, _I64]
    # q8, qs, qmu, k8, ks, k_centered
    codes = [_P] * 5 + [_I]
    L.qfa_attn_fwd.argtypes = [_I64] * 6 + codes + v_view + masks_out + [_P]
    L.qfa_attn_fwd.restype = _I
    L.qfa_attn_fwd_splitk.argtypes = [_I64] * 6 + codes + v_view + masks_out + [_I, _P, ctypes.c_size_t, _P]
    L.qfa_attn_fwd_splitk.restype = _I
    L.qfa_attn_fwd_unquant.argtypes = ([_I64] * 6 + [_P, _I64, _I64, _I64] * 2 + v_view + masks_out
                                       + [_I, _P, ctypes.c_size_t, _P])
    L.qfa_attn_fwd_unquant.restype = _I
    L.qfa_attn_split_workspace_bytes.argtypes = [_I64] * 4 + [_I, ctypes.POINTER(ctypes.c_size_t)]
    L.qfa_attn_split_workspace_bytes.restype = _I
    L.qfa_attn_splits_auto.argtypes = [_I64] * 4 + [_I, ctypes.POINTER(_I)]
    L.qfa_attn_splits_auto.restype = _I
    L.qfa_lse_merge.argtypes = ([_I64] * 4 + [_P, _I, _I64, _I64, _I64, _P] * 2
                                + [_P, _I, _I64, _I64, _I64, _P, _P])
    L.qfa_lse_merge.restype = _I
    L.qfa_qk_scores_i32.argtypes = [_I64] * 5 + [_P, _P, _P, _P]
    L.qfa_qk_scores_i32.restype = _I


def lib() -> ctypes.CDLL:
    """Load libqfa.so once; raise if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise QFAError(f"{LIB_PATH} is missing: build it with quantized_flash_attention_amd.build.build()")
        L = ctypes.CDLL(LIB_PATH)
        _declare(L)
        _lib = L
    return _lib


def check(status: int) -> None:
    """Map a status code to an exception carrying the library's detail message."""
    if status == QFA_OK:
        return
    msg = lib().qfa_last_error().decode() or lib().qfa_status_string(status).decode()
    if status == QFA_ERR_INVALID_ARG:
        raise ValueError(msg)
    if status == QFA_ERR_UNSUPPORTED:
        raise NotImplementedError(msg)
    raise QFAError(msg)
