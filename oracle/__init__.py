"""CPU oracle for INT8-QK / BF16-PV flash attention (forward only).

TEST INFRASTRUCTURE. Only tests/, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package. The product
library never imports, links or runs anything under ``oracle/``.

This module is argument marshalling around ``oracle.c`` (plain C, fp64 from
the logits on; see the header of that file for the steps, the sources they
follow and the readings taken where the pages are silent). Its no-quant mode
(``attn`` with ``q``/``k`` instead of codes) is textbook fp64 attention; the
tests pin it against torch's fp64 scaled_dot_product_attention and logsumexp.

Array conventions: numpy arrays, C-contiguous after ``np.ascontiguousarray``.
bf16 tensors are carried as ``np.uint16`` arrays holding the raw bf16 bits;
``np.float16`` is fp16; ``np.float32`` is fp32.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
# QFA_ORACLE_LIB names another build of oracle.c (the sanitizer test loads one built with ASan/UBSan)
_LIB = os.environ.get("QFA_ORACLE_LIB") or os.path.join(_HERE, "liboracle.so")

BF16, FP16, FP32 = 1, 2, 3

_lib = None


def build(force: bool = True) -> str:
    """Compile ``oracle.c`` into ``liboracle.so`` with gcc (IEEE fp, no contraction)."""
    global _lib
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        cmd = ["gcc", "-O2", "-std=gnu11", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
               "-fPIC", "-shared", "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
        _lib = None
    return _LIB


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=True)
        _lib = ctypes.CDLL(_LIB)
        _declare(_lib)
    return _lib


_P = ctypes.c_void_p
_I64 = ctypes.c_int64


def _declare(L):
    L.oracle_kmean.argtypes = [_P, ctypes.c_int, _I64, _I64, _I64, _I64, _P, _P]
    L.oracle_quantize_rows.argtypes = [_P, ctypes.c_int, _I64, _I64, _I64, _I64, _P, _P, _P, _P]
    L.oracle_qmu.argtypes = [_P, ctypes.c_int, _I64, _I64, _I64, _I64, _I64, _P, _P, _P]
    L.oracle_scores_i32.argtypes = [_P, _P, _I64, _I64, _I64, _P]
    L.oracle_attn.argtypes = ([_I64] * 6 + [_P] * 6 + [_P, ctypes.c_int, ctypes.c_float]
                              + [_P, ctypes.c_int, _I64, _I64, _I64, _I64]
                              + [_P, _P, _P, ctypes.c_int, _P, _P, ctypes.c_int, _P, _I64, _P, _P])
    L.oracle_lse_merge.argtypes = [_P, _P, _P, _P, _I64, _I64, _P, _P]
    L.oracle_blockmask_to_index.argtypes = [_P, _I64, _I64, _P, _P]
    for f in (L.oracle_kmean, L.oracle_quantize_rows, L.oracle_qmu, L.oracle_scores_i32,
              L.oracle_attn, L.oracle_lse_merge, L.oracle_blockmask_to_index):
        f.restype = None


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def dtype_code(a: np.ndarray) -> int:
    if a.dtype == np.uint16:
        return BF16
    if a.dtype == np.float16:
        return FP16
    if a.dtype == np.float32:
        return FP32
    raise TypeError(f"unsupported element type {a.dtype}")


def _c(a, dt=None):
    if a is None:
        return None
    return np.ascontiguousarray(a if dt is None else a.astype(dt, copy=False))


def kmean(k: np.ndarray, vbs: np.ndarray | None = None) -> np.ndarray:
    """Mean of K over the (valid) sequence: [B,H,S,D] -> [B,H,D] fp32."""
    k = _c(k)
    B, H, S, D = k.shape
    vbs = _c(vbs, np.int32)
    out = np.empty((B, H, D), np.float32)
    lib().oracle_kmean(_ptr(k), dtype_code(k), B, H, S, D, _ptr(vbs), _ptr(out))
    return out


def quantize_rows(x: np.ndarray, mean: np.ndarray | None = None, vbs: np.ndarray | None = None):
    """Per-token symmetric int8 of x (minus mean when given): -> (int8 [B,H,S,D], fp32 [B,H,S])."""
    x = _c(x)
    B, H, S, D = x.shape
    mean = _c(mean, np.float32)
    vbs = _c(vbs, np.int32)
    q = np.empty((B, H, S, D), np.int8)
    s = np.empty((B, H, S), np.float32)
    lib().oracle_quantize_rows(_ptr(x), dtype_code(x), B, H, S, D, _ptr(mean), _ptr(vbs), _ptr(q), _ptr(s))
    return q, s


def _kv_heads(H: int, Hkv: int) -> int:
    if Hkv < 1 or H % Hkv:
        raise ValueError(f"{H} query heads cannot share {Hkv} K/V heads")
    return Hkv


def qmu(q: np.ndarray, mean: np.ndarray, vbs: np.ndarray | None = None) -> np.ndarray:
    """Centring term sum_c Q_ic * mu_c in fp64: -> [B,H,S]. ``mean`` is [B,Hkv,D]; query
    head h uses the mean of K/V head h // (H // Hkv)."""
    q = _c(q)
    B, H, S, D = q.shape
    mean = _c(mean, np.float32)
    Hkv = _kv_heads(H, mean.shape[1])
    vbs = _c(vbs, np.int32)
    out = np.empty((B, H, S), np.float64)
    lib().oracle_qmu(_ptr(q), dtype_code(q), B, H, Hkv, S, D, _ptr(mean), _ptr(vbs), _ptr(out))
    return out


def quantize_qk(q: np.ndarray, k: np.ndarray, vbs: np.ndarray | None = None, center_k: bool = True) -> dict:
    """The whole quantize step: K mean, Q and centred-K int8 + scales, centring term.
    K may hold fewer heads than Q (grouped-query attention, reading R8 of oracle.c)."""
    mu = kmean(k, vbs) if center_k else None
    q8, qs = quantize_rows(q, None, vbs)
    k8, ks = quantize_rows(k, mu, vbs)
    out = dict(q8=q8, qs=qs, k8=k8, ks=ks, kmean=mu)
    out["qmu"] = qmu(q, mu, vbs) if center_k else None
    return out


def scores_i32(q8: np.ndarray, k8: np.ndarray) -> np.ndarray:
    """int32 S = Q8 K8^T for one head: [Sq,D] x [Sk,D] -> [Sq,Sk]."""
    q8 = _c(q8, np.int8)
    k8 = _c(k8, np.int8)
    Sq, D = q8.shape
    Sk = k8.shape[0]
    s = np.empty((Sq, Sk), np.int32)
    lib().oracle_scores_i32(_ptr(q8), _ptr(k8), Sq, Sk, D, _ptr(s))
    return s


def _bias_args(bias, B, H, Sq, Sk):
    if bias is None:
        return None, None, FP32, 0, 0, 0, 0
    # keep the caller's broadcast strides (stride 0 on broadcast dims)
    b4 = np.broadcast_to(bias, (B, H, Sq, Sk)) if bias.ndim == 4 else None
    if b4 is None:
        raise ValueError("bias must be 4-D [B|1,H|1,Q|1,K]")
    st = [s // b4.itemsize for s in b4.strides]
    base = np.asarray(bias)
    return base, b4, dtype_code(b4), st[0], st[1], st[2], st[3]


def attn(qk: dict | None, v: np.ndarray, sm_scale: float, *, q: np.ndarray | None = None,
         k: np.ndarray | None = None, bias: np.ndarray | None = None, mask: np.ndarray | None = None,
         vbs: np.ndarray | None = None, v_scale: np.ndarray | None = None, segments=None,
         rows: np.ndarray | None = None, use_qmu: bool = True, causal: bool = False):
    """Attention in fp64 for all rows (or the flat [B,H,Sq] row indices in ``rows``).

    Quantized mode: ``qk`` is the dict from :func:`quantize_qk` (or the same
    fields from any source). No-quant mode: ``qk`` is None and raw ``q``/``k``
    (any float arrays) are used in fp64. ``causal`` (self-attention, Sq == Sk)
    excludes every key j > i from row i. K, V (and ``v_scale`` [Hkv, D]) may hold
    Hkv heads, a divisor of Q's H: query head h reads K/V head h // (H // Hkv).
    Returns (O [nrows, D] f64, LSE [nrows] f64).
    """
    v = _c(v)
    B, Hkv, Sk, D = v.shape
    if qk is not None:
        q8 = _c(qk["q8"], np.int8)
        Sq = q8.shape[2]
        qs, k8, ks = _c(qk["qs"], np.float32), _c(qk["k8"], np.int8), _c(qk["ks"], np.float32)
        qf = kf = None
        qm = _c(qk.get("qmu"), np.float64) if use_qmu else None
    else:
        qf, kf = _c(q, np.float64), _c(k, np.float64)
        Sq = qf.shape[2]
        q8 = qs = k8 = ks = None
        qm = None
    H = (q8 if q8 is not None else qf).shape[1]
    _kv_heads(H, Hkv)
    if causal and Sq != Sk:
        raise ValueError("causal attention is defined here for self-attention (Sq == Sk)")
    base, b4, bdt, bsb, bsh, bsq, bsk = _bias_args(bias, B, H, Sq, Sk)
    mask = _c(mask, np.uint8)
    vbs = _c(vbs, np.int32)
    v_scale = _c(v_scale, np.float32)
    seg = None
    nseg = 0
    if segments is not None:
        seg = np.ascontiguousarray(np.array(segments, np.int64).reshape(-1))
        nseg = len(seg) // 2
    if rows is not None:
        rows = np.ascontiguousarray(rows, np.int64)
        nrows = len(rows)
    else:
        nrows = B * H * Sq
    o = np.empty((nrows, D), np.float64)
    lse = np.empty(nrows, np.float64)
    # the bias pointer is the first element of the broadcast view (strides may be 0)
    bptr = None if b4 is None else ctypes.c_void_p(b4.__array_interface__["data"][0])
    lib().oracle_attn(B, H, Hkv, Sq, Sk, D, _ptr(q8), _ptr(qs), _ptr(k8), _ptr(ks), _ptr(qf), _ptr(kf),
                      _ptr(v), dtype_code(v), float(sm_scale), bptr, bdt, bsb, bsh, bsq, bsk,
                      _ptr(mask), _ptr(vbs), _ptr(v_scale), nseg, _ptr(seg), _ptr(qm), int(bool(causal)),
                      _ptr(rows), nrows, _ptr(o), _ptr(lse))
    del base
    return o, lse


def lse_merge(oa, la, ob, lb):
    """Exact merge of two partial softmaxes: -> (O f64 [N,D], LSE f64 [N])."""
    oa = _c(oa, np.float64)
    ob = _c(ob, np.float64)
    la = _c(la, np.float64).reshape(-1)
    lb = _c(lb, np.float64).reshape(-1)
    D = oa.shape[-1]
    N = la.size
    o = np.empty((N, D), np.float64)
    l = np.empty(N, np.float64)
    lib().oracle_lse_merge(_ptr(oa), _ptr(la), _ptr(ob), _ptr(lb), N, D, _ptr(o), _ptr(l))
    return o, l


def blockmask_to_index(mask: np.ndarray):
    """[B,H,Tq,Tk] bool/uint8 -> (index int32 [B,H,Tq,Tk] (tail entries -1), count int32 [B,H,Tq])."""
    m = _c(mask, np.uint8)
    B, H, Tq, Tk = m.shape
    index = np.full((B, H, Tq, Tk), -1, np.int32)
    count = np.empty((B, H, Tq), np.int32)
    lib().oracle_blockmask_to_index(_ptr(m), B * H * Tq, Tk, _ptr(index), _ptr(count))
    return index, count
