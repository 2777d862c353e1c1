"""INT8-QK / BF16-PV flash attention forward for AMD Instinct MI355X (gfx950).

Thin PyTorch binding of libqfa.so: every function below marshals tensors
into the C ABI of include/qfa.h (pointers, sizes, strides and the current
HIP stream) and allocates outputs with torch when the caller passes none.
All arithmetic runs in the library's HIP kernels; there is no fallback path.

Functions (same names as the C entry points without the ``qfa_`` prefix):
  quantize_qk(q, k, vbs=None, center_k=True)      -> dict of int8 codes and scales
  blockmask_to_index(mask)                         -> (index, count)
  attn_fwd(qk, v, ...)                             -> out or (out, lse)
  lse_merge(o_a, lse_a, o_b, lse_b)                -> (out, lse)
  qk_scores_i32(q8, k8)                            -> int32 scores of the attention kernel's QK stage
plus ``int8_attention``, the quantize + attend convenience call.
"""
from __future__ import annotations

import ctypes
import math

import torch

from . import _lib
from ._lib import QFA_BF16, QFA_BOOL, QFA_FP16, QFA_FP32, QFAError

__all__ = ["quantize_qk", "quantize_qk_noalloc", "blockmask_to_index", "attn_fwd", "lse_merge", "int8_attention", "QFAError",
           "quantize_workspace_bytes", "qk_scores_i32", "split_workspace_bytes", "splits_auto", "attn_fwd_unquant"]

_DT = {torch.bfloat16: QFA_BF16, torch.float16: QFA_FP16, torch.float32: QFA_FP32}


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(dev: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def _view(t: torch.Tensor, name: str):
    if t.dim() != 4:
        raise ValueError(f"{name} must be 4-D [B,H,S,D], got {tuple(t.shape)}")
    if t.stride(-1) != 1:
        raise ValueError(f"{name} needs a unit channel stride")
    if t.dtype not in _DT:
        raise ValueError(f"{name} dtype {t.dtype} is not supported")
    return _DT[t.dtype], t.stride(0), t.stride(1), t.stride(2)


def _no_grad(*ts):
    if torch.is_grad_enabled() and any(t is not None and t.requires_grad for t in ts):
        raise ValueError("INT8-QK attention is inference-only (inputs require grad)")


def _cont(t: torch.Tensor | None, name: str, dtype: torch.dtype):
    if t is None:
        return None
    if t.dtype != dtype or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous {dtype} tensor")
    return t


def quantize_workspace_bytes(B: int, H: int, Sk: int, D: int) -> int:
    n = ctypes.c_size_t(0)
    _lib.check(_lib.lib().qfa_quantize_workspace_bytes(B, H, Sk, D, ctypes.byref(n)))
    return n.value


def _quant_inputs(q, k, vbs):
    _no_grad(q, k)
    B, H, Sq, D = q.shape
    Hkv, Sk = k.shape[1], k.shape[2]
    if k.shape[0] != B or k.shape[3] != D or k.dtype != q.dtype:
        raise ValueError("q and k must agree in B, D and dtype")
    dq, *qst = _view(q, "q")
    _, *kst = _view(k, "k")
    return (B, H, Hkv, Sq, Sk, D), dq, qst, kst, _cont(vbs, "vbs", torch.int32)


def _quant_outputs(dims, center_k: bool, out: dict | None, dev) -> dict:
    """The output tensors of a quantize call: those of ``out`` (checked: shape, dtype, contiguity,
    device; kmean and qmu required exactly when K is centred), else new ones."""
    B, H, Hkv, Sq, Sk, D = dims
    want = dict(q8=((B, H, Sq, D), torch.int8), qs=((B, H, Sq), torch.float32),
                k8=((B, Hkv, Sk, D), torch.int8), ks=((B, Hkv, Sk), torch.float32),
                kmean=((B, Hkv, D), torch.float32), qmu=((B, H, Sq), torch.float32))
    if not center_k:
        want.pop("kmean"), want.pop("qmu")
    if out is None:
        out = {n: torch.empty(shape, dtype=dt, device=dev) for n, (shape, dt) in want.items()}
        out.setdefault("kmean", None), out.setdefault("qmu", None)
        return out
    for n, (shape, dt) in want.items():
        t = out.get(n)
        if t is None:
            raise ValueError(f"out[{n!r}] is required")
        _shape(t, n, shape)
        _cont(t, n, dt)
        if t.device != dev:
            raise ValueError(f"out[{n!r}] is on {t.device}, the inputs on {dev}")
    if not center_k and (out.get("kmean") is not None or out.get("qmu") is not None):
        raise ValueError("kmean and qmu are outputs of a centred call only (center_k=True)")
    return dict(out, kmean=out.get("kmean"), qmu=out.get("qmu"))


def quantize_qk(q: torch.Tensor, k: torch.Tensor, vbs: torch.Tensor | None = None, center_k: bool = True,
                workspace: torch.Tensor | None = None, out: dict | None = None) -> dict:
    """Per-token symmetric int8 Q/K (+ K mean, centring term) on the GPU.

    K may hold fewer heads than Q (grouped-query attention: query head h shares K/V head
    h // (H // Hkv)); the K outputs then have Hkv heads.
    Returns dict(q8, qs, k8, ks, kmean, qmu); kmean/qmu are None when center_k is False. With
    ``out`` (a dict of those keys) the results land in its tensors.
    """
    dims, dq, qst, kst, vbs = _quant_inputs(q, k, vbs)
    B, H, Hkv, Sq, Sk, D = dims
    dev = q.device
    out = _quant_outputs(dims, center_k, out, dev)
    nbytes = quantize_workspace_bytes(B, Hkv, Sk, D) if center_k else 0
    if workspace is None and nbytes:
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    _lib.check(_lib.lib().qfa_quantize_qk(
        B, H, Hkv, Sq, Sk, D, dq, _ptr(q), *qst, _ptr(k), *kst, _ptr(vbs), int(center_k),
        _ptr(out["q8"]), _ptr(out["qs"]), _ptr(out["k8"]), _ptr(out["ks"]), _ptr(out["kmean"]), _ptr(out["qmu"]),
        _ptr(workspace), workspace.numel() if workspace is not None else 0, _stream(dev)))
    return out


def quantize_qk_noalloc(q: torch.Tensor, k: torch.Tensor, vbs: torch.Tensor | None = None, center_k: bool = True,
                        out: dict | None = None) -> dict:
    """:func:`quantize_qk` through qfa_quantize_qk_noalloc: the library allocates nothing (its K-mean
    partials live in static device memory); the outputs are the tensors of ``out`` (keys q8, qs, k8,
    ks, kmean, qmu as :func:`quantize_qk` returns them), allocated here only when it is None."""
    dims, dq, qst, kst, vbs = _quant_inputs(q, k, vbs)
    B, H, Hkv, Sq, Sk, D = dims
    dev = q.device
    out = _quant_outputs(dims, center_k, out, dev)
    _lib.check(_lib.lib().qfa_quantize_qk_noalloc(
        B, H, Hkv, Sq, Sk, D, dq, _ptr(q), *qst, _ptr(k), *kst, _ptr(vbs), int(center_k),
        _ptr(out["q8"]), _ptr(out["qs"]), _ptr(out["k8"]), _ptr(out["ks"]), _ptr(out["kmean"]),
        _ptr(out["qmu"]), _stream(dev)))
    return out


def blockmask_to_index(mask: torch.Tensor):
    """[B,H,Tq,Tk] bool/uint8 tile mask -> (index int32 [B,H,Tq,Tk], count int32 [B,H,Tq])."""
    if mask.dim() != 4:
        raise ValueError("mask must be [B,H,Tq,Tk]")
    m = mask.contiguous()
    if m.dtype == torch.bool:
        m = m.view(torch.uint8)
    if m.dtype != torch.uint8:
        raise ValueError("mask must be bool or uint8")
    B, H, Tq, Tk = m.shape
    index = torch.empty((B, H, Tq, Tk), dtype=torch.int32, device=m.device)
    count = torch.empty((B, H, Tq), dtype=torch.int32, device=m.device)
    _lib.check(_lib.lib().qfa_blockmask_to_index(_ptr(m), B, H, Tq, Tk, _ptr(index), _ptr(count),
                                                 _stream(m.device)))
    return index, count


def qk_scores_i32(q8: torch.Tensor, k8: torch.Tensor) -> torch.Tensor:
    """int32 [B,H,Sq,Sk] scores Q8 K8^T computed by the attention kernel's own QK stage."""
    _no_grad(q8, k8)
    if q8.dim() != 4 or k8.dim() != 4 or q8.dtype != torch.int8 or k8.dtype != torch.int8:
        raise ValueError("q8, k8 must be int8 [B,H,S,D]")
    B, H, Sq, D = q8.shape
    if k8.shape[0] != B or k8.shape[1] != H or k8.shape[3] != D:
        raise ValueError(f"k8 shape {tuple(k8.shape)} does not match q8 {tuple(q8.shape)}")
    Sk = k8.shape[2]
    q8c, k8c = q8.contiguous(), k8.contiguous()
    s32 = torch.empty((B, H, Sq, Sk), dtype=torch.int32, device=q8.device)
    _lib.check(_lib.lib().qfa_qk_scores_i32(B, H, Sq, Sk, D, _ptr(q8c), _ptr(k8c), _ptr(s32), _stream(q8.device)))
    return s32


def _shape(t, name, shape):
    if t is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} shape {tuple(t.shape)} != {tuple(shape)}")


def _attn_call(B, H, Hkv, Sq, Sk, D, qk_args, unquant, v, sm_scale, bias, index, count, vbs, v_scale, segments,
               causal, out, out_dtype, return_lse, lse, splits, workspace):
    """Shared marshalling of the attention entry points: everything but the Q/K operands."""
    _no_grad(v, bias)
    if v.shape != (B, Hkv, Sk, D):
        raise ValueError(f"v shape {tuple(v.shape)} != {(B, Hkv, Sk, D)}")
    _shape(v_scale, "v_scale", (Hkv, D)), _shape(out, "out", (B, H, Sq, D)), _shape(lse, "lse", (B, H, Sq))
    if index is not None:
        T = Sk // 64
        _shape(index, "index", (B, H, T, T)), _shape(count, "count", (B, H, T)), _shape(vbs, "vbs", (T,))
    dv, *vst = _view(v, "v")
    dev = v.device
    if sm_scale is None:
        sm_scale = D ** -0.5
    if out is None:
        out = torch.empty((B, H, Sq, D), dtype=out_dtype or v.dtype, device=dev)
    do, *ost = _view(out, "out")
    if return_lse and lse is None:
        lse = torch.empty((B, H, Sq), dtype=torch.float32, device=dev)
    _cont(lse, "lse", torch.float32)
    bptr, bdt, bsb, bsh, bsq = None, QFA_FP32, 0, 0, 0
    if bias is not None:
        if bias.dim() != 4 or bias.shape[-1] != Sk or bias.stride(-1) != 1:
            raise ValueError("bias must be [B|1,H|1,Q|1,K] with a unit key stride")
        if bias.shape[-2] not in (1, Sq):
            raise ValueError("bias query dim must be 1 or Sq")
        # a per-query bias (query stride != 0) takes the materialised path
        bsq = bias.stride(-2) if bias.shape[-2] > 1 else 0
        if bias.shape[0] not in (1, B) or bias.shape[1] not in (1, H):
            raise ValueError("bias batch/head dims must be 1 or match")
        bdt = QFA_BOOL if bias.dtype == torch.bool else _DT.get(bias.dtype)
        if bdt is None:
            raise ValueError(f"bias dtype {bias.dtype}")
        bsb = bias.stride(0) if bias.shape[0] > 1 else 0
        bsh = bias.stride(1) if bias.shape[1] > 1 else 0
        bptr = _ptr(bias)
    _cont(index, "index", torch.int32), _cont(count, "count", torch.int32), _cont(vbs, "vbs", torch.int32)
    _cont(v_scale, "v_scale", torch.float32)
    nseg, seg = 0, None
    if segments is not None:
        segs = [int(x) for pair in segments for x in pair]
        nseg = len(segs) // 2
        seg = (ctypes.c_int64 * max(1, len(segs)))(*segs)
    masks = (ctypes.c_float(sm_scale), bptr, bdt, bsb, bsh, bsq, _ptr(index), _ptr(count), _ptr(vbs), _ptr(v_scale),
             nseg, seg, int(bool(causal)), _ptr(out), do, *ost, _ptr(lse))
    ns = 1
    if splits == "auto":
        ns = splits_auto(B, H, Sq, Sk, causal)
    elif splits is not None:
        ns = int(splits)
    nbytes = split_workspace_bytes(B, H, Sq, D, ns) if ns > 1 else 0
    if nbytes and workspace is None:
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    _cont(workspace, "workspace", torch.uint8)
    wsp, wsn = (_ptr(workspace), workspace.numel()) if workspace is not None else (None, 0)
    L = _lib.lib()
    if unquant:
        _lib.check(L.qfa_attn_fwd_unquant(B, H, Hkv, Sq, Sk, D, *qk_args, _ptr(v), dv, *vst, *masks, ns, wsp, wsn,
                                          _stream(dev)))
    elif ns == 1:
        _lib.check(L.qfa_attn_fwd(B, H, Hkv, Sq, Sk, D, *qk_args, _ptr(v), dv, *vst, *masks, _stream(dev)))
    else:
        _lib.check(L.qfa_attn_fwd_splitk(B, H, Hkv, Sq, Sk, D, *qk_args, _ptr(v), dv, *vst, *masks, ns, wsp, wsn,
                                         _stream(dev)))
    return (out, lse) if (return_lse or lse is not None) else out


def attn_fwd(qk: dict, v: torch.Tensor, sm_scale: float | None = None, *, bias: torch.Tensor | None = None,
             index: torch.Tensor | None = None, count: torch.Tensor | None = None, vbs: torch.Tensor | None = None,
             v_scale: torch.Tensor | None = None, segments=None, causal: bool = False,
             out: torch.Tensor | None = None, out_dtype: torch.dtype | None = None, return_lse: bool = False,
             lse: torch.Tensor | None = None, splits: int | str | None = None, workspace: torch.Tensor | None = None):
    """Attention on int8 Q/K codes (the dict from :func:`quantize_qk`) and bf16/fp16 V.

    bias: additive bias [B|1, H|1, 1|Q, K] (natural log), fp32/bf16/fp16, or a bool
        keep mask (True attends) of that layout. A query dimension of size 1 (or a
        stride-0 expansion) is the shared per-key form, applied through the key terms
        at no per-score cost; a materialised per-query one (int8 Q/K only; 16-byte
        aligned rows) is read value by value, the slow path.
    index/count/vbs: block-sparse mode (from :func:`blockmask_to_index`).
    segments: up to 4 ascending disjoint (start, length) key ranges.
    causal: self-attention (Sq == Sk) where row i attends keys j <= i only.
    return_lse / lse: write the fp32 [B,H,Sq] natural-log LSE (into ``lse`` if given).
    K/V may hold Hkv heads, a divisor of H (grouped-query attention; ``qk`` from
    :func:`quantize_qk` with such a K): query head h reads K/V head h // (H // Hkv), and
    ``v_scale`` is [Hkv, D].
    splits: split-K over the key walk (dense calls): an int >= 1, or "auto" for
        :func:`splits_auto`'s choice; the partials go to ``workspace`` (uint8 device
        tensor of :func:`split_workspace_bytes` bytes, allocated when not given).
    """
    q8, qs, k8, ks, qmu = qk["q8"], qk["qs"], qk["k8"], qk["ks"], qk.get("qmu")
    B, H, Sq, D = q8.shape
    Hkv, Sk = k8.shape[1], k8.shape[2]
    _shape(k8, "k8", (B, Hkv, Sk, D)), _shape(qs, "qs", (B, H, Sq)), _shape(ks, "ks", (B, Hkv, Sk))
    _shape(qmu, "qmu", (B, H, Sq))
    _cont(q8, "q8", torch.int8), _cont(k8, "k8", torch.int8)
    _cont(qs, "qs", torch.float32), _cont(ks, "ks", torch.float32), _cont(qmu, "qmu", torch.float32)
    # codes of centred K carry their mean; without it the caller states the K was not centred
    centered = qk.get("kmean") is not None
    qk_args = (_ptr(q8), _ptr(qs), _ptr(qmu), _ptr(k8), _ptr(ks), int(centered))
    return _attn_call(B, H, Hkv, Sq, Sk, D, qk_args, False, v, sm_scale, bias, index, count, vbs, v_scale, segments,
                      causal, out, out_dtype, return_lse, lse, splits, workspace)


def attn_fwd_unquant(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, sm_scale: float | None = None, *,
                     bias: torch.Tensor | None = None, index: torch.Tensor | None = None,
                     count: torch.Tensor | None = None, vbs: torch.Tensor | None = None,
                     v_scale: torch.Tensor | None = None, segments=None, causal: bool = False,
                     out: torch.Tensor | None = None, out_dtype: torch.dtype | None = None,
                     return_lse: bool = False, lse: torch.Tensor | None = None, splits: int | str | None = None,
                     workspace: torch.Tensor | None = None):
    """The BF16-QK ablation: the same attention with Q K^T on the unquantized, uncentred
    bf16/fp16 Q [B,H,Sq,D] and K [B,Hkv,Sk,D] (strided views allowed; Q, K and V of one
    dtype). Every other argument as :func:`attn_fwd`."""
    _no_grad(q, k)
    B, H, Sq, D = q.shape
    Hkv, Sk = k.shape[1], k.shape[2]
    if k.shape != (B, Hkv, Sk, D) or k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("q, k and v must agree in B, D and dtype")
    _, *qst = _view(q, "q")
    _, *kst = _view(k, "k")
    qk_args = (_ptr(q), *qst, _ptr(k), *kst)
    return _attn_call(B, H, Hkv, Sq, Sk, D, qk_args, True, v, sm_scale, bias, index, count, vbs, v_scale, segments,
                      causal, out, out_dtype, return_lse, lse, splits, workspace)


def split_workspace_bytes(B: int, H: int, Sq: int, D: int, splits: int) -> int:
    """Bytes of the split-K workspace (fp32 partial O and LSE of every split)."""
    n = ctypes.c_size_t(0)
    _lib.check(_lib.lib().qfa_attn_split_workspace_bytes(B, H, Sq, D, splits, ctypes.byref(n)))
    return n.value


def splits_auto(B: int, H: int, Sq: int, Sk: int, causal: bool = False) -> int:
    """The library's split count for this shape on the current device (1 = no split)."""
    n = ctypes.c_int(0)
    _lib.check(_lib.lib().qfa_attn_splits_auto(B, H, Sq, Sk, int(bool(causal)), ctypes.byref(n)))
    return n.value


def lse_merge(o_a: torch.Tensor, lse_a: torch.Tensor, o_b: torch.Tensor, lse_b: torch.Tensor,
              out: torch.Tensor | None = None, lse_out: torch.Tensor | None = None, out_dtype=None):
    """Exact merge of two partial attentions over disjoint key sets -> (out, lse)."""
    B, H, S, D = o_a.shape
    if o_b.shape != o_a.shape or lse_a.shape != (B, H, S) or lse_b.shape != (B, H, S):
        raise ValueError("partials must share [B,H,S,D] and lse [B,H,S]")
    da, *ast = _view(o_a, "o_a")
    db, *bst = _view(o_b, "o_b")
    _cont(lse_a, "lse_a", torch.float32), _cont(lse_b, "lse_b", torch.float32)
    if out is None:
        out = torch.empty((B, H, S, D), dtype=out_dtype or o_a.dtype, device=o_a.device)
    do, *ost = _view(out, "out")
    if lse_out is None:
        lse_out = torch.empty((B, H, S), dtype=torch.float32, device=o_a.device)
    _cont(lse_out, "lse_out", torch.float32)
    _lib.check(_lib.lib().qfa_lse_merge(B, H, S, D, _ptr(o_a), da, *ast, _ptr(lse_a), _ptr(o_b), db, *bst,
                                        _ptr(lse_b), _ptr(out), do, *ost, _ptr(lse_out), _stream(o_a.device)))
    return out, lse_out


def int8_attention(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, scale: float | None = None,
                   attn_mask: torch.Tensor | None = None, *, return_lse: bool = False, center_k: bool = True,
                   segments=None, is_causal: bool = False):
    """Quantize Q/K once and attend (the comfy-kitchen-style entry point).

    attn_mask: a per-key additive float bias [B|1,H|1,1|Q,K] (stride-0 over Q).
    """
    qk = quantize_qk(q, k, center_k=center_k)
    if scale is None:
        scale = q.shape[-1] ** -0.5
    return attn_fwd(qk, v, scale, bias=attn_mask, segments=segments, causal=is_causal, return_lse=return_lse)


def sm_scale_default(D: int) -> float:
    return float(torch.tensor(1.0 / math.sqrt(D), dtype=torch.float32))
