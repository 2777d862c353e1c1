"""The allocation-free quantize entry point (qfa_quantize_qk_noalloc, called through the C ABI)
against the workspace entry point qfa_quantize_qk on the same inputs: every output bit for bit, on
calls in a row whose later ones are smaller (the scratch keeps the previous call's contents), with
grouped-query heads, fp16, a validity vector and no centring; and the size limit of its scratch,
refused before any launch."""
import ctypes

import numpy as np
import pytest
import torch

import workloads as W
from quantized_flash_attention_amd import _lib

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import quantized_flash_attention_amd as qfa

DEV = torch.device("cuda:0")
_DT = {torch.bfloat16: _lib.QFA_BF16, torch.float16: _lib.QFA_FP16}


def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _noalloc(q, k, vbs=None, center=True):
    """qfa_quantize_qk_noalloc through ctypes, into outputs allocated here."""
    B, H, Sq, D = q.shape
    Hkv, Sk = k.shape[1], k.shape[2]
    out = dict(q8=torch.full((B, H, Sq, D), 99, dtype=torch.int8, device=DEV),
               qs=torch.full((B, H, Sq), 7.0, device=DEV),
               k8=torch.full((B, Hkv, Sk, D), 99, dtype=torch.int8, device=DEV),
               ks=torch.full((B, Hkv, Sk), 7.0, device=DEV),
               kmean=torch.full((B, Hkv, D), 7.0, device=DEV) if center else None,
               qmu=torch.full((B, H, Sq), 7.0, device=DEV) if center else None)
    st = _lib.lib().qfa_quantize_qk_noalloc(
        B, H, Hkv, Sq, Sk, D, _DT[q.dtype], _p(q), *q.stride()[:3], _p(k), *k.stride()[:3], _p(vbs), int(center),
        _p(out["q8"]), _p(out["qs"]), _p(out["k8"]), _p(out["ks"]), _p(out["kmean"]), _p(out["qmu"]),
        ctypes.c_void_p(torch.cuda.current_stream(DEV).cuda_stream))
    assert st == _lib.QFA_OK, _lib.lib().qfa_last_error()
    return out


def _same(a, b, what):
    for name in ("q8", "qs", "k8", "ks", "kmean", "qmu"):
        x, y = a[name], b[name]
        if x is None:
            assert y is None, f"{what}: {name}"
            continue
        assert torch.equal(x, y), f"{what}: {name} differs from the workspace entry point"


CALLS = [
    # (workload, B, H, Hkv, Sq, Sk, vbs, centre): each call smaller than the one before
    ("band", 1, 8, 8, 700, 20000, None, True),      # 79 chunks of 254 rows per head
    ("dense4k", 2, 4, 2, 1000, 3000, None, True),   # grouped-query, 12 chunks per head
    ("d64", 1, 3, 3, 300, 517, None, True),         # fp16, D = 64
    ("sparse", 1, 2, 2, 320, 320, "vbs", True),     # validity vector: pads out of the mean
    ("tiny", 1, 2, 1, 100, 130, None, False),       # no centring: the scratch is not used
]


def test_noalloc_matches_workspace_entry_point():
    for i, (wn, B, H, Hkv, Sq, Sk, vbs_kind, center) in enumerate(CALLS):
        w = W.WORKLOADS[wn]
        q, k, _ = W.make_qkv(w, B=B, H=H, Hkv=Hkv, Sq=Sq, Sk=Sk)
        vbs = None
        if vbs_kind:
            vbs = np.array([64, 17, 0, 64, 40], np.int32)
            W.zero_pads(q, vbs), W.zero_pads(k, vbs)
        tq, tk = (torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).to(DEV) if x.dtype == np.uint16
                  else torch.from_numpy(x).to(DEV) for x in (q, k))
        tv = None if vbs is None else torch.from_numpy(vbs).to(DEV)
        ref = qfa.quantize_qk(tq, tk, tv, center_k=center)
        got = _noalloc(tq, tk, tv, center)
        torch.cuda.synchronize()
        _same(got, ref, f"call {i} ({wn})")
        # the binding's wrapper of the same entry point
        _same(qfa.quantize_qk_noalloc(tq, tk, tv, center_k=center), ref, f"call {i} ({wn}), binding")


def test_noalloc_rejects_calls_beyond_its_scratch():
    """B*Hkv above 4096 with centring is refused with a message and no launch (the pointers below
    are never dereferenced); without centring the scratch is not needed and the size is accepted
    by this check (it fails later, on the NULL q8 output)."""
    L = _lib.lib()
    fake = ctypes.c_void_p(0x10000)
    args = lambda H, center, q8: (1, H, H, 64, 64, 128, _lib.QFA_BF16, fake, 64 * H * 128, 64 * 128, 128, fake,
                                  64 * H * 128, 64 * 128, 128, None, center, q8, fake, fake, fake, fake, fake, None)
    assert L.qfa_quantize_qk_noalloc(*args(4097, 1, fake)) == _lib.QFA_ERR_UNSUPPORTED
    assert b"4096" in L.qfa_last_error()
    assert L.qfa_quantize_qk_noalloc(*args(4097, 0, None)) == _lib.QFA_ERR_INVALID_ARG
    assert b"q8/qs output is NULL" in L.qfa_last_error()
