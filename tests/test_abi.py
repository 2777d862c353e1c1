"""CPU checks of the C ABI: the library loads, exports every declared symbol,
and rejects bad arguments on the host before launching anything."""
import ctypes
import os
import re

import pytest

import quantized_flash_attention_amd as qfa
from quantized_flash_attention_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qfa.h")

pytestmark = pytest.mark.skipif(not os.path.exists(_lib.LIB_PATH), reason="libqfa.so not built")

FAKE = ctypes.c_void_p(0x10000)  # aligned, never dereferenced: every call below fails validation first


def declared_symbols(header=HEADER):
    text = open(header).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\*?\s+\*?(qfa_\w+)\(", text, re.M)))


def test_exports_every_declared_symbol():
    syms = declared_symbols()
    assert set(syms) == set(_lib.EXPORTS)
    L = _lib.lib()
    for s in syms:
        assert hasattr(L, s), s
    assert L.qfa_version() >= 100
    assert L.qfa_status_string(2) == b"unsupported"


def test_probe_library_exports_its_header():
    """The measurement helper library (include/qfa_probe.h) loads and exports what its header declares;
    its argument checks run on the host (no GPU call happens for a rejected argument)."""
    path = os.path.join(os.path.dirname(_lib.LIB_PATH), "libqfa_probe.so")
    L = ctypes.CDLL(path)
    syms = declared_symbols(os.path.join(ROOT, "include", "qfa_probe.h"))
    assert syms == ["qfa_probe_mfma"]
    for s in syms:
        assert hasattr(L, s), s
    L.qfa_probe_mfma.argtypes = [ctypes.c_int] * 3 + [ctypes.c_void_p] * 3
    assert L.qfa_probe_mfma(0, 4, 0, FAKE, FAKE, None) == 1        # no blocks
    assert L.qfa_probe_mfma(8, 6, 0, FAKE, FAKE, None) == 1        # iterations not a multiple of 4
    assert L.qfa_probe_mfma(8, 4, 11, FAKE, FAKE, None) == 1       # no such mix
    assert L.qfa_probe_mfma(8, 4, 0, None, FAKE, None) == 1


def test_workspace_size():
    """K-mean partials: chunks of at least 256 rows, up to 256 per (b, K/V head) and 4096 in all, 16
    bytes per channel."""
    n = qfa.quantize_workspace_bytes(1, 56, 33600, 128)
    assert n == 56 * 73 * 128 * 16                    # 132 chunks of 256 rows, 4096 slots in all
    assert qfa.quantize_workspace_bytes(1, 20, 9216, 64) == 20 * 36 * 64 * 16
    assert qfa.quantize_workspace_bytes(1, 2, 1 << 20, 128) == 2 * 256 * 128 * 16   # at most 256 per head
    assert qfa.quantize_workspace_bytes(8, 128, 4096, 128) == 1024 * 4 * 128 * 16   # 4096 slots in all
    assert qfa.quantize_workspace_bytes(1, 5000, 300, 64) == 5000 * 64 * 16          # one chunk each
    assert qfa.quantize_workspace_bytes(1, 3, 100, 64) == 3 * 64 * 16
    assert qfa.quantize_workspace_bytes(1, 1, 0, 64) == 0


def _quant(**kw):
    a = dict(B=1, H=2, Sq=128, Sk=128, D=128, dtype=1, q=FAKE, q_s=(32768, 16384, 128), k=FAKE,
             k_s=(32768, 16384, 128), vbs=None, center=1, outs=[FAKE] * 6, ws=FAKE, wsb=1 << 20)
    a.update(kw)
    return _lib.lib().qfa_quantize_qk(a["B"], a["H"], a.get("Hkv", a["H"]), a["Sq"], a["Sk"], a["D"], a["dtype"],
                                      a["q"], *a["q_s"], a["k"], *a["k_s"], a["vbs"], a["center"], *a["outs"],
                                      a["ws"], a["wsb"], None)


def test_quantize_rejects_bad_arguments():
    assert _quant(D=96) == _lib.QFA_ERR_UNSUPPORTED
    assert b"head dimension" in _lib.lib().qfa_last_error()
    assert _quant(dtype=3) == _lib.QFA_ERR_UNSUPPORTED
    assert _quant(dtype=7) == _lib.QFA_ERR_INVALID_ARG
    assert _quant(q=None) == _lib.QFA_ERR_INVALID_ARG
    assert _quant(q=ctypes.c_void_p(0x10008)) == _lib.QFA_ERR_INVALID_ARG  # misaligned
    assert _quant(q_s=(32768, 16384, 100)) == _lib.QFA_ERR_INVALID_ARG     # row stride not 16-byte
    assert _quant(vbs=FAKE, Sq=100, Sk=100) == _lib.QFA_ERR_INVALID_ARG
    assert _quant(ws=None) == _lib.QFA_ERR_INVALID_ARG
    assert _quant(wsb=16) == _lib.QFA_ERR_INVALID_ARG
    assert _quant(outs=[FAKE, FAKE, FAKE, FAKE, None, FAKE]) == _lib.QFA_ERR_INVALID_ARG  # kmean with center_k
    assert _quant(B=-1) == _lib.QFA_ERR_INVALID_ARG
    assert _quant(Hkv=3) == _lib.QFA_ERR_INVALID_ARG
    assert _quant(Hkv=0) == _lib.QFA_ERR_INVALID_ARG


def _attn(**kw):
    a = dict(B=1, H=2, Sq=128, Sk=128, D=128, qk=[FAKE] * 5, v=FAKE, vdt=1, v_s=(32768, 16384, 128), scale=0.088,
             bias=None, bdt=3, b_s=(0, 0), index=None, count=None, vbs=None, vsc=None, nseg=0, seg=None, causal=0,
             out=FAKE, odt=1, o_s=(32768, 16384, 128), lse=None)
    a.update(kw)
    return _lib.lib().qfa_attn_fwd(a["B"], a["H"], a.get("Hkv", a["H"]), a["Sq"], a["Sk"], a["D"], *a["qk"],
                                   a.get("centered", 1), a["v"], a["vdt"], *a["v_s"],
                                   ctypes.c_float(a["scale"]), a["bias"], a["bdt"], *a["b_s"], a.get("bsq", 0), a["index"],
                                   a["count"], a["vbs"], a["vsc"], a["nseg"], a["seg"], a["causal"], a["out"], a["odt"],
                                   *a["o_s"], a["lse"], None)


def _attn_split(ns, ws=FAKE, wsb=1 << 30, **kw):
    a = dict(B=1, H=2, Sq=128, Sk=128, D=128, qk=[FAKE] * 5, v=FAKE, vdt=1, v_s=(32768, 16384, 128), scale=0.088,
             bias=None, bdt=3, b_s=(0, 0), index=None, count=None, vbs=None, vsc=None, nseg=0, seg=None, causal=0,
             out=FAKE, odt=1, o_s=(32768, 16384, 128), lse=None)
    a.update(kw)
    return _lib.lib().qfa_attn_fwd_splitk(a["B"], a["H"], a["H"], a["Sq"], a["Sk"], a["D"], *a["qk"],
                                          a.get("centered", 1), a["v"],
                                          a["vdt"], *a["v_s"], ctypes.c_float(a["scale"]), a["bias"], a["bdt"],
                                          *a["b_s"], 0, a["index"], a["count"], a["vbs"], a["vsc"], a["nseg"],
                                          a["seg"], a["causal"], a["out"], a["odt"], *a["o_s"], a["lse"], ns, ws,
                                          wsb, None)


def test_split_rejects_bad_arguments():
    L = _lib.lib()
    n = ctypes.c_size_t(0)
    assert L.qfa_attn_split_workspace_bytes(2, 3, 100, 128, 4, ctypes.byref(n)) == _lib.QFA_OK
    assert n.value == 4 * 2 * 3 * 100 * 129 * 4
    assert L.qfa_attn_split_workspace_bytes(2, 3, 100, 64, 1, ctypes.byref(n)) == _lib.QFA_OK and n.value == 0
    assert L.qfa_attn_split_workspace_bytes(2, 3, 100, 64, 0, ctypes.byref(n)) == _lib.QFA_ERR_INVALID_ARG
    assert L.qfa_attn_split_workspace_bytes(2, 3, 100, 96, 2, ctypes.byref(n)) == _lib.QFA_ERR_UNSUPPORTED
    for ns in (0, -1, 65):
        assert _attn_split(ns) == _lib.QFA_ERR_INVALID_ARG
    assert _attn_split(4, index=FAKE, count=FAKE) == _lib.QFA_ERR_UNSUPPORTED
    assert b"block-sparse" in L.qfa_last_error()
    need = 4 * 2 * 128 * 129 * 4
    assert _attn_split(4, wsb=need - 1) == _lib.QFA_ERR_INVALID_ARG
    assert b"workspace" in L.qfa_last_error()
    assert _attn_split(4, ws=None) == _lib.QFA_ERR_INVALID_ARG
    assert _attn_split(4, ws=ctypes.c_void_p(0x10008)) == _lib.QFA_ERR_INVALID_ARG   # misaligned
    assert _attn_split(4, D=80) == _lib.QFA_ERR_UNSUPPORTED   # the plain checks still apply


def _attn_unquant(dtype=1, q=FAKE, k=FAKE, q_s=(32768, 16384, 128), k_s=(32768, 16384, 128), Sk=128, ns=1,
                  bias=None, bsq=0):
    st = (32768, 16384, 128)
    return _lib.lib().qfa_attn_fwd_unquant(1, 2, 2, 128, Sk, 128, q, *q_s, k, *k_s, FAKE, dtype, *st,
                                           ctypes.c_float(0.088), bias, 3, 0, 0, bsq, None, None, None, None, 0, None, 0,
                                           FAKE, 1, *st, None, ns, None, 0, None)


def test_unquant_rejects_bad_arguments():
    assert _attn_unquant(dtype=3) == _lib.QFA_ERR_UNSUPPORTED                     # fp32 Q/K/V
    assert _attn_unquant(q=None) == _lib.QFA_ERR_INVALID_ARG
    assert _attn_unquant(k=None) == _lib.QFA_ERR_INVALID_ARG
    assert _attn_unquant(q=ctypes.c_void_p(0x10008)) == _lib.QFA_ERR_INVALID_ARG  # misaligned
    assert _attn_unquant(k_s=(32768, 16384, 100)) == _lib.QFA_ERR_INVALID_ARG     # row stride not 16 bytes
    assert _attn_unquant(k_s=(1 << 40, 1 << 32, 1 << 24)) == _lib.QFA_ERR_UNSUPPORTED
    assert _attn_unquant(ns=2) == _lib.QFA_ERR_INVALID_ARG                       # split without workspace
    assert _attn_unquant(q=None, k=None, Sk=0) == _lib.QFA_ERR_INVALID_ARG       # rows still need Q
    assert _attn_unquant(bias=FAKE, bsq=128) == _lib.QFA_ERR_UNSUPPORTED          # per-query bias


def _segs(*pairs):
    flat = [x for p in pairs for x in p]
    return (ctypes.c_int64 * len(flat))(*flat)


def test_attn_rejects_bad_arguments():
    assert _attn(D=80) == _lib.QFA_ERR_UNSUPPORTED
    assert _attn(vdt=3) == _lib.QFA_ERR_UNSUPPORTED
    assert _attn(odt=9) == _lib.QFA_ERR_INVALID_ARG
    assert _attn(qk=[None] + [FAKE] * 4) == _lib.QFA_ERR_INVALID_ARG
    assert _attn(scale=0.0) == _lib.QFA_ERR_INVALID_ARG
    assert _attn(scale=float("nan")) == _lib.QFA_ERR_INVALID_ARG
    assert _attn(bias=FAKE, index=FAKE, count=FAKE) == _lib.QFA_ERR_INVALID_ARG
    assert b"mutually exclusive" in _lib.lib().qfa_last_error()
    assert _attn(bias=FAKE, bdt=5) == _lib.QFA_ERR_INVALID_ARG
    assert _attn(index=FAKE) == _lib.QFA_ERR_INVALID_ARG                       # no count
    assert _attn(index=FAKE, count=FAKE, Sq=128, Sk=192) == _lib.QFA_ERR_INVALID_ARG
    assert _attn(index=FAKE, count=FAKE, nseg=1, seg=_segs((0, 64))) == _lib.QFA_ERR_INVALID_ARG
    assert _attn(nseg=5, seg=_segs(*[(0, 1)] * 5)) == _lib.QFA_ERR_INVALID_ARG
    assert _attn(nseg=1, seg=None) == _lib.QFA_ERR_INVALID_ARG
    assert _attn(nseg=1, seg=_segs((100, 40))) == _lib.QFA_ERR_INVALID_ARG      # past Sk
    assert _attn(nseg=2, seg=_segs((50, 10), (55, 10))) == _lib.QFA_ERR_INVALID_ARG  # overlapping
    assert _attn(nseg=2, seg=_segs((60, 10), (0, 10))) == _lib.QFA_ERR_INVALID_ARG   # descending
    assert _attn(out=ctypes.c_void_p(0x10004)) == _lib.QFA_ERR_INVALID_ARG
    assert _attn(vsc=ctypes.c_void_p(0x10004)) == _lib.QFA_ERR_INVALID_ARG
    # causal: self-attention only; not with segments or a block-sparse mask
    assert _attn(causal=1, Sk=256, v_s=(65536, 32768, 128)) == _lib.QFA_ERR_INVALID_ARG
    assert b"Sq == Sk" in _lib.lib().qfa_last_error()
    assert _attn(causal=1, nseg=1, seg=_segs((0, 128))) == _lib.QFA_ERR_UNSUPPORTED
    assert _attn(causal=1, index=FAKE, count=FAKE) == _lib.QFA_ERR_UNSUPPORTED
    # materialised per-query bias: alignment, stride >= Sk, 32-row span
    assert _attn(bias=FAKE, bsq=-4) == _lib.QFA_ERR_INVALID_ARG
    assert _attn(bias=FAKE, bsq=100) == _lib.QFA_ERR_INVALID_ARG                 # below Sk = 128
    assert _attn(bias=FAKE, bsq=130) == _lib.QFA_ERR_INVALID_ARG                 # 520-byte rows
    assert _attn(bias=ctypes.c_void_p(0x10008), bsq=128) == _lib.QFA_ERR_INVALID_ARG
    assert _attn(bias=FAKE, bsq=1 << 24) == _lib.QFA_ERR_UNSUPPORTED
    assert _attn(bias=FAKE, bsq=128, index=FAKE, count=FAKE) == _lib.QFA_ERR_INVALID_ARG
    # grouped-query heads: Hkv must divide H
    for hkv in (0, 3, 4, -1):
        assert _attn(Hkv=hkv) == _lib.QFA_ERR_INVALID_ARG
    assert b"K/V heads" in _lib.lib().qfa_last_error()


def test_attn_centring_term_guard():
    """On codes of centred K the LSE needs the centring term sm_scale * q.mu: a call asking for the LSE
    without qmu is refused before any launch, and so is a qmu passed for uncentred codes."""
    L = _lib.lib()
    no_qmu = [FAKE, FAKE, None, FAKE, FAKE]
    assert _attn(qk=no_qmu, lse=FAKE) == _lib.QFA_ERR_INVALID_ARG
    assert b"centring term" in L.qfa_last_error()
    assert _attn_split(2, qk=no_qmu, lse=FAKE) == _lib.QFA_ERR_INVALID_ARG
    assert _attn(qk=[FAKE] * 5, centered=0) == _lib.QFA_ERR_INVALID_ARG
    assert b"not centred" in L.qfa_last_error()
    # without the LSE, or on uncentred codes, qmu is not needed: these fail only on a later check
    # (a zero softmax scale), which shows they passed the guard
    assert _attn(qk=no_qmu, scale=0.0) == _lib.QFA_ERR_INVALID_ARG
    assert b"sm_scale" in L.qfa_last_error()
    assert _attn(qk=no_qmu, centered=0, lse=FAKE, scale=0.0) == _lib.QFA_ERR_INVALID_ARG
    assert b"sm_scale" in L.qfa_last_error()


def test_merge_rejects_bad_arguments():
    L = _lib.lib()
    st = (32768, 16384, 128)

    def m(oa=FAKE, adt=1, ob=FAKE, o=FAKE, odt=1, o_s=st, la=FAKE, D=128):
        return L.qfa_lse_merge(1, 2, 128, D, oa, adt, *st, la, ob, 1, *st, FAKE, o, odt, *o_s, None, None)

    assert m(D=32) == _lib.QFA_ERR_UNSUPPORTED
    assert m(adt=4) == _lib.QFA_ERR_INVALID_ARG
    assert m(la=None) == _lib.QFA_ERR_INVALID_ARG
    assert m(o=FAKE, odt=3) == _lib.QFA_ERR_INVALID_ARG         # aliases o_a with another dtype
    assert m(o=FAKE, o_s=(32768, 16384, 256)) == _lib.QFA_ERR_INVALID_ARG


def test_blockmask_rejects_bad_arguments():
    L = _lib.lib()
    assert L.qfa_blockmask_to_index(None, 1, 1, 4, 4, FAKE, FAKE, None) == _lib.QFA_ERR_INVALID_ARG
    assert L.qfa_blockmask_to_index(FAKE, 1, -1, 4, 4, FAKE, FAKE, None) == _lib.QFA_ERR_INVALID_ARG
    assert L.qfa_blockmask_to_index(FAKE, 0, 1, 4, 4, FAKE, FAKE, None) == _lib.QFA_OK  # empty: nothing to do


def test_qk_scores_rejects_bad_arguments():
    L = _lib.lib()
    assert L.qfa_qk_scores_i32(1, 1, 64, 64, 96, FAKE, FAKE, FAKE, None) == _lib.QFA_ERR_UNSUPPORTED
    assert L.qfa_qk_scores_i32(1, 1, 64, 64, 128, None, FAKE, FAKE, None) == _lib.QFA_ERR_INVALID_ARG
    assert L.qfa_qk_scores_i32(1, 1, 64, 64, 128, FAKE, FAKE, ctypes.c_void_p(0x10004), None) == \
        _lib.QFA_ERR_INVALID_ARG                                  # misaligned output
    assert L.qfa_qk_scores_i32(1, 1, -1, 64, 128, FAKE, FAKE, FAKE, None) == _lib.QFA_ERR_INVALID_ARG
    assert L.qfa_qk_scores_i32(1, 1, 64, 0, 128, FAKE, FAKE, FAKE, None) == _lib.QFA_OK  # no keys: no scores


def test_python_binding_refuses_grad_and_bad_bias():
    import torch
    q = torch.zeros(1, 1, 64, 128, dtype=torch.bfloat16, requires_grad=True)
    with pytest.raises(ValueError, match="inference-only"):
        qfa.quantize_qk(q, q)
    qk = dict(q8=torch.zeros(1, 1, 64, 128, dtype=torch.int8), qs=torch.zeros(1, 1, 64),
              k8=torch.zeros(1, 1, 64, 128, dtype=torch.int8), ks=torch.zeros(1, 1, 64))
    v = torch.zeros(1, 1, 64, 128, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="query dim"):
        qfa.attn_fwd(qk, v, bias=torch.zeros(1, 1, 7, 64))


def test_python_binding_checks_quantize_outputs():
    # caller-provided outputs are checked before any call into the library
    import torch
    q = torch.zeros(1, 2, 64, 128, dtype=torch.bfloat16)
    k = torch.zeros(1, 2, 96, 128, dtype=torch.bfloat16)

    def outs(**over):
        o = dict(q8=torch.zeros(1, 2, 64, 128, dtype=torch.int8), qs=torch.zeros(1, 2, 64),
                 k8=torch.zeros(1, 2, 96, 128, dtype=torch.int8), ks=torch.zeros(1, 2, 96),
                 kmean=torch.zeros(1, 2, 128), qmu=torch.zeros(1, 2, 64))
        o.update(over)
        return o

    for fn in (qfa.quantize_qk, qfa.quantize_qk_noalloc):
        with pytest.raises(ValueError, match="kmean shape"):
            fn(q, k, out=outs(kmean=torch.zeros(1, 2, 64)))
        with pytest.raises(ValueError, match="qmu shape"):
            fn(q, k, out=outs(qmu=torch.zeros(1, 2, 63)))
        with pytest.raises(ValueError, match="required"):
            fn(q, k, out=outs(qmu=None))
        with pytest.raises(ValueError, match="k8 must be a contiguous"):
            fn(q, k, out=outs(k8=torch.zeros(1, 2, 96, 128, dtype=torch.uint8)))
        with pytest.raises(ValueError, match="centred call only"):
            fn(q, k, center_k=False, out=outs())
