"""Seeded random configurations of the whole API against the oracle: shapes (ragged S, D 64/128,
bf16/fp16, GQA), both Q K^T paths, and every option combination the API accepts (key segments,
causal, block-sparse with vbs, per-key or per-query bias or bool keep mask, V scale, split-K,
LSE on/off). Every call runs with an fp32 output, checked at the stated bounds, and with V's 16-bit
type, which must equal that output rounded to nearest even bit for bit."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from tests.gpu_util import DEV, both_outputs, check_lse, check_o, sample_rows, up

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import quantized_flash_attention_amd as qfa

N_CONFIGS = 96


def _config(i):
    rs = np.random.default_rng(1000 + i)
    wn = ["tiny", "dense4k", "d64", "band"][rs.integers(4)]
    w = W.WORKLOADS[wn]
    Hkv = int(rs.integers(1, 3))
    H = Hkv * int(rs.integers(1, 3))
    B = int(rs.integers(1, 3))
    unquant = bool(rs.random() < 0.3)
    sparse = bool(rs.random() < 0.2)
    if sparse:
        Sq = Sk = 64 * int(rs.integers(1, 6))
    else:
        Sq = int(rs.integers(1, 520))
        Sk = Sq if rs.random() < 0.5 else int(rs.integers(1, 900))
    causal = (not sparse) and Sq == Sk and bool(rs.random() < 0.5)
    segments = None
    if not sparse and not causal and rs.random() < 0.3 and Sk > 8:
        cuts = np.sort(rs.choice(np.arange(Sk + 1), size=4, replace=False))
        segments = [(int(cuts[0]), int(cuts[1] - cuts[0])), (int(cuts[2]), int(cuts[3] - cuts[2]))]
    kinds = ["none", "key_fp32", "key_bf16", "key_bool"] + ([] if unquant else ["query_fp32", "query_bf16", "query_bool"])
    bias = "none" if sparse else kinds[rs.integers(len(kinds))]
    return dict(w=wn, B=B, H=H, Hkv=Hkv, Sq=Sq, Sk=Sk, unquant=unquant, sparse=sparse, causal=causal,
                segments=segments, bias=bias, vscale=bool(rs.random() < 0.3),
                splits=1 if sparse else int(rs.choice([1, 1, 2, 3])), lse=bool(rs.random() < 0.7),
                fp32out=bool(rs.random() < 0.2),   # drawn to keep each seed's config; every call runs both
                seed=i)


def _bias(kind, B, H, Sq, Sk, rs):
    """(oracle array, device tensor) of a bias kind; per-query rows padded to 16 bytes."""
    if kind == "none":
        return None, None
    form, dt = kind.split("_")
    shape = (1, 1, 1, Sk) if form == "key" else (int(rs.integers(1, B + 1)) if B > 1 else 1, H, Sq, Sk)
    shape = (shape[0], shape[1] if form == "query" else 1, shape[2], Sk)
    esz = {"fp32": 4, "bf16": 2, "bool": 1}[dt]
    pad = -(-Sk * esz // 16) * 16 // esz
    full_shape = shape[:3] + (pad,)
    if dt == "bool":
        full = rs.random(full_shape) < 0.75
        ref = np.where(full[..., :Sk], 0.0, -np.inf).astype(np.float32)
        return ref, torch.from_numpy(full).to(DEV)[..., :Sk]
    vals = (rs.standard_normal(full_shape) * 2).astype(np.float32)
    vals[rs.random(full_shape) < 0.05] = -np.inf
    if dt == "fp32":
        return vals[..., :Sk], up(vals)[..., :Sk]
    bits = W.f32_to_bf16_bits(vals)
    return bits[..., :Sk], up(bits)[..., :Sk]


@pytest.mark.parametrize("i", range(N_CONFIGS))
def test_random_config(i):
    c = _config(i)
    w = W.WORKLOADS[c["w"]]
    rs = np.random.default_rng(c["seed"])
    q, k, v = W.make_qkv(w, B=c["B"], H=c["H"], Hkv=c["Hkv"], Sq=c["Sq"], Sk=c["Sk"])
    B, H, Sq, Sk, Hkv = c["B"], c["H"], c["Sq"], c["Sk"], c["Hkv"]
    bias_ref, bias_dev = _bias(c["bias"], B, H, Sq, Sk, rs)
    vsc = W.v_scale(w, H=Hkv) if c["vscale"] else None
    kw_o = dict(bias=bias_ref, v_scale=vsc, segments=c["segments"], causal=c["causal"])
    kw_g = dict(bias=bias_dev, v_scale=None if vsc is None else up(vsc), segments=c["segments"],
                causal=c["causal"], splits=c["splits"], return_lse=c["lse"])
    if c["sparse"]:
        T = Sk // 64
        mask = rs.random((B, H, T, T)) < 0.6
        vbs = rs.integers(1, 65, size=T).astype(np.int32)
        for x in (q, k, v):
            W.zero_pads(x, vbs)
        kw_o.update(mask=mask.astype(np.uint8), vbs=vbs)
        idx, cnt = qfa.blockmask_to_index(up(mask))
        kw_g.update(index=idx, count=cnt, vbs=up(vbs))
    what = f"config {i}: {c}"
    tv = up(v)
    if c["unquant"]:
        o_ref, l_ref = oracle.attn(None, v, w.sm_scale, q=W.to_f32(q), k=W.to_f32(k), **kw_o)
        tq, tk = up(q), up(k)
        res = both_outputs(lambda dt: qfa.attn_fwd_unquant(tq, tk, tv, w.sm_scale, out_dtype=dt, **kw_g), tv.dtype, what)
    else:
        vbs_q = kw_o.get("vbs")
        ref = oracle.quantize_qk(q, k, vbs_q)
        o_ref, l_ref = oracle.attn(ref, v, w.sm_scale, **kw_o)
        g = qfa.quantize_qk(up(q), up(k), None if vbs_q is None else up(vbs_q))
        res = both_outputs(lambda dt: qfa.attn_fwd(g, tv, w.sm_scale, out_dtype=dt, **kw_g), tv.dtype, what)
    o = res[0] if c["lse"] else res
    check_o(o, o_ref, what=what)
    if c["lse"]:
        check_lse(res[1], l_ref, what=what)


N_LARGE = 12


def _large_config(i):
    """Large shapes: many query blocks per head, long key walks (split-K ranges over hundreds of
    tiles), causal orders over several CU rounds; rows are sampled."""
    rs = np.random.default_rng(5000 + i)
    wn = ["dense4k", "d64", "band"][rs.integers(3)]
    Hkv = int(rs.integers(1, 5))
    H = Hkv * int(rs.integers(1, 3))
    B = int(rs.integers(1, 3))
    unquant = bool(rs.random() < 0.25)
    Sq = int(rs.integers(1, 4500))
    Sk = Sq if rs.random() < 0.4 else int(rs.integers(1, 40000))
    causal = Sq == Sk and bool(rs.random() < 0.6)
    segments = None
    if not causal and rs.random() < 0.4 and Sk > 8:
        cuts = np.sort(rs.choice(np.arange(Sk + 1), size=4, replace=False))
        segments = [(int(cuts[0]), int(cuts[1] - cuts[0])), (int(cuts[2]), int(cuts[3] - cuts[2]))]
    kinds = ["none", "key_fp32", "key_bf16", "key_bool"] + ([] if unquant else ["query_bf16", "query_bool"])
    bias = kinds[rs.integers(len(kinds))]
    if bias.startswith("query") and B * H * Sq * Sk > 3e7:
        bias = "key_bf16"   # keep the host-side draw of a materialised bias to seconds
    return dict(w=wn, B=B, H=H, Hkv=Hkv, Sq=Sq, Sk=Sk, unquant=unquant, causal=causal, segments=segments,
                bias=bias, vscale=bool(rs.random() < 0.3), splits=["auto", 1, 2, 5][rs.integers(4)],
                lse=bool(rs.random() < 0.7), seed=5000 + i)


@pytest.mark.parametrize("i", range(N_LARGE))
def test_random_large_config(i):
    c = _large_config(i)
    w = W.WORKLOADS[c["w"]]
    rs = np.random.default_rng(c["seed"])
    B, H, Sq, Sk, Hkv = c["B"], c["H"], c["Sq"], c["Sk"], c["Hkv"]
    q, k, v = W.make_qkv(w, B=B, H=H, Hkv=Hkv, Sq=Sq, Sk=Sk)
    bias_ref, bias_dev = _bias(c["bias"], B, H, Sq, Sk, rs)
    vsc = W.v_scale(w, H=Hkv) if c["vscale"] else None
    rows = sample_rows(B, H, Sq, per_head=48, heads=sorted({0, H - 1}), seed=c["seed"])
    kw_o = dict(bias=bias_ref, v_scale=vsc, segments=c["segments"], causal=c["causal"], rows=rows)
    kw_g = dict(bias=bias_dev, v_scale=None if vsc is None else up(vsc), segments=c["segments"],
                causal=c["causal"], splits=c["splits"], return_lse=c["lse"])
    what = f"large config {i}: {c}"
    tv = up(v)
    if c["unquant"]:
        o_ref, l_ref = oracle.attn(None, v, w.sm_scale, q=W.to_f32(q), k=W.to_f32(k), **kw_o)
        tq, tk = up(q), up(k)
        res = both_outputs(lambda dt: qfa.attn_fwd_unquant(tq, tk, tv, w.sm_scale, out_dtype=dt, **kw_g), tv.dtype, what)
    else:
        ref = oracle.quantize_qk(q, k)
        o_ref, l_ref = oracle.attn(ref, v, w.sm_scale, **kw_o)
        g = qfa.quantize_qk(up(q), up(k))
        res = both_outputs(lambda dt: qfa.attn_fwd(g, tv, w.sm_scale, out_dtype=dt, **kw_g), tv.dtype, what)
    o = res[0] if c["lse"] else res
    check_o(o, o_ref, rows, what)
    if c["lse"]:
        check_lse(res[1], l_ref, rows, what)
