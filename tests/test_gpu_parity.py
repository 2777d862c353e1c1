"""GPU parity of the HIP path against the CPU oracle, through the C ABI.

Quantized codes, scales, K mean, tile-index lists: bit-exact. Attention
output: every call runs with an fp32 output, checked at max-abs <= 2e-2 and
mean-abs <= 2e-3, and with V's 16-bit type, which must equal the fp32 output
rounded to nearest even bit for bit; LSE <= 1e-3 absolute. Sizes span several
128-query and 64-key tiles plus ragged tails; the dense 4k and d64 workloads
are compared on every row, the banded and block-sparse ones on rows of every
head and every 128-row query block.
"""
import os

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from tests.gpu_util import (DEV, O_MAX_ABS, as_bshd, block_rows, both_outputs, check_lse, check_o, check_rne, down,
                            sample_rows, up)

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import quantized_flash_attention_amd as qfa


def gpu_quant(q, k, vbs=None, center=True, bshd=False):
    tq, tk = up(q), up(k)
    if bshd:
        tq, tk = as_bshd(tq), as_bshd(tk)
    return qfa.quantize_qk(tq, tk, None if vbs is None else up(vbs), center_k=center)


def assert_quant_equal(g, ref, center=True):
    for name in ("q8", "qs", "k8", "ks") + (("kmean",) if center else ()):
        a, b = down(g[name]), ref[name]
        if not np.array_equal(a, b):
            bad = np.argwhere(a != b)
            raise AssertionError(f"{name}: {len(bad)} mismatches, first at {bad[0].tolist()}: "
                                 f"gpu {a[tuple(bad[0])]} oracle {b[tuple(bad[0])]}")
    if center:
        qm = down(g["qmu"]).astype(np.float64)
        assert np.max(np.abs(qm - ref["qmu"])) <= 1e-4 * max(1.0, np.abs(ref["qmu"]).max())


# ------------------------------------------------------------ int32 scores --

SCORE_CASES = {
    "tiny": dict(w="tiny"),
    "dense_ragged": dict(w="dense4k", H=2, Sq=333, Sk=515),
    "d64_fp16": dict(w="d64", B=2, H=1, Sq=130, Sk=200),
    "band_head": dict(w="band", H=1, Sq=257, Sk=33600),
}


@pytest.mark.parametrize("case", list(SCORE_CASES))
def test_qk_scores_bit_exact(case):
    """The attention kernel's int8 MFMA scores equal the oracle's int32 dot products bit for bit."""
    c = dict(SCORE_CASES[case])
    w = W.WORKLOADS[c.pop("w")]
    q, k, _ = W.make_qkv(w, **c)
    ref = oracle.quantize_qk(q, k)
    s32 = down(qfa.qk_scores_i32(up(ref["q8"]), up(ref["k8"])))
    B, H = ref["q8"].shape[:2]
    for b in range(B):
        for h in range(H):
            exp = oracle.scores_i32(ref["q8"][b, h], ref["k8"][b, h])
            got = s32[b, h]
            if not np.array_equal(got, exp):
                bad = np.argwhere(got != exp)
                raise AssertionError(f"(b,h)=({b},{h}): {len(bad)} mismatches, first {bad[0].tolist()}: "
                                     f"gpu {got[tuple(bad[0])]} oracle {exp[tuple(bad[0])]}")


def test_qk_scores_extremes():
    """All-(+127) and all-(-127) codes reach the largest |S| = D*127^2 exactly; zero rows give 0."""
    D = 128
    q8 = np.zeros((1, 1, 96, D), np.int8)
    k8 = np.zeros((1, 1, 130, D), np.int8)
    q8[0, 0, :32] = 127
    q8[0, 0, 32:64] = -127
    k8[0, 0, :70] = 127
    k8[0, 0, 70:129] = -127
    s32 = down(qfa.qk_scores_i32(up(q8), up(k8)))[0, 0]
    assert np.array_equal(s32, oracle.scores_i32(q8[0, 0], k8[0, 0]))
    assert s32.max() == D * 127 * 127 and s32.min() == -D * 127 * 127
    assert (s32[64:] == 0).all() and (s32[:, 129] == 0).all()


# ---------------------------------------------------------------- quantize --

QUANT_CASES = {
    "tiny": dict(w="tiny"),
    "dense4k_ragged": dict(w="dense4k", H=3, Sq=1000, Sk=1111),
    "d64_fp16": dict(w="d64", B=2, H=2, Sq=777, Sk=530),
    "band_small": dict(w="band", H=2, Sq=300, Sk=2100),
}


@pytest.mark.parametrize("case", list(QUANT_CASES))
@pytest.mark.parametrize("bshd", [False, True])
def test_quantize_bit_exact(case, bshd):
    c = dict(QUANT_CASES[case])
    w = W.WORKLOADS[c.pop("w")]
    q, k, _ = W.make_qkv(w, **c)
    g = gpu_quant(q, k, bshd=bshd)
    assert_quant_equal(g, oracle.quantize_qk(q, k))


def test_quantize_uncentred_and_vbs():
    w = W.WORKLOADS["sparse"]
    q, k, _ = W.make_qkv(w, H=3, Sq=320, Sk=320)
    g = gpu_quant(q, k, center=False)
    assert_quant_equal(g, oracle.quantize_qk(q, k, center_k=False), center=False)
    vbs = np.array([64, 0, 64, 30, 17], np.int32)
    W.zero_pads(q, vbs), W.zero_pads(k, vbs)
    assert_quant_equal(gpu_quant(q, k, vbs), oracle.quantize_qk(q, k, vbs))


def test_quantize_special_rows():
    # zero rows, a row below the smallest normal scale, exact ties, huge values
    w = W.WORKLOADS["tiny"]
    q, k, _ = W.make_qkv(w, Sq=64, Sk=64)
    qf = W.to_f32(q)
    qf[0, 0, 0] = 0
    qf[0, 0, 1] = 1e-37
    qf[0, 0, 2, :4] = [2.0, 1.0, 0.5, 0.0]
    qf[0, 0, 2, 4:] = 0
    qf[0, 1, 3] *= 1e30
    q2 = W.f32_to_bf16_bits(qf)
    k2 = np.broadcast_to(k[:, :, :1], k.shape).copy()  # constant K: centres to zero rows
    g = gpu_quant(q2, k2)
    ref = oracle.quantize_qk(q2, k2)
    assert_quant_equal(g, ref)
    assert np.all(ref["k8"] == 0)


@pytest.mark.parametrize("name", ["dense4k", "d64", "band", "sparse"])
def test_quantize_full_size(name):
    w = W.WORKLOADS[name]
    q, k, _ = W.make_qkv(w)
    vbs = None
    if name == "sparse":
        vbs = W.sparse_vbs(w.Sk // 64, w.extras["last_valid"])
        W.zero_pads(q, vbs), W.zero_pads(k, vbs)
    g = gpu_quant(q, k, vbs)
    assert_quant_equal(g, oracle.quantize_qk(q, k, vbs))


# --------------------------------------------------------------- attention --

def _attn_case(w, q, k, v, *, bias=None, segments=None, vsc=None, bshd=False, rows=None):
    """One call with an fp32 output and one with V's type (checked against each other by RNE);
    returns the fp32 output and LSE with the oracle's."""
    ref = oracle.quantize_qk(q, k)
    g = gpu_quant(q, k)
    tv = up(v)
    if bshd:
        tv = as_bshd(tv)
    B, H, Sq, D = q.shape

    def call(dt):
        out = torch.empty((B, Sq, H, D), dtype=dt, device=DEV).transpose(1, 2) if bshd else None
        return qfa.attn_fwd(g, tv, w.sm_scale, bias=None if bias is None else up(bias), segments=segments,
                            v_scale=None if vsc is None else up(vsc), out=out, out_dtype=dt, return_lse=True)

    o, l = both_outputs(call, tv.dtype)
    o_ref, l_ref = oracle.attn(ref, v, w.sm_scale, bias=bias, segments=segments, v_scale=vsc, rows=rows)
    return o, l, o_ref, l_ref


ATTN_CASES = {
    "tiny": dict(w="tiny"),
    "tiny_bias_f32": dict(w="tiny", bias="fp32"),
    "dense4k_ragged": dict(w="dense4k", H=2, Sq=333, Sk=1000),
    "d64_fp16_ragged": dict(w="d64", B=2, H=2, Sq=300, Sk=517),
    "band_bias_bf16": dict(w="band", H=2, Sq=256, Sk=2100, bias="bf16"),
    "band_bias_fp16": dict(w="band", H=1, Sq=130, Sk=700, bias="fp16"),
    "band_segments": dict(w="band", H=2, Sq=200, Sk=2100, bias="fp32", segments=[(3, 600), (700, 1), (1500, 599)]),
    "vscale": dict(w="sparse", H=2, Sq=192, Sk=192, vscale=True),
    "bshd_views": dict(w="tiny", bshd=True, bias="fp32"),
}


@pytest.mark.parametrize("case", list(ATTN_CASES))
def test_attn_parity(case):
    c = dict(ATTN_CASES[case])
    w = W.WORKLOADS[c.pop("w")]
    bias_dt = c.pop("bias", None)
    segments = c.pop("segments", None)
    vscale = c.pop("vscale", False)
    bshd = c.pop("bshd", False)
    q, k, v = W.make_qkv(w, **c)
    Sk = k.shape[2]
    bias = None
    if bias_dt:
        b64 = W.band_bias(Sk, core=(Sk // 5, Sk - 2 * (Sk // 5)), skirt=Sk // 5)
        if bias_dt == "fp16":
            bias = b64.astype(np.float16).reshape(1, 1, 1, -1)
        else:
            bias = W.bias_tensor(b64, bias_dt)
    vsc = W.v_scale(w, H=q.shape[1]) if vscale else None
    o, l, o_ref, l_ref = _attn_case(w, q, k, v, bias=bias, segments=segments, vsc=vsc, bshd=bshd)
    check_o(o, o_ref, what=case)
    check_lse(l, l_ref, what=case)


def test_attn_edge_cases():
    w = W.WORKLOADS["tiny"]
    # one key: O = V_0 (times nothing), LSE = the key's logit
    q, k, v = W.make_qkv(w, Sq=70, Sk=1)
    o, l, o_ref, l_ref = _attn_case(w, q, k, v)
    check_o(o, o_ref, what="Sk=1")
    check_lse(l, l_ref, what="Sk=1")
    # every key masked by a -inf bias, and an empty segment: O = 0, LSE = -inf
    q, k, v = W.make_qkv(w, Sq=40, Sk=100)
    bias = np.full((1, 1, 1, 100), -np.inf, np.float32)
    bias[..., 50:60] = 0.0
    bias_dead = np.full((1, 1, 1, 100), -np.inf, np.float32)
    for b, seg in ((bias_dead, None), (None, [(10, 0)]), (bias, [(0, 30), (70, 30)])):
        o, l, o_ref, l_ref = _attn_case(w, q, k, v, bias=b, segments=seg)
        assert np.all(o.float().cpu().numpy() == 0) and torch.all(torch.isneginf(l))
        check_lse(l, l_ref)
    # zero query rows attend uniformly
    q0 = np.zeros_like(q)
    o, l, o_ref, l_ref = _attn_case(w, q0, k, v, bias=bias)
    check_o(o, o_ref, what="zero q")
    check_lse(l, l_ref, what="zero q")
    # empty query set is a no-op
    g = gpu_quant(q[:, :, :0], k)
    out = qfa.attn_fwd(g, up(v), w.sm_scale)
    assert out.shape[2] == 0


@pytest.mark.parametrize("center", [True, False])
def test_empty_shapes(center):
    """Empty batch, no heads and no keys are valid calls: nothing to do for B = 0 or H = 0; with
    Sk = 0 the K mean is 0 (the count is clamped to 1), every row has nothing to attend (O = 0,
    LSE = -inf), and the centring term is 0."""
    for B, H, Sq, Sk in ((0, 2, 64, 64), (1, 0, 64, 64), (1, 2, 64, 0), (2, 2, 0, 0)):
        q = torch.zeros((B, H, Sq, 128), dtype=torch.bfloat16, device=DEV).normal_()
        k = torch.zeros((B, H, Sk, 128), dtype=torch.bfloat16, device=DEV).normal_()
        v = torch.zeros((B, H, Sk, 128), dtype=torch.bfloat16, device=DEV).normal_()
        g = qfa.quantize_qk(q, k, center_k=center)
        o, l = qfa.attn_fwd(g, v, 128 ** -0.5, return_lse=True)
        torch.cuda.synchronize()
        assert o.shape == (B, H, Sq, 128) and l.shape == (B, H, Sq)
        if center:
            assert torch.all(g["kmean"] == 0) or Sk > 0
        if Sk == 0 and B * H * Sq > 0:
            assert torch.all(o == 0) and torch.all(torch.isneginf(l))
            if center:
                assert torch.all(g["qmu"] == 0)


def test_keep_mask():
    """A bool [1,1,1,K] keep mask (True attends) equals the additive bias 0 / -inf: the banded
    weights thresholded at 1e-3, a random mask over key segments, and an all-false mask (every
    row O = 0, LSE = -inf)."""
    w = W.WORKLOADS["band"]
    Sk = 1680
    q, k, v = W.make_qkv(w, H=2, Sq=256, Sk=Sk)
    ref = oracle.quantize_qk(q, k)
    g = gpu_quant(q, k)
    tv = up(v)
    weights = np.exp(W.band_bias(Sk, core=(336, 1008), skirt=336))
    rs = np.random.default_rng(11)
    segs = [(0, 700), (900, 780)]
    cases = [("band keep w > 1e-3", weights > 1e-3, None), ("random over segments", rs.random(Sk) < 0.6, segs),
             ("all masked", np.zeros(Sk, bool), None)]
    for what, keep, seg in cases:
        keep4 = keep.reshape(1, 1, 1, Sk)
        add = np.where(keep4, 0.0, -np.inf).astype(np.float32)
        o_ref, l_ref = oracle.attn(ref, v, w.sm_scale, bias=add, segments=seg)
        tb = torch.from_numpy(keep4).to(tv.device)
        o, l = both_outputs(lambda dt: qfa.attn_fwd(g, tv, w.sm_scale, bias=tb, segments=seg, out_dtype=dt,
                                                    return_lse=True), tv.dtype, what)
        check_o(o, o_ref, what=what)
        check_lse(l, l_ref, what=what)


CAUSAL_CASES = {
    # (workload, B, H, S, bias): S spans one key, partial first tiles, whole and ragged
    # 128-row blocks (the two diagonal tiles of a block) and several blocks
    "S1": ("dense4k", 1, 1, 1, None),
    "S64": ("dense4k", 1, 2, 64, None),
    "S129": ("dense4k", 1, 2, 129, None),
    "ragged_333": ("dense4k", 1, 2, 333, None),
    "d64_fp16_517": ("d64", 2, 2, 517, None),
    "bias_fp32_700": ("band", 1, 2, 700, "fp32"),
    "keep_mask_640": ("band", 1, 2, 640, "keep"),
}


@pytest.mark.parametrize("case", list(CAUSAL_CASES))
@pytest.mark.parametrize("lse", [True, False])
def test_causal_parity(case, lse):
    """Causal self-attention (key j attended by row i iff j <= i) against the oracle, with and
    without the LSE (different kernel instances), alone and with a bias or a keep mask."""
    wn, B, H, S, bias_kind = CAUSAL_CASES[case]
    w = W.WORKLOADS[wn]
    q, k, v = W.make_qkv(w, B=B, H=H, Sq=S, Sk=S)
    ref = oracle.quantize_qk(q, k)
    g = gpu_quant(q, k)
    bias_ref = bias_gpu = None
    if bias_kind == "fp32":
        bias_ref = W.bias_tensor(W.band_bias(S, core=(S // 5, S - 2 * (S // 5)), skirt=S // 5), "fp32")
        bias_gpu = up(bias_ref)
    elif bias_kind == "keep":
        keep = (np.random.default_rng(5).random(S) < 0.7).reshape(1, 1, 1, S)
        keep[..., 0] = False   # row 0 then attends nothing: O = 0, LSE = -inf
        bias_ref = np.where(keep, 0.0, -np.inf).astype(np.float32)
        bias_gpu = torch.from_numpy(keep).to(DEV)
    o_ref, l_ref = oracle.attn(ref, v, w.sm_scale, bias=bias_ref, causal=True)
    tv = up(v)
    res = both_outputs(lambda dt: qfa.attn_fwd(g, tv, w.sm_scale, bias=bias_gpu, causal=True, out_dtype=dt,
                                               return_lse=lse), tv.dtype, case)
    o = res[0] if lse else res
    check_o(o, o_ref, what=f"causal {case}")
    if lse:
        check_lse(res[1], l_ref, what=f"causal {case}")
    if bias_kind == "keep":
        assert torch.all(o[:, :, 0] == 0)


def test_causal_full_size_sampled():
    """B1 H16 S4096 D128 causal: two rows of every 128-row block of every head, plus the rows around
    block and tile edges."""
    w = W.WORKLOADS["dense4k"]
    q, k, v = W.make_qkv(w)
    ref = oracle.quantize_qk(q, k)
    g = gpu_quant(q, k)
    rows = block_rows(w.B, w.H, w.Sq, per_block=2, seed=3)
    edges = np.array([0, 1, 63, 64, 127, 128, 129, 2047, 2048, 4031, 4032, 4095])
    rows = np.unique(np.r_[rows, edges, 5 * w.Sq + edges])
    tv = up(v)
    o, l = both_outputs(lambda dt: qfa.attn_fwd(g, tv, w.sm_scale, causal=True, out_dtype=dt, return_lse=True),
                        tv.dtype, "causal full")
    o_ref, l_ref = oracle.attn(ref, v, w.sm_scale, rows=rows, causal=True)
    check_o(o, o_ref, rows, "causal full")
    check_lse(l, l_ref, rows, "causal full")
    del o, l
    # the instance without the LSE, as the dense 4k causal call is timed
    o = both_outputs(lambda dt: qfa.attn_fwd(g, tv, w.sm_scale, causal=True, out_dtype=dt), tv.dtype,
                     "causal full, no LSE")
    check_o(o, o_ref, rows, "causal full, no LSE")


GQA_CASES = {
    # (workload, B, H, Hkv, Sq, Sk, options): runs of H / Hkv query heads share a K/V head
    "h4_kv2": ("dense4k", 1, 4, 2, 300, 517, {}),
    "h6_kv1_bias": ("band", 1, 6, 1, 200, 700, {"bias": True}),
    "b2_h4_kv2_causal": ("dense4k", 2, 4, 2, 333, 333, {"causal": True}),
    "h8_kv2_d64_fp16_vscale": ("d64", 1, 8, 2, 130, 260, {"vscale": True}),
}


@pytest.mark.parametrize("case", list(GQA_CASES))
def test_gqa_parity(case):
    """Grouped-query attention: quantization bit-exact (K mean and codes per K/V head, q.mu
    from the group's mean) and attention against the oracle, with and without the LSE."""
    wn, B, H, Hkv, Sq, Sk, opt = GQA_CASES[case]
    w = W.WORKLOADS[wn]
    q, k, v = W.make_qkv(w, B=B, H=H, Hkv=Hkv, Sq=Sq, Sk=Sk)
    ref = oracle.quantize_qk(q, k)
    g = gpu_quant(q, k)
    assert g["k8"].shape[1] == Hkv and g["kmean"].shape[1] == Hkv
    assert_quant_equal(g, ref)
    bias = W.bias_tensor(W.band_bias(Sk, core=(Sk // 5, Sk - 2 * (Sk // 5)), skirt=Sk // 5), "fp32") \
        if opt.get("bias") else None
    vsc = W.v_scale(w, H=Hkv) if opt.get("vscale") else None
    causal = opt.get("causal", False)
    o_ref, l_ref = oracle.attn(ref, v, w.sm_scale, bias=bias, v_scale=vsc, causal=causal)
    kw = dict(bias=None if bias is None else up(bias), v_scale=None if vsc is None else up(vsc), causal=causal)
    tv = up(v)
    o, l = both_outputs(lambda dt: qfa.attn_fwd(g, tv, w.sm_scale, return_lse=True, out_dtype=dt, **kw), tv.dtype, case)
    check_o(o, o_ref, what=case)
    check_lse(l, l_ref, what=case)
    o2 = both_outputs(lambda dt: qfa.attn_fwd(g, tv, w.sm_scale, out_dtype=dt, **kw), tv.dtype, case)
    check_o(o2, o_ref, what=case + " no LSE")


def test_gqa_sparse():
    """Block-sparse with 4 query heads over 2 K/V heads: per-query-head tile lists."""
    T, H = 6, 4
    rs = np.random.default_rng(3)
    mask = rs.random((1, H, T, T)) < 0.5
    mask[..., 0] = True
    vbs = np.array([64, 64, 30, 64, 64, 17], np.int32)
    o, l, o_ref, l_ref = _sparse_case(T, H, mask, vbs, Hkv=2)
    check_o(o, o_ref, what="gqa sparse")
    check_lse(l, l_ref, what="gqa sparse")


def test_gqa_full_size_sampled():
    """B2 S2048 H16 Hkv2 D128 causal (the grouped-query shape of the FlyDSL table): a row of every
    128-row block of every (b, h)."""
    w = W.WORKLOADS["gqa"]
    q, k, v = W.make_qkv(w)
    ref = oracle.quantize_qk(q, k)
    g = gpu_quant(q, k)
    assert_quant_equal(g, ref)
    rows = block_rows(w.B, w.H, w.Sq, per_block=1, seed=4)
    tv = up(v)
    o, l = both_outputs(lambda dt: qfa.attn_fwd(g, tv, w.sm_scale, causal=True, out_dtype=dt, return_lse=True),
                        tv.dtype, "gqa full")
    o_ref, l_ref = oracle.attn(ref, v, w.sm_scale, rows=rows, causal=True)
    check_o(o, o_ref, rows, "gqa full")
    check_lse(l, l_ref, rows, "gqa full")


SPLIT_CASES = {
    # (workload, shape, splits, options); ranges of the split walks are ragged, and some
    # splits get no tile at all (causal short walks, more splits than tiles)
    "dense_ragged_2": ("dense4k", dict(H=2, Sq=333, Sk=1000), 2, {}),
    "dense_ragged_7": ("dense4k", dict(H=2, Sq=333, Sk=1000), 7, {}),
    "band_bias_segments_3": ("band", dict(H=2, Sq=200, Sk=2100), 3,
                             {"bias": True, "segments": [(3, 600), (700, 1), (1500, 599)]}),
    "causal_4": ("dense4k", dict(H=2, Sq=517, Sk=517), 4, {"causal": True}),
    "gqa_keep_mask_5": ("band", dict(H=4, Hkv=2, Sq=256, Sk=1680), 5, {"keep": True}),
    "d64_fp16_vscale_fp32out_3": ("d64", dict(B=2, H=2, Sq=300, Sk=517), 3, {"vscale": True, "fp32out": True}),
    "more_splits_than_tiles": ("tiny", dict(Sq=100, Sk=130), 8, {}),
}


@pytest.mark.parametrize("case", list(SPLIT_CASES))
def test_split_k_parity(case):
    """Split-K (partials + n-way combine) against the oracle's unsplit attention, with and
    without the LSE, and against the unsplit GPU call."""
    wn, shape, ns, opt = SPLIT_CASES[case]
    w = W.WORKLOADS[wn]
    q, k, v = W.make_qkv(w, **shape)
    H, Hkv, Sk = q.shape[1], k.shape[1], k.shape[2]
    ref = oracle.quantize_qk(q, k)
    g = gpu_quant(q, k)
    bias_ref = bias_gpu = None
    if opt.get("bias"):
        bias_ref = W.bias_tensor(W.band_bias(Sk, core=(Sk // 5, Sk - 2 * (Sk // 5)), skirt=Sk // 5), "fp32")
        bias_gpu = up(bias_ref)
    if opt.get("keep"):
        keep = np.exp(W.band_bias(Sk, core=(Sk // 5, Sk - 2 * (Sk // 5)), skirt=Sk // 5)) > 1e-3
        keep = keep.reshape(1, 1, 1, Sk)
        bias_ref = np.where(keep, 0.0, -np.inf).astype(np.float32)
        bias_gpu = torch.from_numpy(keep).to(DEV)
    vsc = W.v_scale(w, H=Hkv) if opt.get("vscale") else None
    seg, causal = opt.get("segments"), opt.get("causal", False)
    o_ref, l_ref = oracle.attn(ref, v, w.sm_scale, bias=bias_ref, v_scale=vsc, segments=seg, causal=causal)
    kw = dict(bias=bias_gpu, v_scale=None if vsc is None else up(vsc), segments=seg, causal=causal)
    tv = up(v)
    o, l = both_outputs(lambda dt: qfa.attn_fwd(g, tv, w.sm_scale, return_lse=True, splits=ns, out_dtype=dt, **kw),
                        tv.dtype, case)
    check_o(o, o_ref, what=case)
    check_lse(l, l_ref, what=case)
    o2 = both_outputs(lambda dt: qfa.attn_fwd(g, tv, w.sm_scale, splits=ns, out_dtype=dt, **kw), tv.dtype, case)
    check_o(o2, o_ref, what=case + " no LSE")
    o1, l1 = qfa.attn_fwd(g, tv, w.sm_scale, return_lse=True, out_dtype=torch.float32, **kw)
    assert (o - o1).abs().max().item() <= 2e-2
    fin = torch.isfinite(l1)
    assert torch.equal(fin, torch.isfinite(l)) and (l[fin] - l1[fin]).abs().max().item() <= 1e-3


def test_split_k_band_shard_sampled():
    """The banded workload's per-GPU shard with 7 heads (B1 H7 Sq4096 Sk33600, 224 query
    blocks for 256 CUs) with the library's own split count, on a row of every 128-row block."""
    w = W.WORKLOADS["band"]
    q, k, v = W.make_qkv(w, H=7)
    ref = oracle.quantize_qk(q, k)
    g = gpu_quant(q, k)
    ns = qfa.splits_auto(1, 7, w.Sq, w.Sk)
    assert ns > 1
    bias = W.bias_tensor(W.band_bias(w.Sk, core=w.extras["core"], skirt=w.extras["skirt"]), "fp32")
    rows = block_rows(w.B, 7, w.Sq, per_block=1, seed=6)
    o_ref, l_ref = oracle.attn(ref, v, w.sm_scale, bias=bias, rows=rows)
    tv, tb = up(v), up(bias)
    o, l = both_outputs(lambda dt: qfa.attn_fwd(g, tv, w.sm_scale, bias=tb, return_lse=True, splits="auto", out_dtype=dt),
                        tv.dtype, "band shard")
    check_o(o, o_ref, rows, f"band shard, {ns} splits")
    check_lse(l, l_ref, rows, f"band shard, {ns} splits")


UNQUANT_CASES = {
    # (workload, shape, options): the BF16-QK ablation against the oracle's no-quant attention
    "tiny": ("tiny", dict(), {}),
    "dense_ragged_bshd": ("dense4k", dict(H=2, Sq=333, Sk=1000), {"bshd": True}),
    "d64_fp16_ragged": ("d64", dict(B=2, H=2, Sq=300, Sk=517), {}),
    "band_bias_segments": ("band", dict(H=2, Sq=200, Sk=2100),
                           {"bias": True, "segments": [(3, 600), (700, 1), (1500, 599)]}),
    "gqa_causal": ("dense4k", dict(H=4, Hkv=2, Sq=333, Sk=333), {"causal": True}),
    "split_3_vscale": ("dense4k", dict(H=2, Sq=300, Sk=1500), {"splits": 3, "vscale": True}),
}


@pytest.mark.parametrize("case", list(UNQUANT_CASES))
def test_unquant_parity(case):
    wn, shape, opt = UNQUANT_CASES[case]
    w = W.WORKLOADS[wn]
    q, k, v = W.make_qkv(w, **shape)
    Hkv, Sk = k.shape[1], k.shape[2]
    bias = W.bias_tensor(W.band_bias(Sk, core=(Sk // 5, Sk - 2 * (Sk // 5)), skirt=Sk // 5), "fp32") \
        if opt.get("bias") else None
    vsc = W.v_scale(w, H=Hkv) if opt.get("vscale") else None
    seg, causal = opt.get("segments"), opt.get("causal", False)
    o_ref, l_ref = oracle.attn(None, v, w.sm_scale, q=W.to_f32(q), k=W.to_f32(k), bias=bias, v_scale=vsc,
                               segments=seg, causal=causal)
    tq, tk, tv = up(q), up(k), up(v)
    if opt.get("bshd"):
        tq, tk, tv = as_bshd(tq), as_bshd(tk), as_bshd(tv)
    kw = dict(bias=None if bias is None else up(bias), v_scale=None if vsc is None else up(vsc), segments=seg,
              causal=causal, splits=opt.get("splits"))
    o, l = both_outputs(lambda dt: qfa.attn_fwd_unquant(tq, tk, tv, w.sm_scale, return_lse=True, out_dtype=dt, **kw),
                        tv.dtype, case)
    check_o(o, o_ref, what=case)
    check_lse(l, l_ref, what=case)
    o2 = both_outputs(lambda dt: qfa.attn_fwd_unquant(tq, tk, tv, w.sm_scale, out_dtype=dt, **kw), tv.dtype, case)
    check_o(o2, o_ref, what=case + " no LSE")


def test_unquant_sparse():
    T, H = 6, 2
    w = W.WORKLOADS["sparse"]
    rs = np.random.default_rng(4)
    mask = rs.random((1, H, T, T)) < 0.5
    mask[..., 0] = True
    vbs = np.array([64, 64, 30, 64, 64, 17], np.int32)
    q, k, v = W.make_qkv(w, H=H, Sq=64 * T, Sk=64 * T)
    for x in (q, k, v):
        W.zero_pads(x, vbs)
    o_ref, l_ref = oracle.attn(None, v, w.sm_scale, q=W.to_f32(q), k=W.to_f32(k), mask=mask, vbs=vbs)
    idx, cnt = qfa.blockmask_to_index(up(mask))
    tq, tk, tv, tvbs = up(q), up(k), up(v), up(vbs)
    o, l = both_outputs(lambda dt: qfa.attn_fwd_unquant(tq, tk, tv, w.sm_scale, index=idx, count=cnt, vbs=tvbs,
                                                        out_dtype=dt, return_lse=True), tv.dtype, "unquant sparse")
    check_o(o, o_ref, what="unquant sparse")
    check_lse(l, l_ref, what="unquant sparse")


def test_unquant_error_below_int8_error():
    """The ablation's point: against exact attention on the same bf16 inputs, the BF16-QK
    path's error is below the INT8-QK path's (dense4k recipe, K with a per-channel offset)."""
    w = W.WORKLOADS["dense4k"]
    q, k, v = W.make_qkv(w, H=2, Sq=512, Sk=2048)
    exact, _ = oracle.attn(None, v, w.sm_scale, q=W.to_f32(q), k=W.to_f32(k))
    f32 = torch.float32
    o8 = qfa.attn_fwd(gpu_quant(q, k), up(v), w.sm_scale, out_dtype=f32).cpu().numpy().reshape(-1, 128)
    ob = qfa.attn_fwd_unquant(up(q), up(k), up(v), w.sm_scale, out_dtype=f32).cpu().numpy().reshape(-1, 128)
    e8, eb = np.abs(o8 - exact), np.abs(ob - exact)
    assert eb.mean() < e8.mean(), (eb.mean(), e8.mean())
    assert eb.max() <= O_MAX_ABS


def _bias2d(kind, B, H, Sq, Sk, seed):
    """A materialised bias [B|1,H|1,Sq,Sk] (rows padded to a 16-byte multiple) as (numpy view for
    the oracle, device view for the kernel)."""
    rs = np.random.default_rng(seed)
    esz = {"fp32": 4, "bf16": 2, "fp16": 2, "bool": 1}[kind]
    pad = -(-Sk * esz // 16) * 16 // esz
    if kind == "bool":
        full = rs.random((B, H, Sq, pad)) < 0.7
        view = full[..., :Sk]
        ref = np.where(view, 0.0, -np.inf).astype(np.float32)
        dev = torch.from_numpy(full).to(DEV)[..., :Sk]
        return ref, dev
    vals = (rs.standard_normal((B, H, Sq, pad)) * 2.0).astype(np.float32)
    vals[rs.random(vals.shape) < 0.05] = -np.inf
    if kind == "fp32":
        full = vals
    elif kind == "bf16":
        full = W.f32_to_bf16_bits(vals)
    else:
        full = vals.astype(np.float16)
    return full[..., :Sk], up(full)[..., :Sk]


BIAS2D_CASES = {
    # (workload, shape, bias kind, bias batch/head extents, options)
    "fp32_ragged_padded_rows": ("dense4k", dict(H=2, Sq=333, Sk=517), "fp32", (1, 1), {}),
    "bf16_per_batch_head": ("tiny", dict(B=2, H=2, Sq=200, Sk=300), "bf16", (2, 2), {}),
    "fp16_per_head_gqa": ("dense4k", dict(H=4, Hkv=2, Sq=256, Sk=640), "fp16", (1, 4), {}),
    "bool_keep_causal": ("dense4k", dict(H=2, Sq=517, Sk=517), "bool", (1, 1), {"causal": True}),
    "fp32_split_3_no_lse": ("band", dict(H=2, Sq=200, Sk=2100), "fp32", (1, 2), {"splits": 3, "lse": False}),
}


@pytest.mark.parametrize("case", list(BIAS2D_CASES))
def test_bias2d_parity(case):
    """Materialised per-query bias / keep mask [B|1,H|1,Q,K] against the oracle."""
    wn, shape, kind, (bb, bh), opt = BIAS2D_CASES[case]
    w = W.WORKLOADS[wn]
    q, k, v = W.make_qkv(w, **shape)
    B, H, Sq, _ = q.shape
    Sk = k.shape[2]
    ref_b, dev_b = _bias2d(kind, bb, bh, Sq, Sk, seed=len(case))
    if kind == "bool":
        dev_b[..., 3, :] = False          # a row with nothing attended
        ref_b[..., 3, :] = -np.inf
    causal = opt.get("causal", False)
    ref = oracle.quantize_qk(q, k)
    o_ref, l_ref = oracle.attn(ref, v, w.sm_scale, bias=ref_b, causal=causal)
    g = gpu_quant(q, k)
    lse = opt.get("lse", True)
    tv = up(v)
    res = both_outputs(lambda dt: qfa.attn_fwd(g, tv, w.sm_scale, bias=dev_b, causal=causal, splits=opt.get("splits"),
                                               out_dtype=dt, return_lse=lse), tv.dtype, case)
    o = res[0] if lse else res
    check_o(o, o_ref, what=case)
    if lse:
        check_lse(res[1], l_ref, what=case)
    if kind == "bool":
        assert torch.all(o[:, :, 3] == 0)


@pytest.mark.parametrize("kind", ["bool", "bf16", "fp16", "fp32"])
@pytest.mark.parametrize("Sk", [461, 462, 463, 464])
def test_bias2d_row_tail(kind, Sk):
    """The last six keys of every row dominate (kept alone but for a few, or biased +6), so a
    lost key Sk - 1 shows: its bytes share a dword with the row padding whenever Sk*esz is not
    a multiple of 4. The padding holds NaN / +inf (fp forms) or stray keep bytes (bool), which
    must not reach the output. Sq = 100 ends 32-row windows at rows 31, 63, 95 and 99."""
    w = W.WORKLOADS["tiny"]
    Sq, H = 100, 2
    q, k, v = W.make_qkv(w, H=H, Sq=Sq, Sk=Sk)
    rs = np.random.default_rng(Sk)
    esz = {"fp32": 4, "bf16": 2, "fp16": 2, "bool": 1}[kind]
    pad = -(-Sk * esz // 16) * 16 // esz
    shape = (1, H, Sq, pad)
    if kind == "bool":
        full = rs.random(shape) < 0.02
        full[..., Sk - 6:Sk] = True
        full[..., Sk:] = rs.random((1, H, Sq, pad - Sk)) < 0.5
        ref_b = np.where(full[..., :Sk], 0.0, -np.inf).astype(np.float32)
        dev_b = torch.from_numpy(full).to(DEV)[..., :Sk]
    else:
        vals = rs.standard_normal(shape).astype(np.float32)
        vals[..., Sk - 6:Sk] += 6.0
        vals[..., Sk::2] = np.nan
        vals[..., Sk + 1::2] = np.inf
        full = {"fp32": vals, "bf16": W.f32_to_bf16_bits(vals), "fp16": vals.astype(np.float16)}[kind]
        ref_b = full[..., :Sk]
        dev_b = up(full)[..., :Sk]
    ref = oracle.quantize_qk(q, k)
    o_ref, l_ref = oracle.attn(ref, v, w.sm_scale, bias=ref_b)
    what = f"{kind} Sk={Sk}"
    g, tv = gpu_quant(q, k), up(v)
    o, l = both_outputs(lambda dt: qfa.attn_fwd(g, tv, w.sm_scale, bias=dev_b, out_dtype=dt, return_lse=True),
                        tv.dtype, what)
    check_o(o, o_ref, what=what)
    check_lse(l, l_ref, what=what)


def test_bias2d_full_size_sampled():
    """B1 H16 S4096 D128 with a materialised bf16 [1,1,4096,4096] bias: a row of every 128-row block of
    every head."""
    w = W.WORKLOADS["dense4k"]
    q, k, v = W.make_qkv(w)
    ref_b, dev_b = _bias2d("bf16", 1, 1, w.Sq, w.Sk, seed=7)
    ref = oracle.quantize_qk(q, k)
    g = gpu_quant(q, k)
    rows = block_rows(w.B, w.H, w.Sq, per_block=1, seed=7)
    tv = up(v)
    o, l = both_outputs(lambda dt: qfa.attn_fwd(g, tv, w.sm_scale, bias=dev_b, out_dtype=dt, return_lse=True),
                        tv.dtype, "bias2d full")
    o_ref, l_ref = oracle.attn(ref, v, w.sm_scale, bias=ref_b, rows=rows)
    check_o(o, o_ref, rows, "bias2d full")
    check_lse(l, l_ref, rows, "bias2d full")


def test_attn_deterministic():
    w = W.WORKLOADS["dense4k"]
    q, k, v = W.make_qkv(w, H=2, Sq=512, Sk=1024)
    g = gpu_quant(q, k)
    tv = up(v)
    o1, l1 = qfa.attn_fwd(g, tv, w.sm_scale, return_lse=True)
    o2, l2 = qfa.attn_fwd(g, tv, w.sm_scale, return_lse=True)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_split_merge_small():
    w = W.WORKLOADS["band"]
    q, k, v = W.make_qkv(w, H=2, Sq=256, Sk=1680)
    core, skirt = (336, 1008), 336
    bias = W.bias_tensor(W.band_bias(1680, core=core, skirt=skirt), "fp32")
    ref = oracle.quantize_qk(q, k)
    o_ref, l_ref = oracle.attn(ref, v, w.sm_scale, bias=bias)
    g = gpu_quant(q, k)
    tv, tb = up(v), up(bias)
    o_c, l_c = qfa.attn_fwd(g, tv, w.sm_scale, segments=[core], out_dtype=torch.float32, return_lse=True)
    o_s, l_s = qfa.attn_fwd(g, tv, w.sm_scale, bias=tb, segments=[(0, skirt), (core[0] + core[1], skirt)],
                            out_dtype=torch.float32, return_lse=True)
    o_m, l_m = both_outputs(lambda dt: qfa.lse_merge(o_c, l_c, o_s, l_s, out_dtype=dt), torch.bfloat16, "merge")
    check_o(o_m, o_ref, what="split+merge")
    check_lse(l_m, l_ref, what="split+merge")
    # the merge kernel itself against the oracle's merge of the same partials
    mo, ml = oracle.lse_merge(o_c.cpu().numpy().reshape(-1, 128).astype(np.float64), l_c.cpu().numpy(),
                              o_s.cpu().numpy().reshape(-1, 128).astype(np.float64), l_s.cpu().numpy())
    o_m32, l_m32 = qfa.lse_merge(o_c, l_c, o_s, l_s)
    assert np.max(np.abs(o_m32.cpu().numpy().reshape(-1, 128) - mo)) <= 1e-5
    assert np.max(np.abs(l_m32.cpu().numpy().reshape(-1) - ml)) <= 1e-5
    # in place into the first partial
    qfa.lse_merge(o_c, l_c, o_s, l_s, out=o_c, lse_out=l_c)
    assert torch.equal(o_c, o_m32) and torch.equal(l_c, l_m32)


def test_merge_neg_inf_partials():
    a = torch.randn(1, 2, 64, 64, device=DEV)
    la = torch.randn(1, 2, 64, device=DEV)
    dead = torch.full_like(la, -float("inf"))
    o, l = qfa.lse_merge(a, la, torch.zeros_like(a), dead)
    assert torch.allclose(o, a, atol=0, rtol=0) and torch.equal(l, la)
    o, l = qfa.lse_merge(torch.zeros_like(a), dead, torch.zeros_like(a), dead)
    assert torch.all(o == 0) and torch.all(torch.isneginf(l))


# ------------------------------------------------------------ block-sparse --

@pytest.mark.parametrize("Tk,aligned", [(200, True), (1, True), (17, True), (16, True), (32, True),
                                         (1024, True), (1040, True), (2048, True), (32, False)])
@pytest.mark.parametrize("density", [0.0, 0.02, 0.5, 1.0])
def test_blockmask_to_index_exact(Tk, aligned, density):
    """Counts and ascending lists bit-exact against the oracle. Rows of a multiple of 16 bytes on an
    aligned base take the 16-bytes-per-lane kernel (1040: a partial 1024-byte step), the others
    (and a base one byte off) the byte-per-lane one."""
    rs = np.random.default_rng(21 + Tk)
    shape = (2, 3, 37, Tk)
    mask = rs.random(shape) < density
    mask[0, 0, 0] = False
    mask[1, 2, 3] = True
    if aligned:
        dev = up(mask)
    else:
        flat = torch.zeros(mask.size + 1, dtype=torch.bool, device=DEV)
        flat[1:] = up(mask.reshape(-1))
        dev = flat[1:].view(shape)
        assert dev.data_ptr() % 16 == 1
    idx, cnt = qfa.blockmask_to_index(dev)
    r_idx, r_cnt = oracle.blockmask_to_index(mask)
    cnt = cnt.cpu().numpy()
    idx = idx.cpu().numpy()
    assert np.array_equal(cnt, r_cnt)
    for b, h, t in np.ndindex(*shape[:3]):
        n = r_cnt[b, h, t]
        assert np.array_equal(idx[b, h, t, :n], r_idx[b, h, t, :n]), (b, h, t)


def _sparse_case(T, H, mask, vbs, rows=None, Hkv=None, no_lse_too=False):
    w = W.WORKLOADS["sparse"]
    S = 64 * T
    q, k, v = W.make_qkv(w, H=H, Sq=S, Sk=S, Hkv=Hkv)
    for x in (q, k, v):
        W.zero_pads(x, vbs)
    vsc = W.v_scale(w, H=Hkv or H)
    ref = oracle.quantize_qk(q, k, vbs)
    g = gpu_quant(q, k, vbs)
    assert_quant_equal(g, ref)
    idx, cnt = qfa.blockmask_to_index(up(mask))
    tv, tvbs, tvsc = up(v), up(vbs), up(vsc)
    o, l = both_outputs(lambda dt: qfa.attn_fwd(g, tv, w.sm_scale, index=idx, count=cnt, vbs=tvbs, v_scale=tvsc,
                                                out_dtype=dt, return_lse=True), tv.dtype, "sparse")
    o_ref, l_ref = oracle.attn(ref, v, w.sm_scale, mask=mask, vbs=vbs, v_scale=vsc, rows=rows)
    if no_lse_too:
        # the instance without the LSE, as the block-sparse call is timed
        o2 = both_outputs(lambda dt: qfa.attn_fwd(g, tv, w.sm_scale, index=idx, count=cnt, vbs=tvbs, v_scale=tvsc,
                                                  out_dtype=dt), tv.dtype, "sparse, no LSE")
        check_o(o2, o_ref, rows, "sparse, no LSE")
        del o2
    return o, l, o_ref, l_ref


def test_sparse_parity_small():
    T, H = 9, 2
    rs = np.random.default_rng(8)
    mask = rs.random((1, H, T, T)) < 0.35
    mask[0, 0, 4] = False          # a query tile with no key tile: O = 0, LSE = -inf
    mask[0, 1, :, 0] = True
    vbs = np.array([64, 64, 10, 64, 0, 64, 64, 33, 17], np.int32)
    o, l, o_ref, l_ref = _sparse_case(T, H, mask, vbs, no_lse_too=True)
    check_o(o, o_ref, what="sparse")
    check_lse(l, l_ref, what="sparse")


def test_sparse_tile_pairs():
    """Query tiles 2p and 2p+1 share a block that walks the union of their key lists: disjoint
    lists (every key tile masked for one half), both lists empty, identical lists, and a last
    block with a single query tile (T odd)."""
    T, H = 7, 1
    mask = np.zeros((1, H, T, T), bool)
    mask[0, 0, 0, 0::2] = True      # tile 0: even key tiles only
    mask[0, 0, 1, 1::2] = True      # tile 1: odd key tiles only
    # tiles 2 and 3 attend nothing: O = 0, LSE = -inf for both
    mask[0, 0, 4, [1, 2, 6]] = True
    mask[0, 0, 5, [1, 2, 6]] = True
    mask[0, 0, 6, [0, 3, 5, 6]] = True
    vbs = np.array([64, 40, 64, 0, 64, 64, 9], np.int32)
    o, l, o_ref, l_ref = _sparse_case(T, H, mask, vbs)
    check_o(o, o_ref, what="sparse tile pairs")
    check_lse(l, l_ref, what="sparse tile pairs")


def test_sparse_band_structure():
    T, H = 40, 2
    mask = W.sparse_mask(T, H, prefix=3, band=5)
    vbs = W.sparse_vbs(T, 17)
    o, l, o_ref, l_ref = _sparse_case(T, H, mask, vbs)
    check_o(o, o_ref, what="sparse band")
    check_lse(l, l_ref, what="sparse band")


# --------------------------------------------------- full-size, sampled rows --

def test_band_full_size_sampled():
    """B1 H56 Sq4096 Sk33600 D128: unmasked, fp32 bias, bf16 bias and core+skirt split on two rows of
    every 128-row query block of every head; the single calls both as timed (no LSE) and with the
    LSE (other kernel instances)."""
    w = W.WORKLOADS["band"]
    q, k, v = W.make_qkv(w)
    core, skirt = w.extras["core"], w.extras["skirt"]
    b64 = W.band_bias(w.Sk, core=core, skirt=skirt)
    ref = oracle.quantize_qk(q, k)
    g = gpu_quant(q, k)
    assert_quant_equal(g, ref)
    tv = up(v)
    rows = block_rows(w.B, w.H, w.Sq, per_block=2, seed=5)
    o, l = both_outputs(lambda dt: qfa.attn_fwd(g, tv, w.sm_scale, out_dtype=dt, return_lse=True), tv.dtype,
                        "unmasked")
    o_ref, l_ref = oracle.attn(ref, v, w.sm_scale, rows=rows)
    check_o(o, o_ref, rows, "unmasked")
    check_lse(l, l_ref, rows, "unmasked")
    del o, l
    o = both_outputs(lambda dt: qfa.attn_fwd(g, tv, w.sm_scale, out_dtype=dt), tv.dtype, "unmasked, no LSE")
    check_o(o, o_ref, rows, "unmasked, no LSE")
    del o
    refs = {}
    for dt_b in ("fp32", "bf16"):
        bias = W.bias_tensor(b64, dt_b)
        tb = up(bias)
        o, l = both_outputs(lambda dt: qfa.attn_fwd(g, tv, w.sm_scale, bias=tb, out_dtype=dt, return_lse=True),
                            tv.dtype, f"bias {dt_b}")
        refs[dt_b] = oracle.attn(ref, v, w.sm_scale, bias=bias, rows=rows)
        check_o(o, refs[dt_b][0], rows, f"bias {dt_b}")
        check_lse(l, refs[dt_b][1], rows, f"bias {dt_b}")
        del o, l
        o = both_outputs(lambda dt: qfa.attn_fwd(g, tv, w.sm_scale, bias=tb, out_dtype=dt), tv.dtype,
                         f"bias {dt_b}, no LSE")
        check_o(o, refs[dt_b][0], rows, f"bias {dt_b}, no LSE")
        del o
    # the split of the fp32-bias call: core unmasked + skirts with the bias, merged by LSE
    o_ref, l_ref = refs["fp32"]
    tb = up(W.bias_tensor(b64, "fp32"))
    o_c, l_c = qfa.attn_fwd(g, tv, w.sm_scale, segments=[core], out_dtype=torch.float32, return_lse=True)
    o_s, l_s = qfa.attn_fwd(g, tv, w.sm_scale, bias=tb, segments=[(0, skirt), (core[0] + core[1], skirt)],
                            out_dtype=torch.float32, return_lse=True)
    o_m, l_m = both_outputs(lambda dt: qfa.lse_merge(o_c, l_c, o_s, l_s, out_dtype=dt), torch.bfloat16, "merge")
    check_o(o_m, o_ref, rows, "split+merge")
    check_lse(l_m, l_ref, rows, "split+merge")


@pytest.mark.parametrize("lse", [False, True])
def test_dense4k_full_size_every_row(lse):
    """B1 H16 S4096 D128 bf16 with the per-channel K offset: every row of every head, LSE off and on
    (different kernel instances)."""
    w = W.WORKLOADS["dense4k"]
    q, k, v = W.make_qkv(w)
    ref = oracle.quantize_qk(q, k)
    g = gpu_quant(q, k)
    assert_quant_equal(g, ref)
    tv = up(v)
    res = both_outputs(lambda dt: qfa.attn_fwd(g, tv, w.sm_scale, out_dtype=dt, return_lse=lse), tv.dtype, "dense4k")
    o_ref, l_ref = oracle.attn(ref, v, w.sm_scale)
    check_o(res[0] if lse else res, o_ref, what="dense4k all rows")
    if lse:
        check_lse(res[1], l_ref, what="dense4k all rows")


def test_d64_full_size_every_row():
    """B2 H10 S9216 D64 fp16: every row of every (b, h), with the LSE and without it (the two
    instances the d64 configuration times)."""
    w = W.WORKLOADS["d64"]
    q, k, v = W.make_qkv(w)
    ref = oracle.quantize_qk(q, k)
    g = gpu_quant(q, k)
    assert_quant_equal(g, ref)
    tv = up(v)
    o, l = both_outputs(lambda dt: qfa.attn_fwd(g, tv, w.sm_scale, out_dtype=dt, return_lse=True), tv.dtype, "d64")
    o_ref, l_ref = oracle.attn(ref, v, w.sm_scale)
    check_o(o, o_ref, what="d64 all rows")
    check_lse(l, l_ref, what="d64 all rows")
    del o, l
    o = both_outputs(lambda dt: qfa.attn_fwd(g, tv, w.sm_scale, out_dtype=dt), tv.dtype, "d64, no LSE")
    check_o(o, o_ref, what="d64 all rows, no LSE")


def test_sparse_full_size_sampled():
    """B1 H24 S131072 D128, prefix-8 + band-48 tile mask, vbs last tile 17, V scale: a row of every
    128-row block (a block-sparse block's pair of query tiles) of every head, and every row of the
    ragged last tile of two heads, pad rows included."""
    w = W.WORKLOADS["sparse"]
    T = w.Sk // 64
    mask = W.sparse_mask(T, w.H, w.extras["prefix"], w.extras["band"])
    vbs = W.sparse_vbs(T, w.extras["last_valid"])
    rows = block_rows(w.B, w.H, w.Sq, per_block=1, seed=8)
    last = w.Sq - 1 - np.arange(64)
    rows = np.unique(np.r_[rows, last, (w.H - 1) * w.Sq + last])
    o, l, o_ref, l_ref = _sparse_case(T, w.H, mask, vbs, rows=rows, no_lse_too=True)
    check_o(o, o_ref, rows, "sparse full")
    check_lse(l, l_ref, rows, "sparse full")


# ------------------------------------------------------------ HIP graph --
def test_graph_capture_replays():
    """One step of the path (quantize, unmasked, fp32 bias, core/skirt split with LSE, merge)
    captured in a HIP graph: every replay, with eager work and synchronisation between replays,
    reproduces the eager results bit for bit (the library enqueues only kernels: no memset
    nodes, no allocation, no synchronisation)."""
    w = W.WORKLOADS["band"]
    Sk = 1680
    core, skirt = (336, 1008), 336
    q, k, v = W.make_qkv(w, H=2, Sq=256, Sk=Sk)
    bias = W.bias_tensor(W.band_bias(Sk, core=core, skirt=skirt), "fp32")
    tq, tk, tv, tb = up(q), up(k), up(v), up(bias)
    ws = torch.empty(qfa.quantize_workspace_bytes(1, 2, Sk, 128), dtype=torch.uint8, device=tq.device)

    def step():
        qk = qfa.quantize_qk(tq, tk, workspace=ws)
        o_un = qfa.attn_fwd(qk, tv, w.sm_scale)
        o_b = qfa.attn_fwd(qk, tv, w.sm_scale, bias=tb)
        o_c, l_c = qfa.attn_fwd(qk, tv, w.sm_scale, segments=[core], out_dtype=torch.float32, return_lse=True)
        o_s, l_s = qfa.attn_fwd(qk, tv, w.sm_scale, bias=tb, segments=[(0, skirt), (core[0] + core[1], skirt)],
                                out_dtype=torch.float32, return_lse=True)
        o_m, l_m = qfa.lse_merge(o_c, l_c, o_s, l_s, out_dtype=torch.bfloat16)
        return [qk["q8"], qk["k8"], qk["qs"], qk["ks"], qk["kmean"], qk["qmu"], o_un, o_b, o_m, l_m]

    eager = [t.clone() for t in step()]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        outs = step()
    for rep in range(3):
        for t in outs:                       # eager work between replays
            t.zero_()
        step()                               # and an eager step on the same inputs
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for t, e in zip(outs, eager):
            assert torch.equal(t, e), f"replay {rep}: a captured output differs from the eager step"


def test_graph_capture_replays_block_sparse():
    """The block-sparse path (tile mask to index lists, quantize with vbs, sparse attention with a
    V scale and LSE) captured in one HIP graph: every replay, with eager work and synchronisation
    between replays, reproduces the eager results bit for bit."""
    w = W.WORKLOADS["sparse"]
    T, H = 32, 2
    S = 64 * T
    q, k, v = W.make_qkv(w, H=H, Sq=S, Sk=S)
    vbs = W.sparse_vbs(T)
    for x in (q, k, v):
        W.zero_pads(x, vbs)
    mask = W.sparse_mask(T, H, prefix=2, band=4)
    tq, tk, tv, tm, tvbs = up(q), up(k), up(v), up(mask), up(vbs)
    tvs = up(W.v_scale(w, H=H))

    def step():
        idx, cnt = qfa.blockmask_to_index(tm)
        qk = qfa.quantize_qk(tq, tk, tvbs)
        o, l = qfa.attn_fwd(qk, tv, w.sm_scale, index=idx, count=cnt, vbs=tvbs, v_scale=tvs, return_lse=True)
        return [cnt, qk["q8"], qk["k8"], qk["qs"], qk["ks"], o, l]

    eager = [t.clone() for t in step()]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        outs = step()
    for rep in range(3):
        for t in outs:
            t.zero_()
        step()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for t, e in zip(outs, eager):
            assert torch.equal(t, e), f"replay {rep}: a captured output differs from the eager step"


def test_graph_capture_replays_new_paths():
    """Split-K (partials + combine), causal with GQA, the unquantized-QK path and a
    materialised per-query keep mask, captured in one HIP graph with caller-provided
    workspaces: every replay matches the eager results bit for bit."""
    w = W.WORKLOADS["dense4k"]
    S = 700
    q, k, v = W.make_qkv(w, H=4, Hkv=2, Sq=S, Sk=S)
    tq, tk, tv = up(q), up(k), up(v)
    wsq = torch.empty(qfa.quantize_workspace_bytes(1, 2, S, 128), dtype=torch.uint8, device=DEV)
    wss = torch.empty(qfa.split_workspace_bytes(1, 4, S, 128, 3), dtype=torch.uint8, device=DEV)
    _, keep = _bias2d("bool", 1, 1, S, S, seed=2)    # rows padded to a 16-byte multiple

    def step():
        qk = qfa.quantize_qk(tq, tk, workspace=wsq)
        o_s, l_s = qfa.attn_fwd(qk, tv, w.sm_scale, splits=3, workspace=wss, return_lse=True)
        o_c, l_c = qfa.attn_fwd(qk, tv, w.sm_scale, causal=True, return_lse=True)
        o_u = qfa.attn_fwd_unquant(tq, tk, tv, w.sm_scale, causal=True)
        o_k = qfa.attn_fwd(qk, tv, w.sm_scale, bias=keep)
        return [qk["k8"], qk["qmu"], o_s, l_s, o_c, l_c, o_u, o_k]

    eager = [t.clone() for t in step()]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        outs = step()
    for rep in range(3):
        for t in outs:
            t.zero_()
        step()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for i, (t, e) in enumerate(zip(outs, eager)):
            assert torch.equal(t, e), f"replay {rep}: captured output {i} differs from the eager step"


def test_offsets_past_2_31_elements():
    """B1 H144 S131072 D128 bf16: every tensor holds 2.4e9 elements, so the last heads' element
    offsets pass 2^31. Quantization of heads 0 and 143 is bit-exact against the oracle, and the
    first and last query rows of those heads match it through a 1000-key segment at the end of
    the keys (which keeps the walk short). Inputs: N(0,1) from a seeded torch generator on the
    device, rounded to bf16; the oracle reads the same values copied back."""
    B, H, S, D = 1, 144, 131072, 128
    assert B * H * S * D > 2**31
    free, _ = torch.cuda.mem_get_info(DEV)
    if free < 40 * 2**30:
        pytest.skip("needs 40 GiB of free device memory")
    gen = torch.Generator(device=DEV)
    gen.manual_seed(2**31 + 7)

    def draw():
        x = torch.randn((B, H, S, D), generator=gen, device=DEV, dtype=torch.float32)
        y = x.to(torch.bfloat16)
        del x
        return y

    q, k, v = draw(), draw(), draw()
    g = qfa.quantize_qk(q, k)
    sm = float(np.float32(D ** -0.5))
    seg = [(S - 1000, 1000)]
    o, lse = qfa.attn_fwd(g, v, sm, segments=seg, out_dtype=torch.float32, return_lse=True)
    o16, lse16 = qfa.attn_fwd(g, v, sm, segments=seg, return_lse=True)   # the same instance, bf16 output
    torch.cuda.synchronize()
    rows = np.r_[0:32, S - 32:S]
    assert torch.equal(lse, lse16)
    for h in (0, H - 1):
        check_rne(o16[0, h], o[0, h], f"head {h}")
        qh, kh, vh = (down(t[:, h:h + 1]) for t in (q, k, v))
        ref = oracle.quantize_qk(qh, kh)
        assert_quant_equal({n: g[n][:, h:h + 1] for n in ("q8", "qs", "k8", "ks", "kmean", "qmu")}, ref)
        o_ref, l_ref = oracle.attn(ref, vh, sm, segments=seg, rows=rows)
        check_o(o[0, h], o_ref, rows, f"head {h}")
        check_lse(lse[0, h], l_ref, rows, f"head {h}")
    del q, k, v, g, o, o16, lse, lse16
    torch.cuda.empty_cache()


@pytest.mark.parametrize("kind", ["bf16", "fp16", "fp32", "bool"])
@pytest.mark.parametrize("walk", ["full_461", "full_462", "full_463", "segs_odd", "segs_even"])
def test_key_terms_last_key(kind, walk):
    """Per-key bias / keep mask `[1,1,1,K]`: the last keys of each walked range decide the output
    (biased +8, or the only keys kept besides a few), so a key term lost at the end of a copy
    range shows. Ranges end at odd and even key counts, with and without key segments."""
    w = W.WORKLOADS["tiny"]
    Sk = {"full_461": 461, "full_462": 462, "full_463": 463}.get(walk, 463)
    segs = {"segs_odd": [(5, 121), (200, 61)], "segs_even": [(4, 124), (201, 60)]}.get(walk)
    q, k, v = W.make_qkv(w, H=2, Sq=96, Sk=Sk)
    rs = np.random.default_rng(Sk + len(walk))
    ends = [s0 + n - 1 for s0, n in segs] if segs else [Sk - 1]
    if kind == "bool":
        keep = rs.random(Sk) < 0.05
        for e in ends:
            keep[e - 2:e + 1] = True
        ref_b = np.where(keep, 0.0, -np.inf).astype(np.float32).reshape(1, 1, 1, Sk)
        dev_b = torch.from_numpy(keep.reshape(1, 1, 1, Sk)).to(DEV)
    else:
        vals = (rs.standard_normal(Sk) * 0.5).astype(np.float32)
        for e in ends:
            vals[e] += 8.0
        full = {"fp32": vals, "bf16": W.f32_to_bf16_bits(vals), "fp16": vals.astype(np.float16)}[kind]
        ref_b = full.reshape(1, 1, 1, Sk)
        dev_b = up(ref_b)
    ref = oracle.quantize_qk(q, k)
    o_ref, l_ref = oracle.attn(ref, v, w.sm_scale, bias=ref_b, segments=segs)
    g, tv = gpu_quant(q, k), up(v)
    o, l = both_outputs(lambda dt: qfa.attn_fwd(g, tv, w.sm_scale, bias=dev_b, segments=segs, out_dtype=dt,
                                                return_lse=True), tv.dtype, f"{kind} {walk}")
    check_o(o, o_ref, what=f"{kind} {walk}")
    check_lse(l, l_ref, what=f"{kind} {walk}")


@pytest.mark.parametrize("splits", [1, 2])
def test_nan_rows_past_walked_ranges_never_read(splits):
    """NaN in V after a segment's end inside a visited tile (keys 100..127 and 227..299 for
    segments (0,100), (150,77); keys 128..149 before the second segment's start stay finite,
    as the header requires) leaves the output equal to the oracle's, which never reads them."""
    w = W.WORKLOADS["tiny"]
    Sk = 300
    q, k, v = W.make_qkv(w, H=2, Sq=130, Sk=Sk)
    segs = [(0, 100), (150, 77)]
    ref = oracle.quantize_qk(q, k)
    o_ref, l_ref = oracle.attn(ref, v, w.sm_scale, segments=segs)
    vn = v.copy()
    nan_bits = np.uint16(0x7FC0)   # bf16 quiet NaN
    vn[:, :, 100:128, :] = nan_bits
    vn[:, :, 227:, :] = nan_bits
    g, tvn = gpu_quant(q, k), up(vn)
    o, l = both_outputs(lambda dt: qfa.attn_fwd(g, tvn, w.sm_scale, segments=segs, splits=splits, out_dtype=dt,
                                                return_lse=True), tvn.dtype, f"splits {splits}")
    check_o(o, o_ref, what=f"segments, splits {splits}")
    check_lse(l, l_ref, what=f"segments, splits {splits}")


def test_nan_pad_rows_block_sparse():
    """Block-sparse: NaN in the pad rows (j mod 64 >= vbs) of Q, K and V; quantization gives
    their codes 0 / scale 0 and leaves them out of the K mean, and the V copies stop at vbs, so
    the output equals the oracle's on the same inputs with zero pad rows."""
    w = W.WORKLOADS["sparse"]
    S, H = 512, 2
    T = S // 64
    q, k, v = W.make_qkv(w, H=H, Sq=S, Sk=S)
    vbs = np.array([64, 17, 0, 40, 64, 1, 63, 17], np.int32)
    for x in (q, k, v):
        W.zero_pads(x, vbs)
    mask = np.random.default_rng(5).random((1, H, T, T)) < 0.7
    ref = oracle.quantize_qk(q, k, vbs)
    o_ref, l_ref = oracle.attn(ref, v, w.sm_scale, mask=mask.astype(np.uint8), vbs=vbs)
    j = np.arange(S)
    pad = (j % 64) >= vbs[j // 64]
    qn, kn, vn = q.copy(), k.copy(), v.copy()
    for x in (qn, kn, vn):
        x[:, :, pad, :] = np.uint16(0x7FC0)
    g = qfa.quantize_qk(up(qn), up(kn), up(vbs))
    idx, cnt = qfa.blockmask_to_index(up(mask))
    tvn, tvbs = up(vn), up(vbs)
    o, l = both_outputs(lambda dt: qfa.attn_fwd(g, tvn, w.sm_scale, index=idx, count=cnt, vbs=tvbs, out_dtype=dt,
                                                return_lse=True), tvn.dtype, "sparse pads NaN")
    valid_rows = np.flatnonzero(~np.tile(pad, H))
    check_o(o, o_ref[valid_rows], valid_rows, "sparse pads NaN")
    check_lse(l, l_ref[valid_rows], valid_rows, "sparse pads NaN")


def test_quantize_non_finite_rows():
    """Non-finite Q/K values: rows holding NaN or +-inf get codes 0, scale NaN (and a NaN centring
    term for Q); an inf among a K channel's valid keys makes that channel's mean NaN, so every
    centred row of that K/V head gets scale NaN; heads without one are unaffected. Bit-exact
    against the oracle, NaN positions included, for bf16 and fp16."""
    w = W.WORKLOADS["d64"]
    for dt in ("bf16", "fp16"):
        q, k, _ = W.make_qkv(w, B=1, H=4, Hkv=2, Sq=200, Sk=300)
        qf, kf = W.to_f32(q), W.to_f32(k)
        qf[0, 0, 3, 5] = np.nan
        qf[0, 1, 7, 0] = np.inf
        qf[0, 3, 199, 63] = -np.inf
        kf[0, 1, 17, 9] = np.inf        # K/V head 1: mean of channel 9 is NaN
        conv = W.f32_to_bf16_bits if dt == "bf16" else (lambda x: x.astype(np.float16))
        q2, k2 = conv(qf), conv(kf)
        g = gpu_quant(q2, k2)
        ref = oracle.quantize_qk(q2, k2)
        for name in ("q8", "qs", "k8", "ks", "kmean"):
            a, b = down(g[name]), ref[name]
            assert np.array_equal(a, b, equal_nan=a.dtype.kind == "f"), f"{dt} {name}"
        # the centring term: NaN on the same rows, the finite ones within the usual bound
        assert np.array_equal(np.isnan(down(g["qmu"])), np.isnan(ref["qmu"])), f"{dt} qmu"
        assert np.isnan(ref["qs"][0, 0, 3]) and np.isnan(ref["qs"][0, 1, 7]) and np.isnan(ref["qs"][0, 3, 199])
        assert np.all(np.isnan(ref["ks"][0, 1])) and np.all(np.isfinite(ref["ks"][0, 0]))
        fin = np.isfinite(ref["qmu"])
        assert np.max(np.abs(down(g["qmu"])[fin] - ref["qmu"][fin])) <= 1e-4 * max(1.0, np.abs(ref["qmu"][fin]).max())


def test_debug_log_names_the_instance():
    """QFA_DEBUG=1 prints one line per launch naming the kernel instance and its grid."""
    import subprocess
    import sys
    code = ("import torch, quantized_flash_attention_amd as qfa\n"
            "q = torch.randn(1, 2, 300, 128, device='cuda').to(torch.bfloat16)\n"
            "g = qfa.quantize_qk(q, q)\n"
            "qfa.attn_fwd(g, q, 0.088, return_lse=True, causal=True)\n"
            "torch.cuda.synchronize()\n")
    env = dict(os.environ, QFA_DEBUG="1")
    r = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True, timeout=300,
                       cwd=os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [x for x in r.stderr.splitlines() if x.startswith("qfa: ")]
    assert any("kmean_partial_kernel<bf16, D=128>" in x for x in lines), lines
    assert any("quantize_kernel<bf16, D=128>" in x for x in lines), lines
    assert any("attn_fwd_kernel<D=128, V=bf16, sparse=0, bias=0, lse=1, causal=1, qk=int8" in x and "grid 6 x 256" in x
               for x in lines), lines


def test_quantize_into_caller_outputs():
    """quantize_qk(out=...) writes the same bytes into caller-provided (previously garbage-filled)
    tensors as the allocating call, centred and uncentred, and a second call into the same tensors
    overwrites every element."""
    w = W.WORKLOADS["dense4k"]
    q, k, _ = W.make_qkv(w, H=4, Hkv=2, Sq=333, Sk=517)
    tq, tk = up(q), up(k)
    for center in (True, False):
        ref = qfa.quantize_qk(tq, tk, center_k=center)
        out = {n: None if t is None else torch.full_like(t, 77 if t.dtype == torch.int8 else float("nan"))
               for n, t in ref.items()}
        for _ in range(2):
            got = qfa.quantize_qk(tq, tk, center_k=center, out=out)
            for n, t in ref.items():
                assert (t is None) == (got[n] is None), n
                if t is not None:
                    assert got[n].data_ptr() == out[n].data_ptr(), n
                    assert torch.equal(got[n].view(torch.int8) if t.dtype == torch.int8 else got[n].view(torch.int32),
                                       t.view(torch.int8) if t.dtype == torch.int8 else t.view(torch.int32)), n
        assert_quant_equal(got, oracle.quantize_qk(q, k, center_k=center), center)


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
def test_kmean_wide_exponent_spans(dtype):
    """K-mean exactness where the kernel's plain fp64 sum is not certified exact: channels mixing values
    near 2^30 (bf16) or 6e4 (fp16) with values near 2^-60 (bf16) or subnormal fp16, exact zeros and a
    bf16 subnormal (12 chunks of 250 rows per head, lanes holding both extremes); the kernel's
    double-double path for such lanes must reproduce the oracle's exact mean bit for bit."""
    w = W.WORKLOADS["dense4k"]
    q, k, _ = W.make_qkv(w, H=3, Sq=64, Sk=3000)
    kf = W.to_f32(k)
    rs = np.random.default_rng(31)
    if dtype == "bf16":
        kf[0, 0, ::7, 3] *= np.float32(2.0 ** 30)
        kf[0, 0, 1::7, 3] *= np.float32(2.0 ** -60)
        kf[0, 1, :, 5] = 0.0
        kf[0, 1, 17, 5] = np.float32(2.0 ** -130)          # a subnormal
        kf[0, 2, rs.integers(0, 3000, 40), 9] *= np.float32(2.0 ** -40)
        k2, q2 = W.f32_to_bf16_bits(kf), q
    else:
        kf[0, 0, ::7, 3] = 60000.0
        kf[0, 0, 1::7, 3] = np.float32(2.0 ** -24)          # the smallest fp16 subnormal
        kf[0, 1, :, 5] = 0.0
        k2, q2 = kf.astype(np.float16), W.to_f32(q).astype(np.float16)
    g = gpu_quant(q2, k2)
    assert_quant_equal(g, oracle.quantize_qk(q2, k2))
