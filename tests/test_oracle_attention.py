"""Pins of the oracle's attention, LSE, merge and tile-index steps.

Independent references: torch's scaled_dot_product_attention and logsumexp
run in float64 on the CPU (library routines), numpy's nonzero, and closed
forms / identities the method fixes (Sk = 1, Q = 0, fully masked rows, a
constant bias, the shift invariance of K centring, broadcast == expanded
bias, block-sparse == dense with -inf bias, split + merge == unsplit).
"""
import math

import numpy as np
import pytest
import torch

import workloads as W


def _sdpa64(q, k, v, scale, mask=None, is_causal=False):
    """fp64 CPU SDPA and its log-sum-exp, the library reference for no-quant attention. K/V with
    fewer heads than Q use torch's grouped-query mode (``enable_gqa``), and the log-sum-exp
    reads K through ``repeat_interleave``, torch's statement of the same head grouping."""
    qt = torch.tensor(W.to_f32(q), dtype=torch.float64)
    kt = torch.tensor(W.to_f32(k), dtype=torch.float64)
    vt = torch.tensor(W.to_f32(v), dtype=torch.float64)
    m = None if mask is None else torch.tensor(mask, dtype=torch.float64)
    gqa = kt.shape[1] != qt.shape[1]
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=m, scale=scale, is_causal=is_causal,
                                                         enable_gqa=gqa)
    if gqa:
        kt = kt.repeat_interleave(qt.shape[1] // kt.shape[1], dim=1)
    s = scale * torch.matmul(qt, kt.transpose(-1, -2).contiguous())
    if m is not None:
        s = s + m
    if is_causal:
        s = s.masked_fill(torch.ones(s.shape[-2:], dtype=torch.bool).triu(1), -math.inf)
    lse = torch.logsumexp(s, dim=-1)
    return o.numpy(), lse.numpy()


def _small(name="tiny", **kw):
    w = W.WORKLOADS[name]
    return w, W.make_qkv(w, **kw)


def test_noquant_matches_sdpa(oracle_lib):
    w, (q, k, v) = _small(Sq=96, Sk=160)
    o, lse = oracle_lib.attn(None, v, w.sm_scale, q=W.to_f32(q), k=W.to_f32(k))
    ro, rl = _sdpa64(q, k, v, w.sm_scale)
    assert np.max(np.abs(o - ro.reshape(-1, 128))) < 1e-12
    assert np.max(np.abs(lse - rl.reshape(-1))) < 1e-12


def test_noquant_causal_matches_sdpa(oracle_lib):
    # self-attention with the key range ending at each row (torch's is_causal)
    w, (q, k, v) = _small(Sq=160, Sk=160)
    o, lse = oracle_lib.attn(None, v, w.sm_scale, q=W.to_f32(q), k=W.to_f32(k), causal=True)
    ro, rl = _sdpa64(q, k, v, w.sm_scale, is_causal=True)
    assert np.max(np.abs(o - ro.reshape(-1, 128))) < 1e-12
    assert np.max(np.abs(lse - rl.reshape(-1))) < 1e-12


@pytest.mark.parametrize("hkv,causal", [(2, False), (1, False), (2, True)])
def test_noquant_gqa_matches_sdpa(oracle_lib, hkv, causal):
    # grouped-query attention: 4 query heads over hkv K/V heads, head h reading K/V head
    # h // (4 // hkv), against torch's SDPA in its grouped-query mode
    w = W.WORKLOADS["tiny"]
    q, k, v = W.make_qkv(w, H=4, Hkv=hkv, Sq=160, Sk=160)
    assert k.shape[1] == hkv and v.shape[1] == hkv
    o, lse = oracle_lib.attn(None, v, w.sm_scale, q=W.to_f32(q), k=W.to_f32(k), causal=causal)
    ro, rl = _sdpa64(q, k, v, w.sm_scale, is_causal=causal)
    assert np.max(np.abs(o - ro.reshape(-1, 128))) < 1e-12
    assert np.max(np.abs(lse - rl.reshape(-1))) < 1e-12


def test_quantized_gqa_equals_repeated_kv(oracle_lib):
    # quantized mode: K/V heads shared by runs of query heads give exactly what multi-head
    # attention gives on K/V (and V scale) repeated per query head: the K mean and K codes are
    # per K/V head, and each query row's centring term uses its K/V head's mean
    w = W.WORKLOADS["dense4k"]          # per-channel K offset: a nonzero mean per K/V head
    H, hkv, S = 6, 2, 200
    q, k, v = W.make_qkv(w, H=H, Hkv=hkv, Sq=S, Sk=S)
    g = H // hkv
    k_rep, v_rep = np.repeat(k, g, axis=1), np.repeat(v, g, axis=1)
    vsc = W.v_scale(w, H=hkv)
    qk = oracle_lib.quantize_qk(q, k)
    qk_rep = oracle_lib.quantize_qk(q, k_rep)
    for name in ("k8", "ks", "kmean"):
        assert np.array_equal(np.repeat(qk[name], g, axis=1), qk_rep[name]), name
    for name in ("q8", "qs", "qmu"):
        assert np.array_equal(qk[name], qk_rep[name]), name
    bias = W.bias_tensor(W.band_bias(S, core=(40, 120), skirt=40), "fp32")
    for causal in (False, True):
        o, l = oracle_lib.attn(qk, v, w.sm_scale, bias=bias, v_scale=vsc, causal=causal)
        o_r, l_r = oracle_lib.attn(qk_rep, v_rep, w.sm_scale, bias=bias, v_scale=np.repeat(vsc, g, axis=0),
                                   causal=causal)
        assert np.array_equal(o, o_r) and np.array_equal(l, l_r)
    with pytest.raises(ValueError):
        oracle_lib.attn(qk, v[:, :1].repeat(4, axis=1), w.sm_scale)   # 6 query heads over 4


def test_causal_equals_triangular_bias(oracle_lib):
    # quantized mode: the causal exclusion and a materialised 0 / -inf upper-triangular bias are
    # two code paths to one definition; row 0 sees key 0 alone, so its output is V[0] exactly
    w, (q, k, v) = _small(Sq=200, Sk=200)
    qk = oracle_lib.quantize_qk(q, k)
    tri = np.where(np.triu(np.ones((200, 200), bool), 1), -np.inf, 0.0).astype(np.float32).reshape(1, 1, 200, 200)
    o_c, l_c = oracle_lib.attn(qk, v, w.sm_scale, causal=True)
    o_b, l_b = oracle_lib.attn(qk, v, w.sm_scale, bias=tri)
    assert np.array_equal(o_c, o_b) and np.array_equal(l_c, l_b)
    v0 = W.to_f32(v)[0, :, 0, :].astype(np.float64)     # [H, D]
    assert np.array_equal(o_c.reshape(1, 2, 200, 128)[0, :, 0, :], v0)
    with pytest.raises(ValueError):
        oracle_lib.attn(qk, v[:, :, :100], w.sm_scale, causal=True)


def test_noquant_full_bias_matches_sdpa(oracle_lib):
    # a materialised [B,H,Q,K] bias with distinct values per (h, i, j) pins bias indexing
    w, (q, k, v) = _small(Sq=64, Sk=96)
    rs = np.random.default_rng(5)
    bias = rs.standard_normal((1, 2, 64, 96)).astype(np.float32)
    bias[0, 1, 3, :50] = -np.inf
    o, lse = oracle_lib.attn(None, v, w.sm_scale, q=W.to_f32(q), k=W.to_f32(k), bias=bias)
    ro, rl = _sdpa64(q, k, v, w.sm_scale, bias.astype(np.float64))
    assert np.max(np.abs(o - ro.reshape(-1, 128))) < 1e-12
    assert np.max(np.abs(lse - rl.reshape(-1))) < 1e-12


def test_noquant_segments_and_sparse_match_sdpa(oracle_lib):
    w, (q, k, v) = _small(Sq=192, Sk=256)
    segs = [(0, 40), (100, 77)]
    o, lse = oracle_lib.attn(None, v, w.sm_scale, q=W.to_f32(q), k=W.to_f32(k), segments=segs)
    m = np.full((192, 256), -np.inf)
    for s0, n in segs:
        m[:, s0:s0 + n] = 0
    ro, rl = _sdpa64(q, k, v, w.sm_scale, m)
    assert np.max(np.abs(o - ro.reshape(-1, 128))) < 1e-12
    assert np.max(np.abs(lse - rl.reshape(-1))) < 1e-12
    # tile-64 mask with a validity vector (Sq = Sk = 256: 4 tiles)
    w2, (q2, k2, v2) = _small(Sq=256, Sk=256)
    mask = np.zeros((1, 2, 4, 4), np.uint8)
    mask[0, 0] = [[1, 0, 0, 1], [1, 1, 0, 0], [0, 0, 0, 0], [1, 1, 1, 1]]
    mask[0, 1] = [[0, 1, 1, 0], [1, 0, 0, 1], [1, 1, 1, 1], [0, 0, 0, 1]]
    vbs = np.array([64, 30, 64, 7], np.int32)
    o, lse = oracle_lib.attn(None, v2, w2.sm_scale, q=W.to_f32(q2), k=W.to_f32(k2), mask=mask, vbs=vbs)
    dense = np.full((1, 2, 256, 256), -np.inf)
    for h in range(2):
        for t in range(4):
            for u in range(4):
                if mask[0, h, t, u]:
                    dense[0, h, 64 * t:64 * t + 64, 64 * u:64 * u + vbs[u]] = 0
    rows_live = np.isfinite(dense).any(-1).reshape(-1)
    ro, rl = _sdpa64(q2, k2, v2, w2.sm_scale, np.where(np.isfinite(dense), dense, -1e300))
    assert np.max(np.abs(o[rows_live] - ro.reshape(-1, 128)[rows_live])) < 1e-12
    assert np.max(np.abs(lse[rows_live] - rl.reshape(-1)[rows_live])) < 1e-9
    # fully masked query tile (head 0, tile 2): O = 0, LSE = -inf
    dead = ~rows_live
    assert dead.sum() == 64
    assert np.all(o[dead] == 0) and np.all(lse[dead] == -np.inf)


def test_quantized_accuracy_model_kernels_recipe(oracle_lib):
    """fp16 [1,8,64,64] N(0,1) against SDPA: mean error must sit far below the
    failure signature (0.168 mean / 1.69 max) and within ~1e-2 as expected
    there for int8 attention (model-kernels issue #3, accuracy section)."""
    rs = np.random.default_rng(2024)
    q, k, v = (rs.standard_normal((1, 8, 64, 64)).astype(np.float16) for _ in range(3))
    scale = float(np.float32(64 ** -0.5))
    qk = oracle_lib.quantize_qk(q, k)
    o, lse = oracle_lib.attn(qk, v, scale)
    ro, rl = _sdpa64(q, k, v, scale)
    err = np.abs(o - ro.reshape(-1, 64))
    assert err.mean() < 1e-2 and err.max() < 0.1
    assert np.max(np.abs(lse - rl.reshape(-1))) < 2e-2


def test_quantized_with_offset_k_tracks_exact(oracle_lib):
    # K with a large per-channel offset: centring keeps the int8 error small and
    # the qmu term puts the LSE back on the uncentred scores
    w, (q, k, v) = _small("dense4k", H=2, Sq=128, Sk=192)
    qk = oracle_lib.quantize_qk(q, k)
    o, lse = oracle_lib.attn(qk, v, w.sm_scale)
    ro, rl = _sdpa64(q, k, v, w.sm_scale)
    assert np.abs(o - ro.reshape(-1, 128)).mean() < 2e-3
    assert np.max(np.abs(lse - rl.reshape(-1))) < 2e-2
    # without the centring term the LSE is off by sm_scale*q.mu (several nats here)
    _, lse_nc = oracle_lib.attn(qk, v, w.sm_scale, use_qmu=False)
    assert np.max(np.abs(lse_nc - rl.reshape(-1))) > 1.0


def test_single_key_closed_form(oracle_lib):
    w, (q, k, v) = _small(Sq=8, Sk=1)
    rs = np.random.default_rng(1)
    bias = rs.standard_normal((1, 1, 1, 1)).astype(np.float32)
    vs = rs.uniform(0.5, 2, (2, 128)).astype(np.float32)
    qk = oracle_lib.quantize_qk(q, k)
    o, lse = oracle_lib.attn(qk, v, w.sm_scale, bias=bias, v_scale=vs)
    vf = W.to_f32(v).astype(np.float64)
    for h in range(2):
        assert np.allclose(o[8 * h:8 * h + 8], (vf[0, h, 0] * vs[h])[None], rtol=0, atol=1e-12)
    # one key: LSE is that key's true logit; the centred K is all zero so it comes
    # entirely from the centring term (mean of a single row is the row itself)
    s = w.sm_scale * (W.to_f32(q).astype(np.float64) @ W.to_f32(k).astype(np.float64).transpose(0, 1, 3, 2))
    want = s.reshape(-1) + float(bias.reshape(-1)[0])
    assert np.max(np.abs(lse - want)) < 1e-9


def test_zero_query_closed_form(oracle_lib):
    w, (q, k, v) = _small(Sq=4, Sk=100)
    q = np.zeros_like(q)
    qk = oracle_lib.quantize_qk(q, k)
    segs = [(10, 30), (60, 15)]
    o, lse = oracle_lib.attn(qk, v, w.sm_scale, segments=segs)
    vf = W.to_f32(v).astype(np.float64)
    idx = np.r_[10:40, 60:75]
    for h in range(2):
        assert np.allclose(o[4 * h:4 * h + 4], vf[0, h, idx].mean(0)[None], rtol=0, atol=1e-12)
    assert np.allclose(lse, math.log(45), rtol=0, atol=1e-12)


def test_fully_masked_rows(oracle_lib):
    w, (q, k, v) = _small(Sq=8, Sk=64)
    qk = oracle_lib.quantize_qk(q, k)
    bias = np.full((1, 1, 1, 64), -np.inf, np.float32)
    o, lse = oracle_lib.attn(qk, v, w.sm_scale, bias=bias)
    assert np.all(o == 0) and np.all(lse == -np.inf) and not np.isnan(o).any()
    o, lse = oracle_lib.attn(qk, v, w.sm_scale, segments=[(5, 0)])
    assert np.all(o == 0) and np.all(lse == -np.inf)


def test_constant_bias_shifts_lse_only(oracle_lib):
    w, (q, k, v) = _small(Sq=32, Sk=96)
    qk = oracle_lib.quantize_qk(q, k)
    o0, l0 = oracle_lib.attn(qk, v, w.sm_scale)
    o1, l1 = oracle_lib.attn(qk, v, w.sm_scale, bias=np.full((1, 1, 1, 96), -3.25, np.float32))
    assert np.max(np.abs(o1 - o0)) < 1e-12
    assert np.max(np.abs(l1 - (l0 - 3.25))) < 1e-12


def test_k_shift_invariance(oracle_lib):
    """K -> K + 1 c^T leaves O unchanged and moves the LSE by sm_scale * q.c
    (the centring step is a softmax-invariant shift: FastVideo docs, module description)."""
    w, (q, k, v) = _small(Sq=64, Sk=128)
    c = W.f32_to_bf16_bits(np.linspace(-4, 4, 128, dtype=np.float32))
    cf = W.bf16_bits_to_f32(c).astype(np.float64)
    kf = W.to_f32(k).astype(np.float64)
    # no-quant: exact identities
    o0, l0 = oracle_lib.attn(None, v, w.sm_scale, q=W.to_f32(q), k=kf)
    o1, l1 = oracle_lib.attn(None, v, w.sm_scale, q=W.to_f32(q), k=kf + cf)
    shift = w.sm_scale * (W.to_f32(q).astype(np.float64) @ cf).reshape(-1)
    assert np.max(np.abs(o1 - o0)) < 1e-12
    assert np.max(np.abs(l1 - l0 - shift)) < 1e-10
    # quantized with centring: the shifted K (rounded to bf16) gives nearly the same O and LSE + shift
    k_shift = W.f32_to_bf16_bits((kf + cf).astype(np.float32))
    qa, qb = oracle_lib.quantize_qk(q, k), oracle_lib.quantize_qk(q, k_shift)
    oa, la = oracle_lib.attn(qa, v, w.sm_scale)
    ob, lb = oracle_lib.attn(qb, v, w.sm_scale)
    assert np.abs(ob - oa).mean() < 2e-3
    assert np.max(np.abs(lb - la - shift)) < 2e-2


def test_broadcast_bias_equals_expanded(oracle_lib):
    """A [1,1,1,K] bias and its materialised [1,1,Q,K] expansion give identical results
    (comfy-kitchen issue #177, measurement table and first observation)."""
    w, (q, k, v) = _small(Sq=64, Sk=200)
    qk = oracle_lib.quantize_qk(q, k)
    b = W.bias_tensor(W.band_bias(200, core=(60, 80), skirt=60), "bf16")
    expanded = np.ascontiguousarray(np.broadcast_to(b, (1, 1, 64, 200)))
    o1, l1 = oracle_lib.attn(qk, v, w.sm_scale, bias=b)
    o2, l2 = oracle_lib.attn(qk, v, w.sm_scale, bias=expanded)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def test_sparse_equals_dense_with_neg_inf_bias(oracle_lib):
    w, (q, k, v) = _small(Sq=256, Sk=256)
    vbs = np.array([64, 64, 64, 23], np.int32)
    W.zero_pads(q, vbs), W.zero_pads(k, vbs), W.zero_pads(v, vbs)
    mask = W.sparse_mask(4, 2, prefix=1, band=1)
    qk = oracle_lib.quantize_qk(q, k, vbs)
    o1, l1 = oracle_lib.attn(qk, v, w.sm_scale, mask=mask, vbs=vbs)
    bias = np.zeros((1, 2, 256, 256), np.float32)
    for h in range(2):
        for t in range(4):
            for u in range(4):
                if not mask[0, h, t, u]:
                    bias[0, h, 64 * t:64 * t + 64, 64 * u:64 * u + 64] = -np.inf
    bias[..., (np.arange(256) % 64) >= vbs[np.arange(256) // 64]] = -np.inf
    o2, l2 = oracle_lib.attn(qk, v, w.sm_scale, bias=bias)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def test_v_scale_equals_scaled_v(oracle_lib):
    w, (q, k, v) = _small(Sq=32, Sk=80)
    vs = W.v_scale(w, H=2)
    qk = oracle_lib.quantize_qk(q, k)
    o1, l1 = oracle_lib.attn(qk, v, w.sm_scale, v_scale=vs)
    vscaled = (W.to_f32(v).astype(np.float64) * vs[None, :, None, :]).astype(np.float32)
    o2, l2 = oracle_lib.attn(qk, vscaled, w.sm_scale)
    assert np.max(np.abs(o1 - o2)) < 1e-6 and np.array_equal(l1, l2)


@pytest.mark.parametrize("quant", [False, True])
def test_split_merge_equals_unsplit(oracle_lib, quant):
    """core (unmasked) + skirt (masked) calls merged by LSE == one masked call
    (comfy-kitchen issue #177, Question 2)."""
    w, (q, k, v) = _small(Sq=64, Sk=336)
    core, skirt = (72, 192), 72
    bias64 = W.band_bias(336, core=core, skirt=skirt)
    bias = W.bias_tensor(bias64, "fp32")
    kw = dict(q=W.to_f32(q), k=W.to_f32(k)) if not quant else {}
    qk = oracle_lib.quantize_qk(q, k) if quant else None
    o_full, l_full = oracle_lib.attn(qk, v, w.sm_scale, bias=bias, **kw)
    o_core, l_core = oracle_lib.attn(qk, v, w.sm_scale, segments=[core], **kw)
    o_sk, l_sk = oracle_lib.attn(qk, v, w.sm_scale, bias=bias, segments=[(0, 72), (264, 72)], **kw)
    o_m, l_m = oracle_lib.lse_merge(o_core, l_core, o_sk, l_sk)
    assert np.max(np.abs(o_m - o_full)) < 1e-12
    assert np.max(np.abs(l_m - l_full)) < 1e-12
    # commutative, and matches torch's logaddexp for the LSE
    o_r, l_r = oracle_lib.lse_merge(o_sk, l_sk, o_core, l_core)
    assert np.max(np.abs(o_r - o_m)) < 1e-15 and np.array_equal(l_r, l_m)
    assert np.max(np.abs(l_m - torch.logaddexp(torch.tensor(l_core), torch.tensor(l_sk)).numpy())) < 1e-12


def test_merge_identities(oracle_lib):
    rs = np.random.default_rng(9)
    oa, ob, oc = (rs.standard_normal((10, 16)) for _ in range(3))
    la, lb, lc = (rs.standard_normal(10) * 3 for _ in range(3))
    # (-inf) partial is the identity
    o, l = oracle_lib.lse_merge(oa, la, np.zeros_like(oa), np.full(10, -np.inf))
    assert np.array_equal(o, oa) and np.array_equal(l, la)
    o, l = oracle_lib.lse_merge(np.zeros_like(oa), np.full(10, -np.inf), np.zeros_like(oa), np.full(10, -np.inf))
    assert np.all(o == 0) and np.all(l == -np.inf)
    # associative
    o1, l1 = oracle_lib.lse_merge(*oracle_lib.lse_merge(oa, la, ob, lb), oc, lc)
    o2, l2 = oracle_lib.lse_merge(oa, la, *oracle_lib.lse_merge(ob, lb, oc, lc))
    assert np.max(np.abs(o1 - o2)) < 1e-12 and np.max(np.abs(l1 - l2)) < 1e-12
    # weights: O = (e^la oa + e^lb ob) / (e^la + e^lb)
    o, l = oracle_lib.lse_merge(oa, la, ob, lb)
    wa, wb = np.exp(la)[:, None], np.exp(lb)[:, None]
    assert np.max(np.abs(o - (wa * oa + wb * ob) / (wa + wb))) < 1e-12


def test_blockmask_to_index_matches_nonzero(oracle_lib):
    rs = np.random.default_rng(4)
    mask = rs.random((2, 3, 17, 40)) < 0.3
    mask[0, 0, 0] = False
    mask[1, 2, 5] = True
    index, count = oracle_lib.blockmask_to_index(mask)
    for b in range(2):
        for h in range(3):
            for t in range(17):
                nz = np.nonzero(mask[b, h, t])[0]
                assert count[b, h, t] == len(nz)
                assert index[b, h, t, :len(nz)].tolist() == nz.tolist()


def test_sparse_workload_structure():
    # tile pairs per head of the 2048-tile band+prefix mask (a property of the input, checked by counting)
    m = W.sparse_mask(2048, 1)
    assert int(m.sum()) == 212268
    v = W.sparse_vbs(2048)
    assert int(v.sum()) == 131025
