"""Property-based pins of the oracle's masking (hypothesis): on random small shapes with random
key segments, causal masks, block-sparse tile masks with validity vectors, per-key or per-query
additive biases (with -inf entries) and grouped-query heads, the oracle's no-quant attention
equals torch's fp64 SDPA given the same exclusions written out as one dense additive mask, and
its LSE equals torch.logsumexp of the masked logits. Rows with nothing attended give O = 0 and
LSE = -inf (SDPA has no defined output there)."""
import math

import numpy as np
import pytest
import torch
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

import oracle


@st.composite
def configs(draw):
    D = draw(st.sampled_from([64, 128]))
    B = draw(st.integers(1, 2))
    Hkv = draw(st.integers(1, 2))
    H = Hkv * draw(st.integers(1, 2))
    sparse = draw(st.booleans())
    if sparse:
        T = draw(st.integers(1, 4))
        Sq = Sk = 64 * T
    else:
        Sq = draw(st.integers(1, 300))
        Sk = Sq if draw(st.booleans()) else draw(st.integers(1, 300))
    causal = (not sparse) and Sq == Sk and draw(st.booleans())
    segments = None
    if not sparse and draw(st.booleans()):
        cuts = sorted(draw(st.lists(st.integers(0, Sk), min_size=2, max_size=8, unique=True)))
        segs = [(cuts[i], cuts[i + 1] - cuts[i]) for i in range(0, len(cuts) - 1, 2)][:4]
        segments = segs or None
    bias_kind = draw(st.sampled_from(["none", "key", "query"])) if not sparse else "none"
    seed = draw(st.integers(0, 2**31 - 1))
    return dict(B=B, H=H, Hkv=Hkv, Sq=Sq, Sk=Sk, D=D, sparse=sparse, causal=causal, segments=segments,
                bias_kind=bias_kind, seed=seed)


@settings(max_examples=150, deadline=None, suppress_health_check=[HealthCheck.too_slow])
@given(configs())
def test_noquant_matches_sdpa_with_dense_mask(c):
    rs = np.random.default_rng(c["seed"])
    B, H, Hkv, Sq, Sk, D = c["B"], c["H"], c["Hkv"], c["Sq"], c["Sk"], c["D"]
    q = rs.standard_normal((B, H, Sq, D))
    k = rs.standard_normal((B, Hkv, Sk, D))
    v = rs.standard_normal((B, Hkv, Sk, D)).astype(np.float32)
    scale = float(np.float32(D ** -0.5))             # the oracle takes the softmax scale in fp32
    add = np.zeros((B, H, Sq, Sk))                     # the dense additive mask, written out here
    kw = {}
    if c["segments"]:
        keep = np.zeros(Sk, bool)
        for s0, n in c["segments"]:
            keep[s0:s0 + n] = True
        add[..., ~keep] = -np.inf
        kw["segments"] = c["segments"]
    if c["causal"]:
        add[..., np.triu(np.ones((Sq, Sk), bool), 1)] = -np.inf
        kw["causal"] = True
    if c["sparse"]:
        T = Sk // 64
        mask = rs.random((B, H, T, T)) < 0.6
        vbs = rs.integers(0, 65, size=T).astype(np.int32)
        tile_ok = np.repeat(np.repeat(mask, 64, axis=2), 64, axis=3)
        key_ok = (np.arange(Sk) % 64) < np.repeat(vbs, 64)
        add[~(tile_ok & key_ok[None, None, None, :])] = -np.inf
        kw.update(mask=mask.astype(np.uint8), vbs=vbs)
    if c["bias_kind"] != "none":
        shape = (1, 1, 1, Sk) if c["bias_kind"] == "key" else (B, H, Sq, Sk)
        bias = (rs.standard_normal(shape) * 2).astype(np.float32)
        bias[rs.random(shape) < 0.1] = -np.inf
        add = add + bias
        kw["bias"] = bias
    o, lse = oracle.attn(None, v, scale, q=q, k=k, **kw)
    o = o.reshape(B, H, Sq, D)
    lse = lse.reshape(B, H, Sq)

    g = H // Hkv
    qt = torch.tensor(q)
    kt = torch.tensor(k).repeat_interleave(g, dim=1)
    vt = torch.tensor(v, dtype=torch.float64).repeat_interleave(g, dim=1)
    logits = scale * torch.matmul(qt, kt.transpose(-1, -2).contiguous()) + torch.tensor(add)
    ref_lse = torch.logsumexp(logits, dim=-1).numpy()
    live = np.isfinite(ref_lse)
    assert np.array_equal(np.isneginf(lse), ~live)
    assert np.all(o[~live] == 0)
    if live.any():
        ref_o = torch.nn.functional.scaled_dot_product_attention(
            qt, kt, vt, attn_mask=torch.tensor(add), scale=scale).numpy()
        assert np.max(np.abs(o[live] - ref_o[live])) < 1e-10
        assert np.max(np.abs(lse[live] - ref_lse[live])) < 1e-10
