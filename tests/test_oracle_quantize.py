"""Pins of the oracle's K mean, per-token int8 quantization, centring term and int32 scores.

Every expected value here comes from something other than the oracle's own
code: hand-worked cases (tests/golden/quantize_hand.json), exact rational
arithmetic (fractions.Fraction), brute-force Python integers, or invariants
the quantizer definition implies.
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest

import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "quantize_hand.json")


def _f32_of_fraction(fr: Fraction) -> np.float32:
    # nearest fp32 to an exact rational: round to fp64 first (53 bits) and
    # check that this cannot have crossed an fp32 rounding boundary
    d = float(fr)
    f = np.float32(d)
    lo, hi = np.nextafter(f, np.float32(-np.inf)), np.nextafter(f, np.float32(np.inf))
    assert abs(Fraction(float(f)) - fr) <= min(abs(Fraction(float(lo)) - fr), abs(Fraction(float(hi)) - fr))
    return f


def test_hand_worked_quantization(oracle_lib):
    g = json.load(open(GOLDEN))
    for case in g["cases"]:
        x = np.array(case["x"], np.float32).reshape(1, 1, 1, -1)
        q8, qs = oracle_lib.quantize_rows(x)
        assert q8.reshape(-1).tolist() == case["q"], case["name"]
        want = _f32_of_fraction(Fraction(case["scale_num"], case["scale_den"]))
        assert qs.reshape(-1)[0] == want, case["name"]


def test_hand_worked_centring(oracle_lib):
    c = json.load(open(GOLDEN))["centring_case"]
    k = np.array(c["k"], np.float32).reshape(1, 1, 2, 2)
    mu = oracle_lib.kmean(k)
    assert mu.reshape(-1).tolist() == c["mean"]
    k8, ks = oracle_lib.quantize_rows(k, mu)
    assert k8.reshape(2, 2).tolist() == c["k8"]
    assert np.all(ks == _f32_of_fraction(Fraction(c["ks_num"], c["ks_den"])))
    # Q is never centred: the same rows quantize without the shift
    q8, _ = oracle_lib.quantize_rows(k)
    assert q8.reshape(2, 2).tolist() != c["k8"]


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
def test_kmean_is_exact_rational_mean(oracle_lib, dtype):
    # B1 H2 S300 D8 with values spread over many binades, including a vbs-free and a vbs case
    rs = np.random.default_rng(7)
    x = rs.standard_normal((1, 2, 300, 8)).astype(np.float32) * np.float32(2.0) ** rs.integers(-12, 8, (1, 2, 300, 8))
    if dtype == "fp16":
        x = np.clip(x, -60000, 60000)
    arr = W.f32_to_bf16_bits(x) if dtype == "bf16" else x.astype(np.float16)
    xf = W.to_f32(arr).astype(np.float64)
    mu = oracle_lib.kmean(arr)
    for h in range(2):
        for c in range(8):
            exact = sum((Fraction(float(v)) for v in xf[0, h, :, c]), Fraction(0))
            want = np.float32(float(Fraction(float(exact)) / 300))  # round sum to fp64, fp64 divide, round to fp32
            assert mu[0, h, c] == want
    # with a validity vector: S = 320 = 5 tiles, last tile holds 12 valid rows; pads excluded
    vbs = np.array([64, 64, 64, 64, 12], np.int32)
    arr2 = np.concatenate([arr, arr[:, :, :20]], axis=2)
    xf2 = W.to_f32(arr2).astype(np.float64)
    valid = (np.arange(320) % 64) < vbs[np.arange(320) // 64]
    mu2 = oracle_lib.kmean(arr2, vbs)
    n = int(vbs.sum())
    for h in range(2):
        for c in range(8):
            exact = sum((Fraction(float(v)) for v in xf2[0, h, valid, c]), Fraction(0))
            assert mu2[0, h, c] == np.float32(float(exact) / n)


def test_kmean_count_clamped_to_one(oracle_lib):
    k = np.ones((1, 1, 64, 4), np.float32)
    mu = oracle_lib.kmean(k, np.array([0], np.int32))
    assert np.all(mu == 0.0)


def test_quantizer_invariants(oracle_lib):
    rs = np.random.default_rng(11)
    x = (rs.standard_normal((2, 3, 257, 128)) * rs.uniform(1e-3, 1e3, (2, 3, 257, 1))).astype(np.float32)
    q8, qs = oracle_lib.quantize_rows(x)
    # max |q| is exactly 127 on every non-degenerate row
    assert np.all(np.abs(q8.astype(np.int32)).max(-1) == 127)
    # odd symmetry
    qn, qsn = oracle_lib.quantize_rows(-x)
    assert np.array_equal(qn, -q8) and np.array_equal(qsn, qs)
    # reconstruction error bounded by half a step (plus fp32 rounding of x*inv)
    err = np.abs(x.astype(np.float64) - qs[..., None].astype(np.float64) * q8)
    assert np.all(err <= qs[..., None].astype(np.float64) * (0.5 + 1e-5))
    # scale invariance by powers of two (exact in fp32)
    q2, qs2 = oracle_lib.quantize_rows(x * np.float32(8.0))
    assert np.array_equal(q2, q8) and np.array_equal(qs2, qs * np.float32(8.0))


def test_constant_k_centres_to_zero(oracle_lib):
    row = W.f32_to_bf16_bits(np.linspace(-3, 3, 128, dtype=np.float32))
    k = np.broadcast_to(row, (1, 2, 100, 128)).copy()
    qk = oracle_lib.quantize_qk(np.zeros((1, 2, 10, 128), np.uint16), k)
    assert np.all(qk["k8"] == 0) and np.all(qk["ks"] == 0)
    assert np.array_equal(qk["kmean"][0, 0], W.bf16_bits_to_f32(row))


def test_pad_rows_quantize_to_zero(oracle_lib):
    w = W.WORKLOADS["tiny"]
    q, k, v = W.make_qkv(w, Sq=192, Sk=192)
    vbs = np.array([64, 64, 5], np.int32)
    qk = oracle_lib.quantize_qk(q, k, vbs)
    pad = (np.arange(192) % 64) >= vbs[np.arange(192) // 64]
    assert np.all(qk["k8"][:, :, pad] == 0) and np.all(qk["ks"][:, :, pad] == 0)
    assert np.all(qk["q8"][:, :, pad] == 0) and np.all(qk["qs"][:, :, pad] == 0)
    assert np.all(qk["qmu"][:, :, pad] == 0)
    assert np.all(qk["ks"][:, :, ~pad] > 0)


def test_qmu_definition(oracle_lib):
    w = W.WORKLOADS["tiny"]
    q, k, _ = W.make_qkv(w, Sq=16, Sk=16)
    qk = oracle_lib.quantize_qk(q, k)
    qf = W.to_f32(q).astype(np.float64)
    mu = qk["kmean"].astype(np.float64)
    for h in range(2):
        for i in range(16):
            want = float(sum(Fraction(float(a)) * Fraction(float(b)) for a, b in zip(qf[0, h, i], mu[0, h])))
            assert abs(qk["qmu"][0, h, i] - want) <= 1e-12 * max(1.0, abs(want))


def test_scores_i32_brute_force(oracle_lib):
    rs = np.random.default_rng(3)
    q8 = rs.integers(-127, 128, (37, 128), dtype=np.int64).astype(np.int8)
    k8 = rs.integers(-127, 128, (53, 128), dtype=np.int64).astype(np.int8)
    s = oracle_lib.scores_i32(q8, k8)
    for i in range(0, 37, 5):
        for j in range(0, 53, 7):
            assert s[i, j] == sum(int(a) * int(b) for a, b in zip(q8[i], k8[j]))
    # extreme magnitudes: every product 127*127 or -127*127
    big = np.full((2, 128), 127, np.int8)
    big[1] = -127
    s2 = oracle_lib.scores_i32(big, big)
    assert s2.tolist() == [[128 * 127 * 127, -128 * 127 * 127], [-128 * 127 * 127, 128 * 127 * 127]]


def test_kmean_of_no_keys_is_zero(oracle_lib):
    """Reading R1: the count is clamped to 1, so an empty K (dense or all-pad) has mean 0 and the
    centring term of every query row is 0."""
    k = np.zeros((2, 3, 0, 128), np.uint16)
    assert np.array_equal(oracle_lib.kmean(k), np.zeros((2, 3, 128), np.float32))
    q = W.normal(1, 0, (2, 3, 5, 128), "bf16")
    ref = oracle_lib.quantize_qk(q, k)
    assert np.array_equal(ref["kmean"], np.zeros((2, 3, 128), np.float32))
    assert np.array_equal(ref["qmu"], np.zeros((2, 3, 5)))
    kp = W.normal(1, 1, (1, 1, 64, 128), "bf16")
    assert np.array_equal(oracle_lib.kmean(kp, np.array([0], np.int32)), np.zeros((1, 1, 128), np.float32))


def test_non_finite_rows(oracle_lib):
    """The non-finite reading: a Q row holding NaN or +-inf quantizes to codes 0 with scale NaN and a
    NaN centring term, its finite neighbours are unaffected; a K channel with an inf among its valid
    keys has mean NaN, so every centred row of that head is such a row. A NaN in a pad row (vbs) is
    never read. Hand-built rows, checked element by element."""
    D = 8
    q = np.zeros((1, 1, 4, D), np.float32)
    q[0, 0, 0] = [1, -2, 3, -4, 5, -6, 7, -127]          # finite: codes are the values themselves
    q[0, 0, 1] = [1, np.nan, 3, 4, 5, 6, 7, 8]
    q[0, 0, 2] = [np.inf, 0, 0, 0, 0, 0, 0, 0]
    q[0, 0, 3] = [-np.inf, np.nan, 1, 1, 1, 1, 1, 1]
    k = np.zeros((1, 1, 3, D), np.float32)
    k[0, 0, :, :] = [[1, 2, 3, 4, 5, 6, 7, 8], [2, 2, 2, 2, 2, 2, 2, 2], [0, 1, 0, 1, 0, 1, 0, 1]]
    r = oracle_lib.quantize_qk(q, k)
    assert r["q8"][0, 0, 0].tolist() == [1, -2, 3, -4, 5, -6, 7, -127] and r["qs"][0, 0, 0] == 1.0
    for i in (1, 2, 3):
        assert np.all(r["q8"][0, 0, i] == 0) and np.isnan(r["qs"][0, 0, i]) and np.isnan(r["qmu"][0, 0, i])
    assert np.isfinite(r["qmu"][0, 0, 0]) and np.all(np.isfinite(r["kmean"]))
    # K: an inf in channel 3 makes that channel's mean NaN and every centred row non-finite
    k_bad = k.copy()
    k_bad[0, 0, 1, 3] = np.inf
    r = oracle_lib.quantize_qk(q[:, :, :1], k_bad)
    mu = r["kmean"].reshape(-1)
    assert np.isnan(mu[3]) and np.all(np.isfinite(np.delete(mu, 3)))
    assert np.all(r["k8"] == 0) and np.all(np.isnan(r["ks"]))
    assert np.isnan(r["qmu"][0, 0, 0])                      # q . mu meets the NaN channel
    # uncentred, only the row holding the inf is affected
    r = oracle_lib.quantize_qk(q[:, :, :1], k_bad, center_k=False)
    assert np.isnan(r["ks"][0, 0, 1]) and np.all(r["k8"][0, 0, 1] == 0)
    assert np.all(np.isfinite(r["ks"][0, 0, [0, 2]])) and r["k8"][0, 0, 0].tolist() == [16, 32, 48, 64, 79, 95, 111, 127]
    # a NaN in a pad row of a vbs call is never read: same result as a zero there
    kv = np.zeros((1, 1, 64, D), np.float32)
    kv[0, 0, :5] = np.arange(40, dtype=np.float32).reshape(5, 8) - 20
    kv_nan = kv.copy()
    kv_nan[0, 0, 5:] = np.nan
    vbs = np.array([5], np.int32)
    a, b = oracle_lib.quantize_qk(kv, kv, vbs), oracle_lib.quantize_qk(kv_nan, kv_nan, vbs)
    for name in ("q8", "qs", "k8", "ks", "kmean", "qmu"):
        assert np.array_equal(a[name], b[name]), name
