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
