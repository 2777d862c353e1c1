"""Seeded synthetic inputs for INT8-QK / BF16-PV attention.

This module only draws and lays out inputs; it holds none of the method's
arithmetic, so the CPU oracle and the GPU path can both take their inputs
from it.

Recipe (every tensor is reproducible from (config id, tensor id)):
  * generator: numpy PCG64 ``default_rng([cfg_id, tensor_id])`` with tensor
    ids 0 = Q, 1 = K, 2 = V, 3 = K channel offset, 4 = V scale;
  * values: ``standard_normal`` in fp32, then rounded to bf16 (round to
    nearest even on the bit pattern) or to fp16 (numpy ``astype``);
  * bf16 tensors are carried as ``np.uint16`` bit arrays.

Workloads (shapes and structure follow the pages' own workloads; the real
activations they were measured on are not available, N(0,1) tensors of the
same shapes stand in for them):
  * tiny:    B1 H2 S256 D128 bf16, K centred, LSE on.
  * dense4k: B1 H16 S4096 D128 bf16, K plus a per-channel offset ~ N(0, std 2)
             shared by every batch, head and token.
  * d64:     B2 H10 S9216 D64 fp16.
  * band:    B1 H56 Sq4096 Sk33600 D128 bf16 with a [1,1,1,K] natural-log
             bias: 0 over the central 20160-key core, a raised-cosine fade
             from 0 down to ln(1e-4) over a 6720-key skirt on either side
             (the soft-edged window of comfy-kitchen issue #177, made
             two-sided).
  * sparse:  B1 H24 S131072 D128 bf16, tile-64 block mask where query tile t
             attends key tiles u < 8 (prefix) or |u - t| <= 48 (band), the same
             for every head; validity vector 64 everywhere except 17 in the
             last tile, pad rows of Q/K/V zero; V scale [H,D] ~ U(0.5, 2).
  * gqa:     B2 S2048 H16 Hkv2 D128 bf16, causal self-attention: the
             grouped-query shape of ROCm/FlyDSL PR #886's timed table (runs
             of 8 query heads share one K/V head).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

Q_ID, K_ID, V_ID, KOFF_ID, VSCALE_ID = 0, 1, 2, 3, 4


def rng(cfg_id: int, tensor_id: int) -> np.random.Generator:
    return np.random.default_rng([cfg_id, tensor_id])


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (nearest, ties to even) and return the raw 16-bit patterns."""
    u = np.ascontiguousarray(x, np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def to_f32(x: np.ndarray) -> np.ndarray:
    """Exact fp32 view of a bf16 (uint16 bits), fp16 or fp32 array."""
    if x.dtype == np.uint16:
        return bf16_bits_to_f32(x)
    return x.astype(np.float32)


def normal(cfg_id: int, tensor_id: int, shape, dtype: str, std: float = 1.0, offset=None) -> np.ndarray:
    x = rng(cfg_id, tensor_id).standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    if offset is not None:
        x += offset
    return f32_to_bf16_bits(x) if dtype == "bf16" else x.astype(np.float16)


@dataclass
class Workload:
    name: str
    cfg_id: int
    B: int
    H: int
    Sq: int
    Sk: int
    D: int
    dtype: str                  # "bf16" | "fp16"
    center_k: bool = True
    extras: dict = field(default_factory=dict)

    @property
    def sm_scale(self) -> float:
        return float(np.float32(self.D ** -0.5))


WORKLOADS = {
    "tiny": Workload("tiny", 1, 1, 2, 256, 256, 128, "bf16"),
    "dense4k": Workload("dense4k", 2, 1, 16, 4096, 4096, 128, "bf16", extras={"k_offset_std": 2.0}),
    "d64": Workload("d64", 3, 2, 10, 9216, 9216, 64, "fp16"),
    "band": Workload("band", 4, 1, 56, 4096, 33600, 128, "bf16",
                     extras={"core": (6720, 20160), "skirt": 6720}),
    "sparse": Workload("sparse", 5, 1, 24, 131072, 131072, 128, "bf16",
                       extras={"prefix": 8, "band": 48, "last_valid": 17}),
    "gqa": Workload("gqa", 6, 2, 16, 2048, 2048, 128, "bf16", extras={"hkv": 2, "causal": True}),
}


def make_qkv(w: Workload, B=None, H=None, Sq=None, Sk=None, Hkv=None):
    """Q, K, V of the workload (optionally with smaller B/H/Sq/Sk for parity tests).

    K and V hold Hkv heads (the workload's "hkv", else H). A smaller draw
    uses the same recipe and seeds, so its values differ from a slice of the
    full-size draw; it is a workload of the same kind.
    """
    B = B or w.B
    H = H or w.H
    Hkv = Hkv or w.extras.get("hkv", H)
    Sq = Sq or w.Sq
    Sk = Sk or w.Sk
    offset = None
    if "k_offset_std" in w.extras:
        offset = rng(w.cfg_id, KOFF_ID).standard_normal(size=(w.D,), dtype=np.float32) * np.float32(
            w.extras["k_offset_std"])
    q = normal(w.cfg_id, Q_ID, (B, H, Sq, w.D), w.dtype)
    k = normal(w.cfg_id, K_ID, (B, Hkv, Sk, w.D), w.dtype, offset=offset)
    v = normal(w.cfg_id, V_ID, (B, Hkv, Sk, w.D), w.dtype)
    return q, k, v


def band_bias(Sk: int = 33600, core=(6720, 20160), skirt: int = 6720) -> np.ndarray:
    """Two-sided raised-cosine per-key bias in fp64, natural-log units, shape [Sk].

    For r = 0..skirt-1, x = r/(skirt-1), w = (1 + cos(pi x))/2, b = ln(max(w, 1e-4)).
    The right skirt is b at core_end + r, the left skirt is b mirrored, the
    core is 0. Values adjacent to the core are 0; the outer edges reach ln(1e-4).
    """
    c0, clen = core
    out = np.zeros(Sk, np.float64)
    r = np.arange(skirt, dtype=np.float64)
    x = r / (skirt - 1)
    wv = 0.5 * (1.0 + np.cos(math.pi * x))
    b = np.log(np.maximum(wv, 1e-4))
    right0 = c0 + clen
    n_right = min(skirt, Sk - right0)
    out[right0:right0 + n_right] = b[:n_right]
    n_left = min(skirt, c0)
    out[c0 - n_left:c0] = b[:n_left][::-1]
    return out


def bias_tensor(b64: np.ndarray, dtype: str) -> np.ndarray:
    """[Sk] fp64 bias -> [1,1,1,Sk] fp32 or bf16 bits (round to nearest even)."""
    f = b64.astype(np.float32)
    if dtype == "bf16":
        # the bf16 bias is the fp32 bias rounded to bf16 (nearest even)
        return f32_to_bf16_bits(f).reshape(1, 1, 1, -1)
    return f.reshape(1, 1, 1, -1)


def sparse_mask(T: int, H: int, prefix: int = 8, band: int = 48) -> np.ndarray:
    """Bool tile mask [1,H,T,T]: key tile u is attended by query tile t if u < prefix or |u-t| <= band."""
    t = np.arange(T)[:, None]
    u = np.arange(T)[None, :]
    m = (u < prefix) | (np.abs(u - t) <= band)
    return np.broadcast_to(m, (1, H, T, T)).copy()


def sparse_vbs(T: int, last_valid: int = 17) -> np.ndarray:
    v = np.full(T, 64, np.int32)
    v[-1] = last_valid
    return v


def zero_pads(x: np.ndarray, vbs: np.ndarray) -> np.ndarray:
    """Zero the pad rows (j mod 64 >= vbs[j/64]) of a [B,H,S,D] array in place."""
    S = x.shape[2]
    j = np.arange(S)
    pad = (j % 64) >= vbs[j // 64]
    x[:, :, pad, :] = 0
    return x


def v_scale(w: Workload, H=None) -> np.ndarray:
    H = H or w.H
    return rng(w.cfg_id, VSCALE_ID).uniform(0.5, 2.0, size=(H, w.D)).astype(np.float32)
