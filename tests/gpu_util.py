"""Helpers shared by the GPU parity tests: host <-> device transfer of the
seeded numpy inputs and the tolerance checks stated for the method."""
from __future__ import annotations

import numpy as np
import torch

# Tolerances of the attention output and LSE against the oracle (fp64):
# O max-abs 2e-2 and mean-abs 2e-3 in fp32, LSE 1e-3 absolute.
O_MAX_ABS = 2e-2
O_MEAN_ABS = 2e-3
LSE_ABS = 1e-3

DEV = torch.device("cuda:0")


def up(a: np.ndarray, dev=DEV) -> torch.Tensor:
    """numpy -> device tensor; uint16 arrays hold bf16 bits."""
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev)


def down(t: torch.Tensor) -> np.ndarray:
    """device tensor -> numpy (bf16 -> uint16 bits, other types as is)."""
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def as_bshd(t: torch.Tensor) -> torch.Tensor:
    """The same [B,H,S,D] values held in BSHD memory (a strided view)."""
    return t.transpose(1, 2).contiguous().transpose(1, 2)


# significand bits (implicit bit included) of the 16-bit output types
_SIG_BITS = {torch.bfloat16: 8, torch.float16: 11}


def half_ulp(x: np.ndarray, dtype: torch.dtype) -> np.ndarray:
    """Half an ulp of |x| in a bf16/fp16 output (0 for fp32): the most that rounding the exact
    value to the output type can add."""
    p = _SIG_BITS.get(dtype)
    if p is None:
        return np.zeros_like(x, dtype=np.float64)
    e = np.floor(np.log2(np.maximum(np.abs(x), 2.0 ** -14)))
    return np.exp2(e - p)


def check_o(o_gpu: torch.Tensor, o_ref: np.ndarray, rows=None, what=""):
    """The stated bounds (max-abs 2e-2, mean-abs 2e-3) hold for fp32 outputs; a bf16/fp16 output
    adds its own rounding, so each element's bound grows by half an ulp of the output type at
    that element's magnitude (the larger of the two values, in case they straddle a power of 2)."""
    o = o_gpu.float().cpu().numpy().reshape(-1, o_gpu.shape[-1])
    if rows is not None:
        o = o[rows]
    assert np.isfinite(o).all(), f"{what}: non-finite output"
    o = o.astype(np.float64)
    err = np.abs(o - o_ref)
    rnd = half_ulp(np.maximum(np.abs(o), np.abs(o_ref)), o_gpu.dtype)
    excess = err - rnd
    assert excess.max() <= O_MAX_ABS and (err.mean() - rnd.mean()) <= O_MEAN_ABS, \
        f"{what}: O max-abs {err.max():.3e} (beyond output rounding {excess.max():.3e}) mean-abs {err.mean():.3e}"
    return err


def check_lse(l_gpu: torch.Tensor, l_ref: np.ndarray, rows=None, what=""):
    l = l_gpu.cpu().numpy().reshape(-1).astype(np.float64)
    if rows is not None:
        l = l[rows]
    inf_ref = np.isneginf(l_ref)
    assert np.array_equal(np.isneginf(l), inf_ref), f"{what}: -inf rows differ"
    d = np.abs(l[~inf_ref] - l_ref[~inf_ref])
    assert d.size == 0 or d.max() <= LSE_ABS, f"{what}: LSE max-abs {d.max():.3e}"


def sample_rows(B, H, Sq, per_head=48, heads=None, seed=0):
    """Flat [B,H,Sq] row indices: first/last rows plus random rows of a few heads."""
    rs = np.random.default_rng(seed)
    heads = heads if heads is not None else sorted({0, H // 2, H - 1})
    rows = []
    for b in range(B):
        for h in heads:
            base = (b * H + h) * Sq
            pick = np.unique(np.r_[0, Sq - 1, rs.integers(0, Sq, per_head)])
            rows.extend(base + pick)
    return np.array(rows, np.int64)
