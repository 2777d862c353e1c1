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


def check_o(o_gpu: torch.Tensor, o_ref: np.ndarray, rows=None, what=""):
    """The stated bounds on an fp32 output: max-abs 2e-2 and mean-abs 2e-3 against the oracle. A
    bf16/fp16 output of the same call is checked separately, bit for bit, by check_rne."""
    assert o_gpu.dtype == torch.float32, f"{what}: the bounds apply to an fp32 output, got {o_gpu.dtype}"
    o = o_gpu.cpu().numpy().reshape(-1, o_gpu.shape[-1])
    if rows is not None:
        o = o[rows]
    assert np.isfinite(o).all(), f"{what}: non-finite output"
    err = np.abs(o.astype(np.float64) - o_ref)
    assert err.max() <= O_MAX_ABS and err.mean() <= O_MEAN_ABS, \
        f"{what}: O max-abs {err.max():.3e} mean-abs {err.mean():.3e}"
    return err


def check_rne(o16: torch.Tensor, o32: torch.Tensor, what=""):
    """The 16-bit output of a call equals its fp32 output rounded to nearest even, bit for bit (the
    epilogue rounds once, from the same fp32 value; the conversion here runs on the host)."""
    assert o16.dtype in (torch.bfloat16, torch.float16) and o32.dtype == torch.float32
    want = o32.cpu().to(o16.dtype).contiguous().view(torch.int16)
    got = o16.cpu().contiguous().view(torch.int16)
    if not torch.equal(got, want):
        bad = (got != want).nonzero()
        i = tuple(bad[0].tolist())
        raise AssertionError(f"{what}: {len(bad)} 16-bit outputs differ from RNE of the fp32 output, first at {i}: "
                             f"{o16.cpu()[i].item()!r} vs {o32.cpu()[i].item()!r}")


def both_outputs(fn, dtype16: torch.dtype, what=""):
    """Run one attention (or merge) call twice, fn(out_dtype) -> out or (out, lse): with an fp32 output and
    with the 16-bit type dtype16. Checks the 16-bit output against RNE of the fp32 one (check_rne) and
    that the LSE does not depend on the output type; returns the fp32 call's result."""
    r32 = fn(torch.float32)
    r16 = fn(dtype16)
    pair = isinstance(r32, tuple)
    o32, o16 = (r32[0], r16[0]) if pair else (r32, r16)
    assert o32.dtype == torch.float32 and o16.dtype == dtype16
    check_rne(o16, o32, what)
    if pair and r32[1] is not None:
        assert torch.equal(r32[1], r16[1]), f"{what}: the LSE depends on the output type"
    return r32


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


def block_rows(B, H, Sq, per_block=1, seed=0, block=128):
    """Flat [B,H,Sq] row indices covering every (b, h) and every `block`-row query block: `per_block`
    seeded rows of each block plus each head's first and last row."""
    rs = np.random.default_rng(seed)
    nblk = -(-Sq // block)
    starts = np.arange(nblk) * block
    lens = np.minimum(block, Sq - starts)
    rows = []
    for bh in range(B * H):
        pick = starts[:, None] + (rs.random((nblk, per_block)) * lens[:, None]).astype(np.int64)
        rows.append(bh * Sq + np.unique(np.r_[pick.reshape(-1), 0, Sq - 1]))
    return np.concatenate(rows).astype(np.int64)

