"""Build libqfa.so (the gfx950 kernels and the C ABI of include/qfa.h) in-tree.

Every source is compiled with hipcc for gfx950 only; packed fp32 VALU
instructions are disabled (-packed-fp32-ops), and no fast-math flag is used:
the quantizer depends on IEEE fp32 rounding and correctly rounded division.
The attention kernel alone is compiled with NaN-free semantics: it never
produces a NaN (excluded keys are -inf, and every -inf row is guarded), so
its max reductions need no NaN-quieting instructions. Rounding of every
arithmetic operation is unchanged by the flag.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
ROOT = os.path.dirname(PKG)
BUILD = os.path.join(ROOT, "_build", "qfa")
LIB = os.path.join(PKG, "libqfa.so")
# the measurement helper (include/qfa_probe.h): its own library, not part of the attention ABI
PROBE_SRC = "mfma_probe.hip"
PROBE_LIB = os.path.join(PKG, "libqfa_probe.so")

# the attention kernel's instances are split over four translation units compiled in parallel
ATTN_INST = ["attn_fwd_inst_d128_bf16.hip", "attn_fwd_inst_d128_fp16.hip", "attn_fwd_inst_d64_bf16.hip",
             "attn_fwd_inst_d64_fp16.hip"]
SOURCES = ATTN_INST + ["quantize.hip", "attn_fwd.hip", "blockmask.hip", "lse_merge.hip", "api.cpp"]

HIPCC = os.environ.get("HIPCC", shutil.which("hipcc") or "/opt/rocm/bin/hipcc")
COMMON = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-I", os.path.join(ROOT, "include")]


# the attention kernel's assembly is kept (-save-temps=obj) for the check below
EXTRA = {src: ["-fno-honor-nans", "-save-temps=obj"] for src in ATTN_INST}
EXTRA["attn_fwd.hip"] = ["-fno-honor-nans"]
EXTRA["mfma_probe.hip"] = ["-fno-honor-nans", "-save-temps=obj"]
ATTN_ASM = [os.path.join(BUILD, os.path.splitext(src)[0] + "-hip-amdgcn-amd-amdhsa-gfx950.s") for src in ATTN_INST]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *COMMON, *EXTRA.get(src, []), "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    return obj


def build(jobs: int = 8) -> str:
    """Compile every source and link libqfa.so next to this file; returns its path."""
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(jobs, len(SOURCES) + 1)) as ex:
        objs = list(ex.map(_compile, SOURCES + [PROBE_SRC]))
    probe_obj = objs.pop()
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    # hand-issued bias loads: nothing may touch their registers before their wait
    from .asm_check import check
    bad = {k: v for asm in ATTN_ASM for k, v in check(asm).items() if v}
    if bad:
        os.remove(LIB) if os.path.exists(LIB) else None
        raise RuntimeError(f"bias-load registers used before their wait: {bad}")
    os.replace(tmp, LIB)
    tmp = PROBE_LIB + ".tmp"
    r = subprocess.run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, probe_obj], capture_output=True,
                       text=True)
    if r.returncode != 0:
        raise RuntimeError(f"probe link failed:\n{r.stderr}")
    os.replace(tmp, PROBE_LIB)
    return LIB


if __name__ == "__main__":
    print(build())
