"""The build's check of the hand-issued bias loads (quantized_flash_attention_amd.asm_check):
it passes on the built kernels and catches a register read before the retiring wait."""
import os

import pytest

from quantized_flash_attention_amd import asm_check, build

SYM = "_ZN3qfa12_GLOBAL__N_115attn_fwd_kernelILi64ELi1ELi4ELb0ELb0ELb0ELb0ELb0ELb0ELb1EEEvNS_8AttnArgsEii"


def _asm(body: str) -> str:
    return f"{SYM}:\n{body}\n.Lfunc_end0:\n"


def test_built_kernels_keep_bias_loads_untouched():
    if not all(os.path.exists(p) for p in build.ATTN_ASM):
        pytest.skip("library not built")
    res = {k: v for p in build.ATTN_ASM for k, v in asm_check.check(p).items()}
    assert len(res) >= 16                       # every materialised-bias instance
    assert all(not v for v in res.values()), {k: v for k, v in res.items() if v}


def test_checker_catches_reads_before_the_wait(tmp_path):
    load = "\tbuffer_load_dwordx4 v[10:13], v1, s[8:11], 0 offen\n"
    copy = "\tbuffer_load_dwordx4 v2, s[12:15], 0 offen lds\n"
    cases = {
        # read of v12 while the load is in flight
        "read_before_wait": (load + "\tv_mov_b32_e32 v0, v12\n\ts_waitcnt vmcnt(0)\n", 1),
        # the wait retires it (one newer vector-memory op, vmcnt(1))
        "read_after_wait": (load + copy + "\ts_waitcnt vmcnt(1)\n\tv_mov_b32_e32 v0, v12\n", 0),
        # vmcnt(1) does not retire the newest load
        "wait_too_weak": (copy + load + "\ts_waitcnt vmcnt(1)\n\tv_mov_b32_e32 v0, v12\n", 1),
        # a read on only one branch path still counts
        "read_on_a_branch": (load + "\ts_cbranch_scc0 .LBB0_2\n\tv_add_f32_e32 v0, v11, v0\n.LBB0_2:\n"
                             "\ts_waitcnt vmcnt(0)\n", 1),
    }
    for name, (body, n) in cases.items():
        p = tmp_path / f"{name}.s"
        p.write_text(_asm(body))
        assert len(asm_check.check(str(p))[SYM]) == n, name
