"""The CPU side under AddressSanitizer and UndefinedBehaviorSanitizer.

The oracle (oracle.c, built by gcc) and the host half of the C ABI (api.cpp, built by hipcc with
the sanitizers on the host side only) are rebuilt instrumented into a temporary directory, and the
CPU tests that exercise them run against those builds in child processes with the sanitizer
runtime preloaded (gcc's for the oracle, clang's for the ABI: the two runtimes cannot share a
process). Any sanitizer report fails the child (halt_on_error, no recovery from UB)."""
import glob
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BUILD = os.path.join(ROOT, "_build", "qfa")
SAN_ENV = {"ASAN_OPTIONS": "detect_leaks=0:halt_on_error=1:abort_on_error=1",
           "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1"}


def _run_child(tests, env_extra, preload):
    env = dict(os.environ, **SAN_ENV, **env_extra, LD_PRELOAD=preload)
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", "-m", "not gpu",
                        *tests], cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    return out


def test_oracle_under_asan_ubsan(tmp_path):
    asan = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    if not os.path.isabs(asan):
        pytest.skip("gcc has no ASan runtime")
    lib = str(tmp_path / "liboracle_san.so")
    subprocess.run(["gcc", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
                    "-fno-sanitize-recover=all", "-std=gnu11", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
                    "-fPIC", "-shared", "-o", lib, os.path.join(ROOT, "oracle", "oracle.c"), "-lm"], check=True)
    tests = sorted(glob.glob(os.path.join(ROOT, "tests", "test_oracle_*.py")))
    out = _run_child(tests, {"QFA_ORACLE_LIB": lib}, asan)
    assert " passed" in out


def test_abi_host_code_under_asan_ubsan(tmp_path):
    clang_rt = glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so")
    objs = [os.path.join(BUILD, f) for f in ("attn_fwd_inst_d128_bf16.o", "attn_fwd_inst_d128_fp16.o",
                                              "attn_fwd_inst_d64_bf16.o", "attn_fwd_inst_d64_fp16.o", "quantize.o",
                                              "attn_fwd.o", "blockmask.o", "lse_merge.o")]
    if not clang_rt or not all(os.path.exists(o) for o in objs):
        pytest.skip("needs clang's ASan runtime and a built library (_build/qfa)")
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    api_o = str(tmp_path / "api_san.o")
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]
    subprocess.run([hipcc, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC", *san, "-I",
                    os.path.join(ROOT, "include"), "-x", "hip", "-c",
                    os.path.join(ROOT, "quantized_flash_attention_amd", "csrc", "api.cpp"), "-o", api_o], check=True)
    lib = str(tmp_path / "libqfa.so")
    # the sanitizer runtime is preloaded at run time, so the library leaves its symbols unresolved
    subprocess.run([hipcc, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", lib, api_o, *objs], check=True)
    shutil.copy(os.path.join(ROOT, "quantized_flash_attention_amd", "libqfa_probe.so"), tmp_path / "libqfa_probe.so")
    out = _run_child([os.path.join(ROOT, "tests", "test_abi.py")], {"QFA_LIB_PATH": lib}, clang_rt[0])
    assert " passed" in out
