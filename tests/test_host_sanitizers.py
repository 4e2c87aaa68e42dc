"""Host AddressSanitizer + UndefinedBehaviorSanitizer run of the CPU suite.

The oracle, the input generator and the host code of the HIP library (its
argument checks, launch set-up and error paths; the device code is built as
usual) are rebuilt with ASan and UBSan into a temporary directory, and the
CPU tests that exercise them (the oracle's pins and planted mutants, the
generator, every C-ABI export's validation, the binding's size checks, the
GEMM address replay) run in a child process with the sanitizer runtime
preloaded and those builds selected through MOE_ORACLE_LIB, MOE_SYNTH_LIB
and MOE_MI355X_LIB. Any sanitizer report, or a failing test, fails this test.
No GPU is used.
"""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CLANG = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "llvm", "bin", "clang")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer", "-g", "-O1"]
SUITE = ["tests/test_oracle_pins.py", "tests/test_oracle_mutants.py", "tests/test_synth.py", "tests/test_abi_cpu.py",
         "tests/test_gemm_address_bounds.py", "tests/test_act_layout.py"]

pytestmark = pytest.mark.skipif(not os.path.exists(CLANG), reason="ROCm clang (with its sanitizer runtimes) not found")


def _c_library(src: str, out: str) -> str:
    subprocess.check_call([CLANG, *SAN, "-fopenmp", "-fPIC", "-shared", src, "-o", out, "-lm"])
    return out


def test_cpu_suite_under_host_sanitizers(tmp_path):
    from sparse_mixture_experts_softmax_amd import build as hip_build

    runtime = subprocess.check_output([CLANG, "-print-file-name=libclang_rt.asan-x86_64.so"], text=True).strip()
    assert os.path.exists(runtime), runtime
    oracle_lib = _c_library(os.path.join(ROOT, "oracle", "moe_oracle.c"), str(tmp_path / "libmoe_oracle_san.so"))
    synth_lib = _c_library(os.path.join(ROOT, "synth", "synth.c"), str(tmp_path / "libmoe_synth_san.so"))
    hip_lib = hip_build.build(out=str(tmp_path / "libmoe_mi355x_san.so"), host_sanitize=True)
    env = dict(os.environ)
    env.update({
        "LD_PRELOAD": runtime,
        "LD_LIBRARY_PATH": os.path.dirname(runtime) + os.pathsep + env.get("LD_LIBRARY_PATH", ""),
        # Python itself is not instrumented and keeps memory until exit
        "ASAN_OPTIONS": "detect_leaks=0:abort_on_error=1:verify_asan_link_order=0",
        "UBSAN_OPTIONS": "print_stacktrace=1:halt_on_error=1",
        "MOE_ORACLE_LIB": oracle_lib,
        "MOE_SYNTH_LIB": synth_lib,
        "MOE_MI355X_LIB": hip_lib,
    })
    cmd = [sys.executable, "-m", "pytest", "-q", "-x", "-m", "not gpu", "-p", "no:cacheprovider", *SUITE]
    res = subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    out = res.stdout + res.stderr
    for marker in ("ERROR: AddressSanitizer", "runtime error:", "ERROR: LeakSanitizer"):
        assert marker not in out, out[-6000:]
    assert res.returncode == 0, out[-6000:]
    assert " passed" in out
    shutil.rmtree(tmp_path / "_objs", ignore_errors=True)
