"""Builds libmoe_mi355x.so in this directory with hipcc for gfx950.

    python -m sparse_mixture_experts_softmax_amd.build [--jobs N]

Every HIP translation unit is compiled with packed-fp32 instructions
disabled (-Xclang -target-feature -Xclang -packed-fp32-ops); hipcc's host
pass warns that it does not know that feature, which is harmless.
"""
from __future__ import annotations

import argparse
import concurrent.futures
import os
import re
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB_NAME = "libmoe_mi355x.so"
LIB_PATH = os.path.join(HERE, LIB_NAME)
ARCH = "gfx950"

SOURCES = ["abi.cpp", "route.hip", "align.hip", "pack.hip", "gemm.hip", "combine.hip", "rmsnorm.hip"]
HIP_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    path = os.path.join(rocm, "bin", "hipcc")
    return path if os.path.exists(path) else "hipcc"


def _scratch_users(remarks: str) -> list:
    """Kernels whose resource-usage remark reports scratch (register spills).

    The copy pipelines count their outstanding memory operations by hand
    (s_waitcnt vmcnt), so a spill reload inside a loop would break the count;
    every kernel here must run without scratch.
    """
    bad, name = [], None
    for line in remarks.splitlines():
        m = re.search(r"remark: Function Name: (\S+)", line)
        if m:
            name = m.group(1)
            continue
        m = re.search(r"remark:\s+ScratchSize \[bytes/lane\]: (\d+)", line)
        if m and int(m.group(1)) > 0:
            bad.append(f"{name} ({m.group(1)} bytes/lane)")
    return bad


# Host-side AddressSanitizer + UndefinedBehaviorSanitizer (argument checks,
# launch set-up, error paths): each flag applies to the host compilation only,
# the device code is built as usual.
HOST_SANITIZE = ["-Xarch_host", "-fsanitize=address,undefined", "-Xarch_host", "-fno-sanitize-recover=undefined",
                 "-Xarch_host", "-fno-omit-frame-pointer", "-g"]


def _compile(src: str, build_dir: str = BUILD_DIR, extra=()) -> str:
    obj = os.path.join(build_dir, os.path.basename(src) + ".o")
    remarks = ["-Rpass-analysis=kernel-resource-usage"] if src.endswith(".hip") else []
    cmd = [hipcc(), *HIP_FLAGS, *extra, *remarks, f"-I{INCLUDE}", f"-I{CSRC}", "-c", os.path.join(CSRC, src), "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{res.stdout}\n{res.stderr}")
    bad = _scratch_users(res.stderr)
    if bad:
        raise RuntimeError(f"{src}: kernels use scratch (register spills): " + ", ".join(bad))
    return obj


def build(jobs: int = 0, out: str = LIB_PATH, host_sanitize: bool = False) -> str:
    """Compile all sources and link the shared library; returns its path.
    ``host_sanitize``: instrument the host code with ASan and UBSan (a test
    build, loaded with the sanitizer runtime preloaded; written to ``out``)."""
    build_dir = BUILD_DIR if not host_sanitize else os.path.join(os.path.dirname(os.path.abspath(out)), "_objs")
    os.makedirs(build_dir, exist_ok=True)
    extra = HOST_SANITIZE if host_sanitize else []
    jobs = jobs or min(len(SOURCES), os.cpu_count() or 1, 16)
    with concurrent.futures.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(lambda src: _compile(src, build_dir, extra), SOURCES))
    tmp = out + ".tmp"
    link_extra = ["-Xarch_host", "-fsanitize=address,undefined", "-shared-libasan"] if host_sanitize else []
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *link_extra, *objs, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=0)
    print(build(ap.parse_args().jobs))
    sys.exit(0)
