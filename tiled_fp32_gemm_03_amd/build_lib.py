"""Build ``libgemm_f32.so`` for gfx950 in-tree with hipcc.

Each ``csrc/*.hip`` translation unit is compiled to an object in parallel,
the host-only planning unit ``csrc/host_plan.cpp`` with the host C++
compiler, and the objects are linked into one shared library next to this
file.  Packed fp32 VALU forms are disabled for all device code.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libgemm_f32.so")
ARCH = "gfx950"

SOURCES = ["gemm_f32_abi.hip", "naive_tiled.hip", "prod.hip", "w16_vgpr.hip", "valu.hip", "mixed.hip",
           "mixed16.hip", "probes.hip"]

# Host-only C++ (no device code): argument checks, launch table, choice model.
HOST_SOURCES = ["host_plan.cpp"]
HOST_FLAGS = ["-std=c++17", "-O2", "-fPIC", "-Wall", "-Wextra", "-I", CSRC]

# Per-source flags: the kernels of w16_vgpr.hip keep their accumulators in
# VGPRs (the MFMAs' VGPR form); see that file.
SOURCE_FLAGS = {"w16_vgpr.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]}

COMMON_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Wall", "-Wextra", "-Wno-unused-parameter",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE, "-I", CSRC,
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the gfx950 library)")


def host_cxx() -> str:
    for cand in (os.environ.get("CXX"), shutil.which("g++"), shutil.which("c++")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("no host C++ compiler (g++) found")


def _compile(src: str, extra: list[str], verbose: bool) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    if src in HOST_SOURCES:
        cmd = [host_cxx(), *HOST_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    else:
        cmd = [hipcc(), *COMMON_FLAGS, *SOURCE_FLAGS.get(src, []), *extra, "-c",
               os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compiling {src} failed:\n{r.stdout}\n{r.stderr}")
    # The host pass does not know the packed-fp32 feature and says so; keep
    # every other diagnostic visible.
    noise = "is not a recognized feature for this target"
    msgs = [ln for ln in r.stderr.splitlines() if noise not in ln and ln.strip()
            and not ln.startswith("(ignoring feature)")]
    if msgs and verbose:
        print("\n".join(msgs), file=sys.stderr, flush=True)
    return obj


def build(verbose: bool = False, extra: list[str] | None = None) -> str:
    os.makedirs(BUILD, exist_ok=True)
    extra = list(extra or [])
    srcs = SOURCES + HOST_SOURCES
    jobs = min(len(srcs), int(os.environ.get("MAX_JOBS", os.cpu_count() or 4)))
    with cf.ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
        objs = list(ex.map(lambda s: _compile(s, extra, verbose), srcs))
    tmp = LIB + f".tmp{os.getpid()}"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
