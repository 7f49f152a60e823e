"""Compile libssm.so (the HIP kernels and the C ABI) for gfx950, in-tree.

    python -m selective_state_space_28_amd.build

Cross-compiles without a GPU.  Packed-fp32 instructions are switched off for
all device code (-packed-fp32-ops); the host pass warns that it does not know
that feature, which is harmless.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libssm.so")
SOURCES = ["scan_fwd.hip", "scan_wave.hip", "scan_bwd.hip", "ssd.hip", "state_update.hip", "ssm_api.cpp"]
ARCH = "gfx950"
# Per-source options.  The backward sweep runs two waves per SIMD, so the
# scheduler that favours instruction-level parallelism hides more of its
# latency (3% on the backward of batch 16, D 5120, N 16, L 2048, both input
# terms); the forward kernels are best with the default scheduler.
SOURCE_FLAGS = {"scan_bwd.hip": ["-mllvm", "-amdgpu-sched-strategy=iterative-ilp"]}


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libssm)")


def flags() -> list[str]:
    return [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-I", INCLUDE, "-I", CSRC]


def build(verbose: bool = False) -> str:
    hipcc = _hipcc()
    objdir = os.path.join(PKG, "_build")
    os.makedirs(objdir, exist_ok=True)

    def compile_one(src):
        obj = os.path.join(objdir, os.path.splitext(src)[0] + ".o")
        cmd = [hipcc, *flags(), *SOURCE_FLAGS.get(src, []), "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed on {src}:\n{r.stderr}")
        return obj

    with ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(compile_one, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link of libssm.so failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


MICROBENCH = os.path.join(PKG, "microbench", "valu_rate.hip")


def build_microbench(verbose: bool = False) -> str:
    """Compile the standalone VALU-rate microbenchmark (microbench/valu_rate.hip)
    into an executable beside its source."""
    exe = os.path.splitext(MICROBENCH)[0]
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-mllvm", "-amdgpu-mfma-vgpr-form",
           MICROBENCH, "-o", exe]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {MICROBENCH}:\n{r.stderr}")
    return exe


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
    print(build_microbench(verbose="-v" in sys.argv))
