"""Build libdlm.so for gfx950 with hipcc (in-tree, next to the Python package).

Usage: python -m masked_block_diffusion_denoise_amd.csrc.build  [--jobs N]
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
PKG = os.path.dirname(HERE)
ROOT = os.path.dirname(PKG)
BUILD = os.path.join(HERE, "_build")
OUT = os.path.join(PKG, "libdlm.so")

SOURCES = ["api.cpp", "k_small.hip", "k_gemm.hip", "k_attention.hip"]
ARCH = "gfx950"
# Packed fp32 instructions are switched off for all device code (the compiler
# would otherwise form them from scalar float code).
FLAGS = ["-O3", "-fPIC", "-std=c++17", f"--offload-arch={ARCH}", "-Wall", "-Wno-unused-function",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         f"-I{os.path.join(ROOT, 'include')}", f"-I{HERE}"]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm is required to build libdlm)")


# Per-source flags.  The MFMA kernels keep their accumulators in VGPRs: where a
# loop-carried accumulator also meets vector ALU code (attention's online
# softmax rescale, a GEMM wavefront that skips its MFMAs) the compiler otherwise
# copies every accumulator between AGPRs and VGPRs on every iteration.
VGPR_MFMA = ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]
SOURCE_FLAGS = {"k_attention.hip": VGPR_MFMA, "k_gemm.hip": VGPR_MFMA}


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *FLAGS, *SOURCE_FLAGS.get(src, []), "-c", os.path.join(HERE, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build(jobs: int = 4, verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = OUT + ".tmp"
    cmd = [hipcc(), "-shared", f"--offload-arch={ARCH}", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    # a kernel whose host-side launch stub was not emitted links fine and only
    # fails when the library is loaded: refuse such a build here
    nm = shutil.which("nm")
    if nm:
        und = subprocess.run([nm, "-C", "--undefined-only", tmp], capture_output=True, text=True).stdout
        stubs = [l.strip() for l in und.splitlines() if "__device_stub__" in l]
        if stubs:
            os.remove(tmp)
            raise RuntimeError("kernel launch stubs missing from the host objects:\n" + "\n".join(stubs))
    os.replace(tmp, OUT)
    if verbose:
        print(f"built {OUT}")
    return OUT


def main(argv=None) -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=min(4, os.cpu_count() or 1))
    a = ap.parse_args(argv)
    build(a.jobs, verbose=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
