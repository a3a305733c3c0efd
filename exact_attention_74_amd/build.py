"""Compile libexattn.so (all HIP sources of the package) for gfx950, in-tree.

Usage: python -m exact_attention_74_amd.build [--verbose]
"""
from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libexattn.so")
SOURCES = ["attn_bf16.hip", "attn_fp8.hip", "attn_bwd.hip", "blockquant.hip", "api.hip"]
ARCH = "gfx950"

# -packed-fp32-ops: keep the compiler from forming v_pk_{add,mul,fma}_f32.
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


# Per-source extra flags.  -fno-honor-nans lets max() of MFMA results lower to
# v_max3_f32 without NaN-quieting copies (the attention kernels never form a
# NaN from valid input; infinities, used for masking, are still honoured).
# -amdgpu-mfma-vgpr-form: the compiler-issued MFMAs write VGPRs (S and dP are
# read by the VALU right away); the accumulators that need the AGPR file (the
# gradients' dK/dV at head dim 128, the bf16 forward's O at head dim 256) are
# placed there by the kernels' own assembly MFMAs, so no accumulator is copied
# between the two files.  (At head dims 64 and 128 the forward kernels fit
# the 256 VGPRs, and the flag leaves their code unchanged.)
EXTRA = {
    "attn_bf16.hip": ["-fno-honor-nans", "-mllvm", "-amdgpu-mfma-vgpr-form"],
    "attn_fp8.hip": ["-fno-honor-nans"],
    "attn_bwd.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
}


def _compile(src: str, obj: str, verbose: bool) -> None:
    cmd = [hipcc(), *FLAGS, *EXTRA.get(os.path.basename(src), []), "-I", INCLUDE, "-I", CSRC,
           "-c", src, "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")


def build(verbose: bool = False) -> str:
    """Compile every source and link the shared library; returns its path."""
    objdir = os.path.join(PKG, "_build")
    os.makedirs(objdir, exist_ok=True)
    objs = []
    with concurrent.futures.ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        futs = []
        for s in SOURCES:
            obj = os.path.join(objdir, s.replace(".hip", ".o"))
            objs.append(obj)
            futs.append(ex.submit(_compile, os.path.join(CSRC, s), obj, verbose))
        for f in futs:
            f.result()
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="--verbose" in sys.argv))
