"""Builds libdsa.so (the gfx950 kernels and the C ABI of include/dsa.h) in this directory."""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libdsa.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

SOURCES = ["dsa_api.cpp", "k_index.hip", "k_mla.hip", "k_up.hip", "k_absorb.hip", "k_gemm.hip", "k_bwd.hip"]
# Per-file code generation options. The attention kernel keeps 256 fp32 accumulators per lane in
# AGPRs; selecting the VGPR form of MFMA lets the query fragments live in AGPRs as MFMA operands and
# the QK^T accumulators in VGPRs, instead of evicting an output tile every key tile.
FILE_FLAGS = {
    "k_mla.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"],
    "k_index.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"],
}
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    # no packed FP32 VALU instructions anywhere in the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def _run(cmd, verbose):
    r = subprocess.run(cmd, capture_output=True, text=True)
    msgs = [l for l in (r.stdout + r.stderr).splitlines() if "packed-fp32-ops" not in l]
    if r.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + " ".join(cmd) + "\n" + "\n".join(msgs))
    if verbose and msgs:
        print("\n".join(msgs), file=sys.stderr)


def build(verbose: bool = False) -> str:
    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)
    objs = []
    for s in SOURCES:
        obj = os.path.join(objdir, s + ".o")
        cmd = [HIPCC, *[f for f in FLAGS if f != "-shared"], *FILE_FLAGS.get(s, []), "-I", os.path.join(ROOT, "include"),
               "-I", CSRC, "-x", "hip", "-c", os.path.join(CSRC, s), "-o", obj]
        _run(cmd, verbose)
        objs.append(obj)
    _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", LIB + ".tmp"], verbose)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
