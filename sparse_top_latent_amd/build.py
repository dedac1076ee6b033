"""Compiles the HIP library libsparse_attn.so in-tree for gfx950 with hipcc."""
from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRC = os.path.join(HERE, "csrc", "sparse_attn.hip")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libsparse_attn.so")

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    # packed fp32 instructions are kept out of the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA results stay in arch VGPRs: the softmax rescale touches the output
    # accumulators with VALU ops, which cannot read AGPRs
    "-mllvm", "-amdgpu-mfma-vgpr-form=1",
    # every loop marked for unrolling is unrolled: the QK^T loops are sized
    # before their per-step row-request branches fold to constants, and the
    # default limit left the FP4 builds' loops rolled, indexing the operand
    # arrays through select chains (the 32-head FP4 decode kernel ran 37x
    # slower than its bf16 build)
    "-mllvm", "-pragma-unroll-threshold=65536",
    "-Wall", "-Wno-unused-function",
]


def build(verbose: bool = False) -> str:
    """Compile the library (always; callers rely on a fresh build) and return its path."""
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    tmp = LIB + ".tmp"
    cmd = [hipcc, *HIPCC_FLAGS, "-I", INCLUDE, SRC, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + res.stdout + res.stderr)
    # a rolled operand loop indexes register arrays through select chains
    # (tens of times slower); every loop marked for unrolling must unroll
    if "loop not unrolled" in res.stderr:
        raise RuntimeError("hipcc left a loop marked for unrolling rolled:\n" + res.stderr)
    if verbose:
        print(res.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
