"""Host-side AddressSanitizer / UndefinedBehaviorSanitizer builds (CPU only):
the oracle's C code on edge cases, and the HIP library's host code (every
entry point's argument checks) through a driver that makes no GPU call."""
import ctypes
import os
import shutil
import subprocess

import numpy as np
import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SAN_ENV = dict(os.environ, ASAN_OPTIONS="halt_on_error=1:detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1", OMP_NUM_THREADS="2")


def _run(cmd, **kw):
    res = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert res.returncode == 0, f"{cmd[0]} failed ({res.returncode}):\n{res.stdout}\n{res.stderr}"
    return res.stdout


def test_oracle_under_asan_ubsan(tmp_path):
    exe = tmp_path / "oracle_asan"
    _run(["gcc", "-O1", "-g", "-std=c99", "-fopenmp", "-fsanitize=address,undefined",
          "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
          os.path.join(HERE, "sanitize", "oracle_driver.c"),
          os.path.join(ROOT, "oracle", "sparse_attn_ref.c"), "-lm", "-o", str(exe)])
    out = _run([str(exe)], env=SAN_ENV)
    lines = out.strip().splitlines()
    assert "bad rc=1" in lines and "dims rc=2" in lines
    assert any(l.startswith("empty rc=0 sum=0") for l in lines)
    # the sanitized build computes what the ordinary one does
    sums = {l.split(" rc=")[0]: l for l in lines if l.startswith("full")}
    assert len(sums) == 16 and all(" rc=0 " in l for l in sums.values())


@pytest.mark.skipif(not os.path.exists("/opt/rocm/bin/hipcc"), reason="hipcc not installed")
def test_library_host_code_under_asan_ubsan(tmp_path):
    exe = tmp_path / "abi_asan"
    _run(["/opt/rocm/bin/hipcc", "--offload-arch=gfx950", "-O1", "-g", "-std=c++17",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
          "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer",
          "-I", os.path.join(ROOT, "include"),
          os.path.join(ROOT, "sparse_top_latent_amd", "csrc", "sparse_attn.hip"),
          os.path.join(HERE, "sanitize", "abi_driver.cpp"), "-o", str(exe)])
    env = dict(SAN_ENV, ASAN_OPTIONS="halt_on_error=1:detect_leaks=0")
    out = _run([str(exe)], env=env)
    st = {l.split(" ", 1)[1].rsplit(" ", 1)[0]: int(l.rsplit(" ", 1)[1])
          for l in out.splitlines() if l[:2].isdigit()}
    assert st["fwd null dims"] == 1 and st["fwd bad D"] == 3 and st["fwd big K"] == 3
    assert st["fwd neg T"] == 2 and st["fwd null q"] == 1 and st["fwd misaligned out"] == 4
    assert st["fwd zero queries"] == 0 and st["splits -1"] == 8 and st["splits 2 no ws"] == 5
    assert st["splits 2 small ws"] == 5 and st["ws bytes bad"] == 0
    assert st["noalloc S=65"] == 8 and st["noalloc too big"] == 5 and st["check null"] == 1
    assert st["fp4 record bytes"] == 288 and st["topk bad stride"] == 2
    assert "unknown status" in out
