"""CPU check of the grouped GEMM's LDS maps (csrc/lds_layout.h): builds
tests/lds_layout_check.cpp with g++ against the header the kernels include and
runs it.  It requires the DMA placement of every operand tile to be a bijection,
every MFMA fragment read to deliver the elements the 32x32x16 bf16 operand
layout needs (K-contiguous ds_read_b128 and MN-contiguous ds_read_b64_tr_b16),
every read phase to cover the 64 LDS banks without conflicts, and the epilogue
staging map to be a conflict-free bijection."""
import os
import shutil
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_lds_maps():
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ not available")
    exe = os.path.join(tempfile.mkdtemp(prefix="moe_lds_"), "lds_layout_check")
    cmd = [gxx, "-std=c++17", "-O1", "-D__host__=", "-D__device__=", "-D__forceinline__=inline",
           "-I", os.path.join(ROOT, "moe_expert_layer_router_amd", "csrc"),
           os.path.join(ROOT, "tests", "lds_layout_check.cpp"), "-o", exe]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-3000:]
    run = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    print(run.stdout)
    assert run.returncode == 0, run.stdout[-3000:]
