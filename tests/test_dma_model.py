"""Host model of the prefill GEMMs' DMA offsets (CPU only).

tests/dma_model.cpp evaluates the offset functions the GEMM kernels use
(csrc/gemm_dma.h) for every DMA of ragged bf16 and MXFP8 launches and checks
that each is a whole in-range piece holding the right data, or lies past the
descriptor's range (zero-filled), with nothing carried in the unchecked
scalar offset.
"""

from __future__ import annotations

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_gemm_dma_offsets_stay_in_range(tmp_path):
    cxx = shutil.which("g++") or shutil.which("c++")
    if cxx is None:
        pytest.skip("no host C++ compiler")
    exe = tmp_path / "dma_model"
    subprocess.run([cxx, "-O2", "-std=c++17", "-I/opt/rocm/include", "-D__HIP_PLATFORM_AMD__",
                    os.path.join(ROOT, "tests", "dma_model.cpp"), "-o", str(exe)], check=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "0 failures" in r.stdout
