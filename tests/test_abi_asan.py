"""The C ABI's argument checks under AddressSanitizer (CPU only).

csrc/abi.hip is compiled with AddressSanitizer on its host side (the device
side is built as usual: sanitizers apply to host code only), linked with
tests/abi_asan_driver.c and the library's other objects from the in-tree
build, and run: every entry point is
called with bad, edge and empty arguments that the checks answer before any
launch, so no GPU is needed, and any out-of-bounds or use-after-free access
in the validation or workspace arithmetic aborts the run.
"""

from __future__ import annotations

import os
import shutil
import subprocess

import pytest

from gram_memory_layer_engram_amd import build as BUILD

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "gram_memory_layer_engram_amd")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


# every other object the library links (the build's source list, less abi.hip)
OTHERS = [s[:-len(".hip")] for s in BUILD.SOURCES if s != "abi.hip"]


def test_abi_checks_under_asan(tmp_path):
    objs = [os.path.join(PKG, "_build", f"{n}.o") for n in OTHERS]
    if not all(os.path.exists(o) for o in objs):
        pytest.skip("the library's objects are not built (python -m gram_memory_layer_engram_amd.build)")
    if not os.path.exists(HIPCC) or shutil.which("gcc") is None:
        pytest.skip("no hipcc / gcc")
    abi_o = tmp_path / "abi_asan.o"
    drv_o = tmp_path / "drv.o"
    exe = tmp_path / "abi_asan"
    subprocess.run([HIPCC, "--offload-arch=gfx950", "-O1", "-fPIC", "-std=c++17", "-g",
                    "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer",
                    "-Wno-unused-result", "-c", os.path.join(PKG, "csrc", "abi.hip"), "-o", str(abi_o)],
                   check=True, capture_output=True)
    subprocess.run(["gcc", "-std=c11", "-g", "-c", os.path.join(ROOT, "tests", "abi_asan_driver.c"),
                    "-o", str(drv_o)], check=True, capture_output=True)
    subprocess.run([HIPCC, "--offload-arch=gfx950", "-Xarch_host", "-fsanitize=address", str(drv_o), str(abi_o),
                    *objs, "-o", str(exe)], check=True, capture_output=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1")
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120, env=env)
    assert r.returncode == 0, r.stdout + r.stderr
    assert " 0 failures" in r.stdout, r.stdout
