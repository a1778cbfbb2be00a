"""The C ABI without a GPU: the library loads, exports every symbol the header
declares, its struct layout matches the binding, and argument validation
answers before any launch. Also host-side checks of the input generator."""

from __future__ import annotations

import ctypes
import os
import re
import subprocess
import sys
import tempfile

import numpy as np
import torch
import pytest

from gram_memory_layer_engram_amd import workloads as W
from oracle import engram_oracle as o

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "engram.h")


@pytest.fixture(scope="module")
def lib():
    from gram_memory_layer_engram_amd import build, engram

    if not os.path.exists(engram.LIB_PATH):
        build.build()
    return engram.load_library()


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(engram_\w+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = _declared_functions()
    for want in ("engram_lookup", "engram_wkv", "engram_gate", "engram_forward",
                 "engram_mx_quantize", "engram_wkv_workspace_size",
                 "engram_forward_workspace_size", "engram_abi_version", "engram_status_string"):
        assert want in names


def test_library_exports_every_declared_symbol(lib):
    from gram_memory_layer_engram_amd import engram

    for name in _declared_functions():
        assert hasattr(lib, name), name
        assert name in engram.EXPORTS, name
    out = subprocess.run(["nm", "-D", "--defined-only", engram.LIB_PATH], capture_output=True, text=True)
    exported = set(re.findall(r"\bT (engram_\w+)", out.stdout))
    assert set(_declared_functions()) <= exported


def test_forward_args_layout_matches_c():
    from gram_memory_layer_engram_amd import engram

    fields = [f for f, _ in engram.ForwardArgs._fields_]
    src = ['#include <stdio.h>', '#include <stddef.h>', f'#include "{HEADER}"', "int main(void) {",
           'printf("%zu\\n", sizeof(engram_forward_args));']
    for f in fields:
        src.append(f'printf("%zu\\n", offsetof(engram_forward_args, {f}));')
    src.append("return 0; }")
    with tempfile.TemporaryDirectory() as d:
        c = os.path.join(d, "layout.c")
        exe = os.path.join(d, "layout")
        open(c, "w").write("\n".join(src))
        subprocess.run(["gcc", "-std=c99", c, "-o", exe], check=True)
        vals = [int(x) for x in subprocess.run([exe], capture_output=True, text=True, check=True).stdout.split()]
    assert vals[0] == ctypes.sizeof(engram.ForwardArgs)
    for f, off in zip(fields, vals[1:]):
        assert getattr(engram.ForwardArgs, f).offset == off, f


def test_status_strings_and_version(lib):
    assert lib.engram_abi_version() == 5
    assert lib.engram_status_string(0) == b"ok"
    assert lib.engram_status_string(1) == b"invalid argument"
    assert lib.engram_status_string(2) == b"unsupported shape"
    assert lib.engram_status_string(3) == b"HIP runtime error"
    assert lib.engram_status_string(4) == b"input larger than the fixed scratch buffer"
    assert lib.engram_status_string(99) == b"unknown status"


def test_validation_answers_before_any_launch(lib):
    # T = 0 is a no-op even with NULL tensors
    assert lib.engram_lookup(None, 10, 128, None, 16, 1, 0, 16, None, None, None) == 0
    assert lib.engram_gate(None, None, None, None, None, 0, 4, 4096, 1e-6, 1e-6, None, None, None) == 0
    assert lib.engram_wkv(None, 0, 2048, None, None, 0, 20480, None, None, 0, None) == 0
    assert lib.engram_mx_quantize(None, 0, 2048, None, None, None) == 0
    # bad arguments
    assert lib.engram_lookup(None, 10, 128, None, 16, 1, -1, 16, None, None, None) == 1
    assert lib.engram_lookup(None, 10, 12, None, 16, 1, 4, 16, None, None, None) == 2   # head_dim % 8
    assert lib.engram_lookup(None, 10, 128, None, 16, 1, 4, 16, None, None, None) == 1  # NULL table
    assert lib.engram_gate(None, None, None, None, None, 4, 4, 4100, 1e-6, 1e-6, None, None, None) == 2
    assert lib.engram_gate(None, None, None, None, None, 4, 9, 4096, 1e-6, 1e-6, None, None, None) == 2
    assert lib.engram_gate(None, None, None, None, None, 4, 4, 4096, 1e-6, 1e-6, None, None, None) == 1
    assert lib.engram_wkv(None, 4, 2048, None, None, 7, 20480, None, None, 0, None) == 1  # bad format
    assert lib.engram_mx_quantize(None, 4, 100, None, None, None) == 2
    # misaligned pointers are refused (never dereferenced)
    assert lib.engram_gate(0x1002, 0x2000, 0x3000, 0x4000, None, 4, 4, 4096, 1e-6, 1e-6, 0x5000,
                           None, None) == 1
    # fp8 tables: head_dim a multiple of 32, scales required
    assert lib.engram_lookup_fp8(None, None, 10, 128, None, 16, 1, 0, 16, None, None, None) == 0
    assert lib.engram_lookup_fp8(0x1000, 0x2000, 10, 48, 0x3000, 16, 1, 4, 16, 0x4000, None, None) == 2
    assert lib.engram_lookup_fp8(0x1000, None, 10, 128, 0x3000, 16, 1, 4, 16, 0x4000, None, None) == 1
    assert lib.engram_lookup_fp8(0x1008, 0x2000, 10, 128, 0x3000, 16, 1, 4, 16, 0x4000, None, None) == 1
    # fused projection + gate partials: dim % 256, hc range, then the wkv and gate checks
    P = 0x1000
    assert lib.engram_wkv_gate_partials(P, 4, 256, P, None, 0, 2, 200, P, P, P, P, P, None, 0, None) == 2
    assert lib.engram_wkv_gate_partials(P, 4, 256, P, None, 0, 9, 256, P, P, P, P, P, None, 0, None) == 2
    assert lib.engram_wkv_gate_partials(P, 4, 256, P, None, 0, 0, 256, P, P, P, P, P, None, 0, None) == 1
    assert lib.engram_wkv_gate_partials(P, 4, 256, None, None, 0, 2, 256, P, P, P, P, P, None, 0, None) == 1
    assert lib.engram_wkv_gate_partials(P, 4, 256, P, None, 0, 2, 256, P, P, P, P, None, None, 0, None) == 1
    assert lib.engram_wkv_gate_partials(None, 0, 256, None, None, 0, 2, 256, None, None, None, None, None,
                                        None, 0, None) == 0
    # MXFP8 needs its workspace (x's codes and scales): none given -> EINVAL
    assert lib.engram_wkv_gate_partials(P, 4, 256, P, P, 1, 2, 256, P, P, P, P, P, None, 0, None) == 1
    # measurement probes: argument checks only (a valid call would launch)
    assert lib.engram_probe_mfma(7, 10, P, None, None) == 1        # unknown format
    assert lib.engram_probe_mfma(0, 0, P, None, None) == 1         # iters <= 0
    assert lib.engram_probe_mfma(0, 10, None, None, None) == 1     # no out
    assert lib.engram_probe_read(P, 17, P, None) == 1              # not a multiple of 16
    assert lib.engram_probe_read(None, 0, P, None) == 0            # empty: no launch
    assert lib.engram_probe_read(0x1008, 32, P, None) == 1         # misaligned source
    assert lib.engram_probe_stream(None, None, 0, 1, None) == 0
    assert lib.engram_probe_stream(P, 0x2008, 32, 1, None) == 1    # misaligned destination
    assert lib.engram_probe_stream(P, 0x2000, 32, 5, None) == 1    # ratio outside 1..4
    assert lib.engram_probe_stream(P, 0x2000, 24, 1, None) == 1    # not a multiple of 16


def test_host_alloc_validation(lib):
    """engram_host_alloc refuses a zero size and NULL out-pointers before
    touching the runtime; engram_host_free(NULL) is a no-op."""
    h, d = ctypes.c_void_p(), ctypes.c_void_p()
    assert lib.engram_host_alloc(0, ctypes.byref(h), ctypes.byref(d)) == 1
    assert lib.engram_host_alloc(4096, None, ctypes.byref(d)) == 1
    assert lib.engram_host_alloc(4096, ctypes.byref(h), None) == 1
    assert lib.engram_host_free(None) == 0
    # the background lookup validates like engram_lookup
    assert lib.engram_lookup_background(None, 10, 128, None, 16, 1, 0, 16, None, None, None) == 0
    assert lib.engram_lookup_background(None, 10, 12, None, 16, 1, 4, 16, None, None, None) == 2
    assert lib.engram_lookup_background(None, 10, 128, None, 16, 1, 4, 16, None, None, None) == 1


def test_workspace_sizes(lib):
    from gram_memory_layer_engram_amd import engram

    assert lib.engram_wkv_workspace_size(16, 2048, 20480, engram.W_BF16) == 0
    ws = lib.engram_wkv_workspace_size(16, 2048, 20480, engram.W_MXFP8)
    assert ws >= 16 * 2048 + 16 * 64 and ws % 256 == 0
    a = engram.ForwardArgs()
    a.T, a.hc, a.dim, a.n_cols, a.head_dim, a.w_format = 8192, 4, 4096, 16, 128, engram.W_BF16
    need = lib.engram_forward_workspace_size(ctypes.byref(a))
    assert need >= 8192 * 2048 * 2 + 8192 * 20480 * 2


def test_forward_rejects_unknown_options(lib):
    """Only ENGRAM_FORWARD_STORE_KV is a known option bit; any other is
    EINVAL before any argument is looked at or anything is launched."""
    from gram_memory_layer_engram_amd import engram

    for fn in (lib.engram_forward, lib.engram_forward_single_launch):
        for bad in (2, 4, 1 | 8, -1):
            a = engram.ForwardArgs()
            a.options = bad
            assert fn(ctypes.byref(a), None, 0, None) == 1


# ------------------------------------------------------ input generator --


def test_generator_table_sizes_follow_the_layout_rule():
    for name, wl in W.WORKLOADS.items():
        sizes, offsets = o.layout_primes(wl.vocab, wl.max_ngram, wl.n_heads)
        assert W.column_sizes(wl) == sizes[0], name
        assert W.column_offsets(wl) == offsets[0], name


def test_generator_ids_and_masks():
    for name in ("tiny", "mid", "prefill", "decode_t16", "long"):
        wl = W.WORKLOADS[name]
        T = min(wl.T, 4096)
        ids = W.make_ids(wl, T=T)
        sizes, offs = W.column_sizes(wl), W.column_offsets(wl)
        for c in range(wl.C):
            assert np.all(ids[:, c] >= offs[c]) and np.all(ids[:, c] < offs[c] + sizes[c])
        assert np.array_equal(ids, W.make_ids(wl, T=T))  # seeded
        m = W.make_mask(wl)
        if wl.mask_frac is None:
            assert m is None
        else:
            assert m.shape == (wl.T,) and int((~m).sum()) == wl.mask_false
    # Zipf ids concentrate on few rows (hot rows), uniform ids do not
    z = W.make_ids(W.WORKLOADS["prefill"])[:, 0]
    u = W.make_ids(W.WORKLOADS["mid"])[:, 0]
    assert len(np.unique(z)) < 0.6 * len(z) and len(np.unique(u)) > 0.99 * len(u)


def test_generator_values():
    wl = W.WORKLOADS["tiny"]
    inp = W.make_inputs(wl)
    assert abs(inp["table"].float().std().item() - 0.02) < 0.002
    assert abs(inp["hidden"].float().std().item() - 1.0) < 0.05
    assert abs(inp["q"].float().mean().item() - 1.0) < 0.02
    wq, ws = W.make_weight(W.WORKLOADS["decode_t16"].with_T(1))
    assert wq.shape == (20480, 2048) and ws.shape == (640, 64)
    assert int(ws.min()) >= 119 and int(ws.max()) <= 127


# ------------------------------------------------------- no fallback path --


def test_binding_has_no_cpu_fallback(tmp_path):
    """Without the built library the binding raises instead of computing
    anything, and with it, host tensors are refused (every step runs in the
    HIP kernels)."""
    from gram_memory_layer_engram_amd import engram

    saved = engram._lib
    try:
        engram._lib = None
        with pytest.raises(RuntimeError, match="not built"):
            engram.load_library(str(tmp_path / "libengram.so"))
    finally:
        engram._lib = saved
    table = torch.zeros((8, 32), dtype=torch.bfloat16)
    ids = torch.zeros((2, 3), dtype=torch.int32)
    with pytest.raises(ValueError, match="device tensors"):
        engram.lookup(table, ids, rows_out=torch.empty((2, 3, 32), dtype=torch.bfloat16))


def test_bench_refuses_more_than_one_gpu():
    """bench.py measures one GPU; asked for more it exits with status 2 and
    says why, before touching any device."""
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120, cwd=root)
    assert r.returncode == 2
    assert "one GPU" in (r.stdout + r.stderr)
