"""engram_forward_noalloc against engram_forward (GPU).

The entry point for callers that cannot allocate runs the same launches on
the library's fixed device scratch instead of a caller workspace, so its
outputs must equal engram_forward's bit for bit; both are also held to the
oracle's output tolerance. Two calls in a row on each route, the second with
fewer tokens (the buffer keeps the first call's contents), and an input too
large for the buffer refused before any launch.
"""

from __future__ import annotations

import ctypes
import sys

import numpy as np
import pytest
import torch

from oracle import engram_oracle as o
from tests._util import assert_close, bf16_values, bits, u8

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _E():
    from gram_memory_layer_engram_amd import engram as E
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    E.load_library()
    return E


def _case(wfmt, T, dim, hc, seed, C=8, hd=128, R=3001):
    g = torch.Generator(device=DEV).manual_seed(seed)
    K, N = C * hd, (hc + 1) * dim
    table = (torch.randn((R, hd), generator=g, device=DEV) * 0.02).to(torch.bfloat16)
    ids = torch.randint(0, R, (T, C), generator=g, device=DEV, dtype=torch.int32)
    if wfmt == "bf16":
        w = (torch.randn((N, K), generator=g, device=DEV) * 0.02).to(torch.bfloat16)
        ws = None
    else:
        w = torch.randn((N, K), generator=g, device=DEV).to(torch.float8_e4m3fn).view(torch.uint8)
        ws = (127 + torch.randint(-8, 1, (N // 32, K // 32), generator=g, device=DEV)).to(torch.uint8)
    hidden = torch.randn((T, hc, dim), generator=g, device=DEV).to(torch.bfloat16)
    q = (1 + 0.1 * torch.randn((hc, dim), generator=g, device=DEV)).to(torch.bfloat16)
    k = (1 + 0.1 * torch.randn((hc, dim), generator=g, device=DEV)).to(torch.bfloat16)
    mask = torch.rand((T,), generator=g, device=DEV) > 0.2
    return dict(table=table, ids=ids, w=w, ws=ws, hidden=hidden, q=q, k=k, mask=mask)


def _sub(c, T):
    """The first T tokens of a case, as fresh contiguous tensors."""
    d = dict(c)
    for key in ("ids", "hidden", "mask"):
        d[key] = c[key][:T].contiguous()
    return d


def _run_both(E, c, store_kv=False):
    args = (c["table"], c["ids"], c["w"], c["ws"], c["hidden"], c["q"], c["k"], c["mask"])
    T, hc = c["hidden"].shape[:2]
    g_ref = torch.empty((T, hc), dtype=torch.float32, device=DEV)
    g_na = torch.empty((T, hc), dtype=torch.float32, device=DEV)
    ref = E.forward(*args, gate_out=g_ref, store_kv=store_kv)
    out = torch.full_like(c["hidden"], 7.0)
    L = E.load_library()
    a = E.forward_args(*args, 1e-6, 1e-6, out, g_na, None, None, store_kv)
    st = L.engram_forward_noalloc(ctypes.byref(a), torch.cuda.current_stream().cuda_stream)
    assert st == E.ENGRAM_OK, st
    torch.cuda.synchronize()
    return ref, out, g_ref, g_na


@pytest.mark.parametrize("wfmt,T1,T2,dim,hc,store_kv", [
    ("bf16", 300, 70, 512, 2, False),      # GEMM with the gate epilogue, then a smaller call
    ("bf16", 300, 70, 512, 2, True),       # kv stored, plain gate
    ("mxfp8", 64, 5, 1024, 3, False),      # fused gather + quantize, decode GEMV
    ("bf16", 64, 9, 512, 2, False),        # bf16 weight-streaming GEMV, plain gate
    ("mxfp8", 257, 16, 512, 2, False),     # scaled GEMM (epilogue), then the decode GEMV
])
def test_noalloc_forward_equals_forward(wfmt, T1, T2, dim, hc, store_kv):
    E = _E()
    print(f"[gpu-test] noalloc {wfmt} T={T1}->{T2} dim={dim} hc={hc} store_kv={store_kv}", flush=True)
    sys.stdout.flush()
    c = _case(wfmt, T1, dim, hc, seed=8000 + T1 + dim + hc)
    for T in (T1, T2):
        ct = _sub(c, T)
        ref, out, g_ref, g_na = _run_both(E, ct, store_kv)
        assert torch.equal(out.view(torch.int16), ref.view(torch.int16)), T
        assert torch.equal(g_na, g_ref), T
        want = o.forward(bits(ct["table"]), ct["ids"].cpu().numpy(),
                         bits(ct["w"]) if ct["ws"] is None else u8(ct["w"]),
                         None if ct["ws"] is None else u8(ct["ws"]), bits(ct["hidden"]), bits(ct["q"]),
                         bits(ct["k"]), ct["mask"].cpu().numpy(), 1e-6, 1e-6)
        assert_close(bf16_values(bits(out)), bf16_values(want["out"]), 1e-2, 2e-2, what=f"out T={T}")
        m = ct["mask"].cpu().numpy()
        assert np.array_equal(bits(out)[~m], bits(ct["hidden"])[~m])


def test_noalloc_refuses_inputs_beyond_its_buffer():
    """An input whose scratch exceeds ENGRAM_NOALLOC_SCRATCH_BYTES is refused
    with ENGRAM_ENOSPACE and nothing is written; engram_forward still serves
    it with a caller workspace."""
    E = _E()
    T, dim, hc = 3000, 1024, 3            # K 2048: rows 12.3 MB + kv 24.6 MB > 32 MiB
    c = _case("bf16", T, dim, hc, seed=8100, C=16, hd=128)
    args = (c["table"], c["ids"], c["w"], c["ws"], c["hidden"], c["q"], c["k"], c["mask"])
    a_out = torch.full_like(c["hidden"], 7.0)
    a = E.forward_args(*args, 1e-6, 1e-6, a_out)
    need = E.forward_workspace_size(a) - 65536
    assert need > E.NOALLOC_SCRATCH_BYTES
    L = E.load_library()
    st = L.engram_forward_noalloc(ctypes.byref(a), torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert st == E.ENGRAM_ENOSPACE
    assert bool((a_out == 7.0).all())
    with pytest.raises(ValueError):
        E.forward_noalloc(*args)
    # a call that fits works right after the refused one
    ct = _sub(c, 100)
    ref, out, _, _ = _run_both(E, ct)
    assert torch.equal(out.view(torch.int16), ref.view(torch.int16))


@pytest.mark.parametrize("wfmt,T,dim,hc", [("mxfp8", 16, 1024, 3), ("bf16", 300, 512, 2), ("bf16", 16, 512, 2)])
def test_noalloc_forward_under_graph_capture(wfmt, T, dim, hc):
    """The callers it is for: a forward captured into a HIP graph with no
    allocation inside the capture. The captured engram_forward_noalloc is
    replayed four times, with eager work and synchronizations between the
    replays, and every replay gives the eager call's output bit for bit."""
    E = _E()
    c = _case(wfmt, T, dim, hc, seed=8200 + T + dim)
    args = (c["table"], c["ids"], c["w"], c["ws"], c["hidden"], c["q"], c["k"], c["mask"])
    eager = E.forward_noalloc(*args).clone()
    out = torch.empty_like(c["hidden"])
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        E.forward_noalloc(*args, out=out)          # warm-up on the capture stream's side
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        E.forward_noalloc(*args, out=out)
    for i in range(4):
        out.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), eager.view(torch.int16)), i
        _ = (c["hidden"].float() * 2).sum().item()   # eager work between replays
