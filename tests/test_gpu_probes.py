"""The measurement probes through the C ABI (they are not steps of the layer:
bench.py uses them for measured ceilings). Each is checked against what it
must compute: the MFMA loop's accumulator sums in closed form, the streaming
read's XOR of the buffer, the streaming copy bit for bit."""

from __future__ import annotations

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _E():
    from gram_memory_layer_engram_amd import engram as E
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    E.load_library()
    return E


@pytest.mark.parametrize("fmt,per_step", [(0, 2.0 ** -12), (1, 64.0)])
def test_probe_mfma_closed_form(fmt, per_step):
    """Each thread's sum of its 128 accumulators after `iters` steps is
    128 * iters * (2^-12 for bf16 2^-8 operands, 64 for e4m3 1.0 at scale
    2^0), exact in fp32 at these sizes; the flop count matches the grid."""
    E = _E()
    out = E.probe_out()
    out.fill_(-1)
    iters = 1000
    flops = E.probe_mfma(fmt, iters, out)
    torch.cuda.synchronize()
    flop_per_mfma = 2 * 32 * 32 * (64 if fmt == 1 else 16)
    waves = flops / (iters * 8 * flop_per_mfma)
    assert waves == int(waves) and waves >= 4
    threads = int(waves) * 64
    vals = out.view(torch.float32).cpu().numpy()
    assert np.all(vals[:threads] == np.float32(128 * iters * per_step))


@pytest.mark.parametrize("words", [3 * 2 ** 20 + 4, 16 * 2 ** 20 + 12])
def test_probe_read(words):
    """Sizes with a ragged last sweep (the smaller one is below one 64 MiB
    sweep, so clamped duplicate loads stand in for most pieces)."""
    E = _E()
    g = torch.Generator(device=DEV).manual_seed(words)
    buf = torch.randint(-2 ** 31, 2 ** 31 - 1, (words,), generator=g, dtype=torch.int32, device=DEV)
    out = E.probe_out()
    out.zero_()
    E.probe_read(buf, out)
    torch.cuda.synchronize()
    want = np.bitwise_xor.reduce(buf.cpu().numpy().view(np.uint32))
    got = np.bitwise_xor.reduce(out.cpu().numpy().view(np.uint32))
    assert got == want


@pytest.mark.parametrize("ratio", [1, 2, 3, 4])
@pytest.mark.parametrize("words", [2 ** 20 + 4, 9 * 2 ** 20 + 8])
def test_probe_stream(words, ratio):
    """dst piece d = XOR of src pieces j*n + d, j < ratio (ratio 1: a copy)."""
    E = _E()
    g = torch.Generator(device=DEV).manual_seed(words + ratio)
    src = torch.randint(-2 ** 31, 2 ** 31 - 1, (ratio * words,), generator=g, dtype=torch.int32, device=DEV)
    dst = torch.full((words,), 7, dtype=torch.int32, device=DEV)
    E.probe_stream(src, dst, ratio)
    torch.cuda.synchronize()
    want = np.bitwise_xor.reduce(src.cpu().numpy().view(np.uint32).reshape(ratio, words), axis=0)
    assert np.array_equal(dst.cpu().numpy().view(np.uint32), want)
