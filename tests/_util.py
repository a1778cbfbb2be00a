"""Helpers shared by the tests (no method arithmetic here)."""

from __future__ import annotations

import numpy as np
import torch


def bits(t: torch.Tensor) -> np.ndarray:
    """bf16 tensor (any device) -> numpy uint16 bit patterns."""
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def u8(t: torch.Tensor) -> np.ndarray:
    return t.detach().contiguous().cpu().numpy().astype(np.uint8)


def from_bits(a: np.ndarray, device) -> torch.Tensor:
    """numpy uint16 bf16 bits -> bf16 tensor on device."""
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(device)


def bf16_values(b: np.ndarray) -> np.ndarray:
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def assert_close(got: np.ndarray, ref: np.ndarray, rel: float, abs_: float, what: str):
    """Elementwise |got - ref| <= abs + rel*|ref| (allclose form)."""
    err = np.abs(got - ref)
    lim = abs_ + rel * np.abs(ref)
    bad = err > lim
    if bad.any():
        i = np.unravel_index(np.argmax(err - lim), err.shape)
        raise AssertionError(
            f"{what}: {int(bad.sum())} of {bad.size} elements out of tolerance "
            f"(rel {rel}, abs {abs_}); worst at {i}: got {got[i]!r}, ref {ref[i]!r}")


def ulp_distance_bf16(a_bits: np.ndarray, b_bits: np.ndarray) -> np.ndarray:
    """Distance in bf16 steps between two bf16 bit arrays (sign-magnitude order)."""
    def ordered(x):
        x = x.astype(np.int64)
        return np.where(x & 0x8000, -(x & 0x7FFF), x & 0x7FFF)
    return np.abs(ordered(a_bits) - ordered(b_bits))


def sample_tokens(T: int, n: int, seed: int = 0, tile: int = 256) -> np.ndarray:
    """A seeded sorted sample of token indices: both ends, one token from
    every ``tile``-token tile (so every token tile of a tiled kernel has a
    checked output, the ragged last one included), then random others up to
    ``n`` in all (more when there are more tiles than that)."""
    if T <= n:
        return np.arange(T)
    rng = np.random.default_rng(seed)
    starts = np.arange(0, T, tile)
    per_tile = starts + rng.integers(0, np.minimum(tile, T - starts))
    chosen = np.unique(np.concatenate([[0, T - 1], per_tile]))
    rest = np.setdiff1d(np.arange(T), chosen)
    extra = max(0, n - len(chosen))
    if extra:
        chosen = np.concatenate([chosen, rng.choice(rest, size=extra, replace=False)])
    return np.sort(chosen)
