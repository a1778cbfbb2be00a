"""Seeded synthetic inputs for the Engram forward hot path.

This module only draws inputs; it holds none of the layer's arithmetic (no
gather, no projection, no gate, no quantization rule). Both the HIP path (its
tests and the benchmark) and the CPU oracle receive exactly the tensors built
here. Number-format conversions of random draws (float -> bf16, float ->
float8_e4m3fn) are torch's own casts.

Workloads (one Engram layer, HBM-resident per-column tables concatenated into
one ``[rows, head_dim]`` bf16 table, as on "vllm.models.deepseek_v4_1.common.
engram", ``ParallelEngramEmbedding``):

=========  ======  =====  ==  =====  =====  ==  ======  =======  =======  ====
name       T       dim    hc  ngram  heads  C   hd      vocab    wkv      ids
=========  ======  =====  ==  =====  =====  ==  ======  =======  =======  ====
tiny       64      256    2   3      4      8   32      10000    bf16     unif
mid        2048    2048   4   3      8      16  64      262144   bf16     unif
prefill    8192    4096   4   3      8      16  128     2097152  bf16     zipf
decode_tN  1/4/16/64 4096 4   3      8      16  128     2097152  mxfp8    unif
long       32768   7168   4   4      8      24  128     4194304  mxfp8    zipf
=========  ======  =====  ==  =====  =====  ==  ======  =======  =======  ====

Per-column table sizes are the first C distinct primes at or above ``vocab``
(the bucket-size rule of ``EngramLayout`` for a single layer); the global id
of column c is ``offset_c + local`` with ``offset`` the exclusive cumsum.

Values: tables N(0, 0.02), bf16 W N(0, 0.02), MXFP8 W codes float8_e4m3fn of
N(0, 1) with E8M0 block bytes 127 + U{-8..0}, hidden N(0, 1), q/k N(1, 0.1),
all bf16. Masks have exactly round(frac * T) False positions at seeded places.
Zipf(1.1) ids: rank ~ Zipf(1.1) redrawn until rank <= p_c, then
``local = ((rank-1) * a_c + b_c) mod p_c`` with seeded a_c in [1, p_c),
b_c in [0, p_c) (a bijection since p_c is prime).

Seeds: ``SeedSequence([20261202, cfg_id, variant])`` spawns children in the
order table, ids, W, W-scales, hidden, q, k, mask, kv (a stand-alone kv input
for exercising the gate step by itself: N(0, kv_std) bf16).
"""

from __future__ import annotations

from dataclasses import dataclass, replace

import numpy as np
import torch

SEED_BASE = 20261202


@dataclass(frozen=True)
class Workload:
    name: str
    cfg_id: int
    T: int
    dim: int
    hc: int
    max_ngram: int
    n_heads: int
    head_dim: int
    vocab: int
    w_format: str  # "bf16" or "mxfp8"
    ids_dist: str  # "uniform" or "zipf"
    mask_frac: float | None  # None: no mask tensor
    eps: float = 1e-6
    clamp: float = 1e-6

    @property
    def C(self) -> int:
        return (self.max_ngram - 1) * self.n_heads

    @property
    def K(self) -> int:
        return self.C * self.head_dim

    @property
    def N(self) -> int:
        return (self.hc + 1) * self.dim

    @property
    def mask_false(self) -> int:
        return 0 if self.mask_frac is None else int(round(self.mask_frac * self.T))

    def with_T(self, T: int) -> "Workload":
        return replace(self, T=T)


WORKLOADS = {
    "tiny": Workload("tiny", 1, 64, 256, 2, 3, 4, 32, 10000, "bf16", "uniform", 0.10),
    "mid": Workload("mid", 2, 2048, 2048, 4, 3, 8, 64, 262144, "bf16", "uniform", 0.05),
    "prefill": Workload("prefill", 3, 8192, 4096, 4, 3, 8, 128, 2097152, "bf16", "zipf", None),
    "decode_t1": Workload("decode_t1", 4, 1, 4096, 4, 3, 8, 128, 2097152, "mxfp8", "uniform", 0.20),
    "decode_t4": Workload("decode_t4", 4, 4, 4096, 4, 3, 8, 128, 2097152, "mxfp8", "uniform", 0.20),
    "decode_t16": Workload("decode_t16", 4, 16, 4096, 4, 3, 8, 128, 2097152, "mxfp8", "uniform", 0.20),
    "decode_t64": Workload("decode_t64", 4, 64, 4096, 4, 3, 8, 128, 2097152, "mxfp8", "uniform", 0.20),
    "long": Workload("long", 5, 32768, 7168, 4, 4, 8, 128, 4194304, "mxfp8", "zipf", 0.10),
}


def _is_prime(n: int) -> bool:
    if n < 2:
        return False
    for p in (2, 3, 5, 7, 11, 13, 17, 19, 23, 29, 31, 37):
        if n % p == 0:
            return n == p
    d, s = n - 1, 0
    while d % 2 == 0:
        d //= 2
        s += 1
    for a in (2, 3, 5, 7, 11, 13, 17, 19, 23, 29, 31, 37):  # exact below 3.3e24
        x = pow(a, d, n)
        if x in (1, n - 1):
            continue
        for _ in range(s - 1):
            x = x * x % n
            if x == n - 1:
                break
        else:
            return False
    return True


def column_sizes(wl: Workload) -> list[int]:
    """Row counts of the C per-column tables: the first C primes >= vocab."""
    out, n = [], wl.vocab
    while len(out) < wl.C:
        if _is_prime(n):
            out.append(n)
        n += 1
    return out


def column_offsets(wl: Workload) -> list[int]:
    sizes = column_sizes(wl)
    return [int(x) for x in np.cumsum([0] + sizes[:-1])]


def num_rows(wl: Workload) -> int:
    return int(sum(column_sizes(wl)))


def _seeds(wl: Workload, variant: int) -> list[int]:
    ss = np.random.SeedSequence([SEED_BASE, wl.cfg_id, variant])
    return [int(c.generate_state(1, dtype=np.uint64)[0] & 0x7FFFFFFFFFFFFFFF) for c in ss.spawn(11)]


def _gen(device, seed):
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def make_table(wl: Workload, device="cpu", variant: int = 0) -> torch.Tensor:
    """``[rows, head_dim]`` bf16, N(0, 0.02), drawn in 2**20-row chunks."""
    R = num_rows(wl)
    g = _gen(device, _seeds(wl, variant)[0])
    table = torch.empty((R, wl.head_dim), dtype=torch.bfloat16, device=device)
    chunk = 1 << 20
    for r0 in range(0, R, chunk):
        r1 = min(R, r0 + chunk)
        x = torch.randn((r1 - r0, wl.head_dim), generator=g, device=device, dtype=torch.float32)
        table[r0:r1] = (x * 0.02).to(torch.bfloat16)
    return table


def make_table_fp8(wl: Workload, device="cpu", variant: int = 0):
    """An fp8 table of the workload's shape: (e4m3fn codes as uint8
    ``[rows, head_dim]``, ue8m0 bytes ``[rows, head_dim / 32]``). Codes are
    N(0, 1) cast to e4m3fn, scale bytes 127 + U{-12 .. -5}, so element values
    have the magnitude of the bf16 tables' N(0, 0.02). 2**20-row chunks."""
    R = num_rows(wl)
    s = _seeds(wl, variant)
    g, gs = _gen(device, s[9]), _gen(device, s[10])
    codes = torch.empty((R, wl.head_dim), dtype=torch.uint8, device=device)
    chunk = 1 << 20
    for r0 in range(0, R, chunk):
        r1 = min(R, r0 + chunk)
        x = torch.randn((r1 - r0, wl.head_dim), generator=g, device=device, dtype=torch.float32)
        codes[r0:r1] = x.to(torch.float8_e4m3fn).view(torch.uint8)
    scales = (127 + torch.randint(-12, -4, (R, wl.head_dim // 32), generator=gs, device=device)).to(torch.uint8)
    return codes, scales


def make_ids(wl: Workload, T: int | None = None, variant: int = 0) -> np.ndarray:
    """``[T, C]`` int32 global row ids (host array)."""
    T = wl.T if T is None else T
    rng = np.random.default_rng(_seeds(wl, variant)[1])
    sizes = column_sizes(wl)
    offs = column_offsets(wl)
    ids = np.empty((T, wl.C), dtype=np.int64)
    for c, (p, off) in enumerate(zip(sizes, offs)):
        if wl.ids_dist == "uniform":
            local = rng.integers(0, p, size=T)
        else:
            rank = rng.zipf(1.1, size=T)
            bad = rank > p
            while bad.any():
                rank[bad] = rng.zipf(1.1, size=int(bad.sum()))
                bad = rank > p
            a = int(rng.integers(1, p))
            b = int(rng.integers(0, p))
            local = ((rank - 1) * a + b) % p
        ids[:, c] = off + local
    return ids.astype(np.int32)


def make_weight(wl: Workload, device="cpu", variant: int = 0):
    """wkv weight ``[N, K]``: bf16, or (e4m3fn codes as uint8, E8M0 uint8 ``[N/32, K/32]``)."""
    s = _seeds(wl, variant)
    g = _gen(device, s[2])
    w = torch.randn((wl.N, wl.K), generator=g, device=device, dtype=torch.float32)
    if wl.w_format == "bf16":
        return (w * 0.02).to(torch.bfloat16), None
    codes = w.to(torch.float8_e4m3fn).view(torch.uint8)
    gs = _gen(device, s[3])
    scales = (127 + torch.randint(-8, 1, (wl.N // 32, wl.K // 32), generator=gs, device=device)).to(torch.uint8)
    return codes, scales


def make_hidden(wl: Workload, T: int | None = None, device="cpu", variant: int = 0) -> torch.Tensor:
    T = wl.T if T is None else T
    g = _gen(device, _seeds(wl, variant)[4])
    return torch.randn((T, wl.hc, wl.dim), generator=g, device=device, dtype=torch.float32).to(torch.bfloat16)


def make_qk(wl: Workload, device="cpu", variant: int = 0):
    s = _seeds(wl, variant)
    out = []
    for seed in (s[5], s[6]):
        g = _gen(device, seed)
        x = torch.randn((wl.hc, wl.dim), generator=g, device=device, dtype=torch.float32)
        out.append((1.0 + 0.1 * x).to(torch.bfloat16))
    return tuple(out)


def make_mask(wl: Workload, T: int | None = None, variant: int = 0):
    """bool ``[T]`` with exactly round(frac*T) False entries, or None."""
    if wl.mask_frac is None:
        return None
    T = wl.T if T is None else T
    rng = np.random.default_rng(_seeds(wl, variant)[7])
    m = np.ones(T, dtype=bool)
    m[rng.permutation(T)[: int(round(wl.mask_frac * T))]] = False
    return m


def kv_std(wl: Workload) -> float:
    """Typical kv standard deviation of the workload's projection."""
    if wl.w_format == "bf16":
        return 0.02 * 0.02 * wl.K ** 0.5
    return 0.35


def make_kv(wl: Workload, T: int | None = None, device="cpu", variant: int = 0) -> torch.Tensor:
    """``[T, (hc+1)*dim]`` bf16 N(0, kv_std): a gate-step input on its own."""
    T = wl.T if T is None else T
    g = _gen(device, _seeds(wl, variant)[8])
    x = torch.randn((T, wl.N), generator=g, device=device, dtype=torch.float32)
    return (x * kv_std(wl)).to(torch.bfloat16)


def make_inputs(wl: Workload, device="cpu", variant: int = 0, table=None, weight=None):
    """All inputs of one forward on ``device`` (the table and weight may be
    passed in to share them between variants)."""
    if table is None:
        table = make_table(wl, device, variant)
    if weight is None:
        weight = make_weight(wl, device, variant)
    w, w_scales = weight
    ids = torch.from_numpy(make_ids(wl, variant=variant)).to(device)
    hidden = make_hidden(wl, device=device, variant=variant)
    q, k = make_qk(wl, device, variant)
    m = make_mask(wl, variant=variant)
    mask = None if m is None else torch.from_numpy(m).to(device)
    return {
        "table": table, "ids": ids, "w": w, "w_scales": w_scales,
        "hidden": hidden, "q": q, "k": k, "mask": mask,
    }
