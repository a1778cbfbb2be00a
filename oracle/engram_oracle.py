"""CPU oracle for the Engram layer's forward hot path.

TEST INFRASTRUCTURE ONLY. Nothing in the product path imports, calls or links
this module; only the tests, the smoke check and the CPU-baseline leg of the
benchmark do. It shares no code, tables or constants with the HIP library.

Everything here is written for a reader to check by eye against the pages it
follows, which are the vLLM API pages:

* "vllm.models.deepseek_v4_1.common.engram" -- class ``Engram`` (docstring,
  ``__init__``, ``prepare_embeddings``, ``forward``), class ``EngramLayout``,
  class ``ParallelEngramEmbedding`` (docstring, ``__init__``, ``lookup``,
  ``forward``);
* "vllm.models.deepseek_v41.amd.engram" -- ``_engram_gate_finish_kernel`` and
  ``_engram_gate_partials_kernel`` (the gate math, the only place the pages
  print it in full);
* "vllm.models.deepseek_v41.nvidia.specialized_decode.engram.prefetch" --
  module docstring (the WKV chain quantizes its input to MXFP8);
* "vllm.models.deepseek_v41.amd.mono.attention.gemv" -- module docstring (the
  MXFP8 weight: row-major e4m3 ``[N, K]`` with E8M0 scales per 32x32 block).

Arithmetic is fp64 on the exact values of the bf16 / e4m3 inputs. The only
roundings are the ones the method itself performs: the bf16 outputs (kv and
out) and the MXFP8 activation codes. Library primitives used as steps:
``numpy.matmul`` (the projection) and ``numpy.sum``.

Parity status per function (each is pinned by ``tests/test_oracle_pins.py``):

* ``round_to_bf16``        -- pinned (brute-force nearest search, library cast)
* ``e4m3fn_decode``        -- pinned (closed form, library cast, worked values)
* ``e4m3fn_encode``        -- pinned (brute force, library cast, saturation)
* ``mx_quantize``          -- pinned to the OCP MX v1.0 rule by worked blocks
                              and invariants; the pages do not fix the rule
* ``gather_rows``          -- pinned (direct indexing)
* ``dequant_table_rows``   -- pinned (library fp8 cast, worked extremes in
                              ``tests/golden/fp8_table_dequant.json``)
* ``gather_rows_fp8``      -- pinned (gather and dequant commute; zero rows)
* ``wkv``                  -- pinned (brute-force loops, one-hot scale probes)
* ``gate`` / ``gate_partials`` / ``gate_finish`` -- pinned (closed forms,
                              second route, invariants)
* ``forward``              -- pinned (composition invariants)
* ``layout_primes``        -- pinned (brute-force primality and gaps)
"""

from __future__ import annotations

import math

import numpy as np

# ---------------------------------------------------------------------------
# Number formats
# ---------------------------------------------------------------------------


def bf16_to_f64(bits):
    """bf16 bit patterns (uint16) -> exact float64 values.

    A bf16 number is the upper half of an IEEE binary32 number, so widening is
    exact: put the 16 bits on top of 16 zero bits and read a float32.
    """
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def round_to_bf16(x):
    """float64 values -> nearest bf16 (ties to even) as uint16 bit patterns.

    Output rounding of both bf16 tensors the layer writes (kv, out) is
    round-to-nearest-even; the pages are silent on the mode and this is the
    IEEE default. bf16 keeps 8 significant bits and the binary32 exponent
    range: normal numbers are m * 2**(e-8) with 128 <= m < 256, subnormals are
    multiples of 2**-133. Values beyond the largest finite bf16 round to inf.
    """
    x = np.asarray(x, dtype=np.float64)
    out = np.empty(x.shape, dtype=np.float64)
    finite = np.isfinite(x)
    ax = np.abs(x)
    # exponent e with ax = f * 2**e, 0.5 <= f < 1
    _, e = np.frexp(ax)
    quantum_exp = np.maximum(e - 8, -133)  # normal: 8 bits; subnormal: 2**-133
    scaled = np.ldexp(ax, -quantum_exp)  # exact (power-of-two scaling)
    rounded = np.rint(scaled)  # numpy rint rounds half to even
    mag = np.ldexp(rounded, quantum_exp)
    max_bf16 = float.fromhex("0x1.fep127")
    # the halfway point between max_bf16 and 2**128 rounds to even = 2**128
    mag = np.where(mag > max_bf16, np.inf, mag)
    out = np.where(finite, np.copysign(mag, x), x)
    f32 = out.astype(np.float32)  # exact: every bf16 value is a binary32 value
    bits = (f32.view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        bits = np.where(nan, np.uint16(0x7FC0), bits)
    return bits


# OCP 8-bit floating point, E4M3 "fn" flavour (torch.float8_e4m3fn, the table
# dtype on "vllm.models.deepseek_v4_1.common.engram", ParallelEngramEmbedding):
# 1 sign, 4 exponent bits (bias 7), 3 mantissa bits, no infinities, NaN is
# S.1111.111, largest finite magnitude 1.75 * 2**8 = 448.
E4M3_BIAS = 7
E4M3_MAX = 448.0
E4M3_EMAX = 8  # exponent of the largest normal, 448 = 1.75 * 2**8


def e4m3fn_decode(codes):
    """uint8 e4m3fn codes -> float64 values (NaN for 0x7F / 0xFF)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    exp = (c >> 3) & 0xF
    man = c & 0x7
    normal = np.ldexp(1.0 + man / 8.0, exp - E4M3_BIAS)
    subnormal = np.ldexp(man / 8.0, 1 - E4M3_BIAS)
    val = sign * np.where(exp == 0, subnormal, normal)
    return np.where((c & 0x7F) == 0x7F, np.nan, val)


def _e4m3_magnitudes():
    """The 127 finite non-negative e4m3fn magnitudes, indexed by code 0..126."""
    return e4m3fn_decode(np.arange(127, dtype=np.uint8))


def e4m3fn_encode(v):
    """float64 values -> e4m3fn codes, round to nearest, ties to even code,
    saturating to +-448 (the OCP saturating conversion used for MX elements).

    Written as a plain nearest search over the 127 finite magnitudes; the
    magnitudes increase with the code, so "even code" is "even mantissa".
    NaN inputs give 0x7F; the sign bit of the input is kept.
    """
    v = np.asarray(v, dtype=np.float64)
    mags = _e4m3_magnitudes()
    a = np.minimum(np.abs(v), E4M3_MAX)
    hi = np.searchsorted(mags, a, side="left")  # first magnitude >= a
    hi = np.minimum(hi, 126)
    lo = np.maximum(hi - 1, 0)
    d_lo = a - mags[lo]
    d_hi = mags[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo)
    code = np.where(mags[hi] == a, hi, code)
    # the sign bit is kept, also when the magnitude rounds to zero (-0 = 0x80)
    out = (code | np.where(np.signbit(v), 0x80, 0)).astype(np.uint8)
    return np.where(np.isnan(v), np.uint8(0x7F), out)


def e8m0_decode(b):
    """E8M0 scale bytes -> 2**(b - 127) (byte 255 is NaN)."""
    b = np.asarray(b, dtype=np.int64)
    return np.where(b == 255, np.nan, np.ldexp(1.0, b - 127))


# ---------------------------------------------------------------------------
# MXFP8 activation quantization
# ---------------------------------------------------------------------------

MX_BLOCK = 32


def mx_quantize(x_bits):
    """bf16 activations ``[T, K]`` -> (e4m3fn codes ``[T, K]``, E8M0 bytes
    ``[T, K/32]``), one shared scale per 32 consecutive K elements of a token.

    The pages say the WKV chain quantizes its bf16 input to MXFP8 before the
    scaled GEMM ("vllm.models.deepseek_v41.nvidia.specialized_decode.engram.
    prefetch", module docstring; "vllm.models.deepseek_v41.amd.mono.attention.
    gemv", module docstring: the tokens' MXFP8 rows) but not the rule. The
    rule taken is the OCP Microscaling Formats (MX) v1.0 conversion:

    * shared exponent X = floor(log2(max |x| over the block)) - emax_elem,
      emax_elem = 8 for E4M3;
    * scale byte = X + 127, clamped to the E8M0 range [0, 254];
    * element code = e4m3fn(x / 2**(byte-127)), nearest-even, saturating;
    * an all-zero block gets byte 0 and zero codes;
    * a block holding an infinity or a NaN has no finite maximum, so no
      shared exponent: it gets the E8M0 NaN byte 255 and every code is the
      e4m3fn NaN 0x7F. A NaN scale makes every element of its block NaN in
      the MX format, so the block decodes to NaN whatever a reader does with
      the codes (reading taken; neither the pages nor the conversion rule
      give a finite encoding for such a block).

    floor(log2 a) is read from the binary exponent of a (exact, no log call).
    """
    x = bf16_to_f64(x_bits)
    T, K = x.shape
    assert K % MX_BLOCK == 0
    blocks = x.reshape(T, K // MX_BLOCK, MX_BLOCK)
    finite = np.isfinite(blocks).all(axis=2)
    amax = np.abs(np.where(np.isfinite(blocks), blocks, 0.0)).max(axis=2)
    _, e = np.frexp(amax)  # amax = f * 2**e, 0.5 <= f < 1 -> floor(log2) = e-1
    shared = (e - 1) - E4M3_EMAX
    scale_byte = np.clip(shared + 127, 0, 254)
    scale_byte = np.where(amax == 0, 0, scale_byte)
    scale_byte = np.where(finite, scale_byte, 255).astype(np.uint8)
    scaled = np.where(finite[:, :, None], blocks, 0.0) / e8m0_decode(scale_byte)[:, :, None]
    codes = e4m3fn_encode(scaled)  # a NaN scale gives NaN quotients -> 0x7F
    codes = np.where(finite[:, :, None], codes, np.uint8(0x7F)).reshape(T, K)
    return codes, scale_byte


def mx_dequantize_activations(codes, scale_bytes):
    """(codes ``[T, K]``, bytes ``[T, K/32]``) -> float64 ``[T, K]``."""
    T, K = codes.shape
    vals = e4m3fn_decode(codes).reshape(T, K // MX_BLOCK, MX_BLOCK)
    return (vals * e8m0_decode(scale_bytes)[:, :, None]).reshape(T, K)


def mx_dequantize_weight(w_codes, w_scales):
    """MXFP8 weight -> float64 ``[N, K]``.

    Layout from "vllm.models.deepseek_v41.amd.mono.attention.gemv" (module
    docstring): row-major e4m3 ``W[N, K]`` and E8M0 bytes ``S[N/32, K/32]``,
    one per 32x32 block; element (n, k) is scaled by 2**(S[n//32, k//32]-127).
    The multiplier reading follows the scale's name on "vllm.models.
    deepseek_v4_1.common.engram" (``weight_scale_inv``: the dequant factor).
    """
    N, K = w_codes.shape
    assert w_scales.shape == (N // 32, K // 32)
    s = e8m0_decode(w_scales)
    s_full = np.repeat(np.repeat(s, 32, axis=0), 32, axis=1)
    return e4m3fn_decode(w_codes) * s_full


# ---------------------------------------------------------------------------
# Step 1: row gather
# ---------------------------------------------------------------------------


def gather_rows(table_bits, hash_ids):
    """``rows[t, c, :] = table[hash_ids[t, c], :]`` as bf16 bit copies.

    "vllm.models.deepseek_v4_1.common.engram": ``Engram.prepare_embeddings``
    looks the layer's ids up into the staged rows; ``ParallelEngramEmbedding.
    lookup`` maps ``[T, heads]`` ids to ``[T, heads, head_dim]`` bf16 rows. The
    ids are global rows of the layer's table (the per-column prime ranges back
    to back; ``EngramLayout.offsets``).

    Out-of-range ids are not defined by the pages; the reading taken is a zero
    row plus an error flag (returned as the second value).
    """
    table_bits = np.asarray(table_bits, dtype=np.uint16)
    ids = np.asarray(hash_ids, dtype=np.int64)
    num_rows = table_bits.shape[0]
    bad = (ids < 0) | (ids >= num_rows)
    safe = np.where(bad, 0, ids)
    rows = table_bits[safe]
    rows[bad] = 0
    return rows, bool(bad.any())


def dequant_table_rows(codes, scale_bytes):
    """fp8 table rows ``[..., hd]`` e4m3fn + ``[..., hd/32]`` ue8m0 bytes ->
    bf16 bit patterns ``[..., hd]``.

    "vllm.models.deepseek_v4_1.common.engram", ``ParallelEngramEmbedding``
    (class docstring and ``__init__``): the table is ``[rows, dim]``
    float8_e4m3fn plus one uint8 ue8m0 scale per row and 32 consecutive
    elements (``weight_scale_inv``, ``[rows, dim // block_size]``,
    block_size 32), and rows are dequantized to bf16 on lookup. The pages do
    not print the arithmetic; the reading taken is the plain one: element
    value times 2**(byte - 127) (E8M0: byte 255 is NaN), rounded to bf16
    (nearest even; beyond the bf16 range -> inf, below half its smallest
    subnormal -> 0). In the ordinary range the product is exact in bf16
    (e4m3 keeps 3 fraction bits, bf16 7), so the rounding only acts at the
    extremes.
    """
    c = np.asarray(codes, dtype=np.uint8)
    s = np.asarray(scale_bytes, dtype=np.uint8)
    if c.shape[-1] != s.shape[-1] * MX_BLOCK:
        raise ValueError("one scale byte per 32 elements")
    scale = np.repeat(e8m0_decode(s), MX_BLOCK, axis=-1)
    return round_to_bf16(e4m3fn_decode(c) * scale)


def gather_rows_fp8(table_codes, table_scales, hash_ids):
    """``rows[t, c, :] = dequant(table[hash_ids[t, c], :])`` as bf16 bits,
    the lookup of an fp8 table ("vllm.models.deepseek_v4_1.common.engram",
    ``ParallelEngramEmbedding``: rows stay fp8 and are dequantized with their
    per-32 scales on lookup). Out-of-range ids: zero row + error flag, as in
    ``gather_rows``."""
    codes = np.asarray(table_codes, dtype=np.uint8)
    scales = np.asarray(table_scales, dtype=np.uint8)
    ids = np.asarray(hash_ids, dtype=np.int64)
    num_rows = codes.shape[0]
    bad = (ids < 0) | (ids >= num_rows)
    safe = np.where(bad, 0, ids)
    rows = dequant_table_rows(codes[safe], scales[safe])
    rows[bad] = 0
    return rows, bool(bad.any())


# ---------------------------------------------------------------------------
# Step 2: wkv projection
# ---------------------------------------------------------------------------


def wkv(x_bits, w, w_scales=None):
    """``kv = bf16(x . W^T)``, returned as (bf16 bits ``[T, N]``, fp64 exact).

    "vllm.models.deepseek_v4_1.common.engram", ``Engram.__init__`` /
    ``forward``: ``wkv`` is a bias-free linear from ``n_hash_cols*head_dim``
    to ``dim*(hc_mult+1)`` applied to the flattened staged rows; its output
    row is ``[key_0 | ... | key_{hc-1} | value]``, each ``dim`` wide (the same
    column split the ROCm page uses for its merged column-parallel linear).

    ``w`` is bf16 bits ``[N, K]`` when ``w_scales`` is None, else e4m3fn codes
    with ``w_scales`` E8M0 bytes ``[N/32, K/32]``; then ``x`` is first
    quantized to MXFP8 (``mx_quantize``) and both operands enter the product
    at their dequantized values.
    """
    if w_scales is None:
        xa = bf16_to_f64(x_bits)
        wa = bf16_to_f64(w)
    else:
        codes, sbytes = mx_quantize(x_bits)
        xa = mx_dequantize_activations(codes, sbytes)
        wa = mx_dequantize_weight(w, w_scales)
    kv64 = xa @ wa.T
    return round_to_bf16(kv64), kv64


# ---------------------------------------------------------------------------
# Step 3: gate and residual update
# ---------------------------------------------------------------------------


def _gate_from_sums(hs, ks, dot, dim, eps, clamp):
    """Gate value from the three per-(token, copy) sums over ``dim``.

    "vllm.models.deepseek_v41.amd.engram", ``_engram_gate_finish_kernel``:
    both norms add ``eps`` to the mean square inside the reciprocal root, the
    dot is further scaled by 1/sqrt(dim), the gate input is the square root of
    max(|d|, clamp) carrying d's sign (negative only when d < 0), and the gate
    is its logistic sigmoid.
    """
    hidden_rms = 1.0 / np.sqrt(hs / dim + eps)
    key_rms = 1.0 / np.sqrt(ks / dim + eps)
    d = dot * hidden_rms * key_rms / math.sqrt(dim)
    s = np.sqrt(np.maximum(np.abs(d), clamp))
    s = np.where(d < 0.0, -s, s)
    return 1.0 / (1.0 + np.exp(-s))


def gate(hidden_bits, kv_bits, q_bits, k_bits, token_mask, eps, clamp):
    """Gate + residual: returns (out bf16 bits ``[T, hc, dim]``, gate fp64 ``[T, hc]``).

    For each token t and copy h, over the ``dim`` elements:
    hs = sum hid^2, ks = sum key^2, dot = sum hid*q[h]*k[h]*key (the key is
    column block h of kv, the value the last block), then the gate above, and
    ``out = hid + g * value`` rounded to bf16.
    ("vllm.models.deepseek_v41.amd.engram", ``_engram_gate_finish_kernel`` with
    a single shard; ``_engram_gate_partials_kernel`` shows which operands enter
    the two sums; "vllm.models.deepseek_v4_1.common.engram", ``Engram``
    docstring and ``forward``.)

    ``token_mask`` False shuts the gate and the position passes through
    untouched (``Engram.forward`` docstring): those rows are copied from
    ``hidden`` bit for bit and get gate 0. ``token_mask`` None = all active.
    """
    hid = bf16_to_f64(hidden_bits)
    T, hc, dim = hid.shape
    kv = bf16_to_f64(kv_bits).reshape(T, hc + 1, dim)
    key = kv[:, :hc, :]
    value = kv[:, hc, :]
    q = bf16_to_f64(q_bits)
    k = bf16_to_f64(k_bits)
    hs = np.sum(hid * hid, axis=2)
    ks = np.sum(key * key, axis=2)
    dot = np.sum(hid * q[None] * k[None] * key, axis=2)
    g = _gate_from_sums(hs, ks, dot, dim, eps, clamp)
    out = round_to_bf16(hid + g[:, :, None] * value[:, None, :])
    if token_mask is not None:
        active = np.asarray(token_mask, dtype=bool)
        g = np.where(active[:, None], g, 0.0)
        out = np.where(active[:, None, None], out, np.asarray(hidden_bits, np.uint16))
    return out, g


def gate_partials(hidden_bits, kv_slice_bits, q_bits, k_bits, dim_start):
    """One shard's per-(token, copy) partial sums, the second route to the gate.

    "vllm.models.deepseek_v41.amd.engram", ``_engram_gate_partials_kernel``:
    a shard holds columns [dim_start, dim_start+width) of every key and of the
    value (``kv_slice`` is ``[T, (hc+1)*width]``) and emits, per copy,
    (sum key^2, sum hid*q*k*key) over its slice, plus its value slice.
    Returns (ks ``[T, hc]``, dot ``[T, hc]``, value slice bits ``[T, width]``).
    """
    hid = bf16_to_f64(hidden_bits)
    T, hc, dim = hid.shape
    kvs = np.asarray(kv_slice_bits, dtype=np.uint16)
    width = kvs.shape[1] // (hc + 1)
    sl = slice(dim_start, dim_start + width)
    key = bf16_to_f64(kvs).reshape(T, hc + 1, width)[:, :hc, :]
    q = bf16_to_f64(q_bits)[:, sl]
    k = bf16_to_f64(k_bits)[:, sl]
    ks = np.sum(key * key, axis=2)
    dot = np.sum(hid[:, :, sl] * q[None] * k[None] * key, axis=2)
    value = kvs.reshape(T, hc + 1, width)[:, hc, :]
    return ks, dot, value


def gate_finish(hidden_bits, parts, token_mask, eps, clamp):
    """Finish step of the shard route: add the shards' partial sums in shard
    order, gather the value from the shards' slices (shard-major), and apply
    the same gate and update as ``gate`` ("vllm.models.deepseek_v41.amd.
    engram", ``_engram_gate_finish_kernel``)."""
    hid = bf16_to_f64(hidden_bits)
    T, hc, dim = hid.shape
    ks = np.zeros((T, hc))
    dot = np.zeros((T, hc))
    for p_ks, p_dot, _ in parts:
        ks = ks + p_ks
        dot = dot + p_dot
    value = bf16_to_f64(np.concatenate([v for _, _, v in parts], axis=1))
    hs = np.sum(hid * hid, axis=2)
    g = _gate_from_sums(hs, ks, dot, dim, eps, clamp)
    if token_mask is not None:
        g = np.where(np.asarray(token_mask, bool)[:, None], g, 0.0)
    out = round_to_bf16(hid + g[:, :, None] * value[:, None, :])
    return out, g


# ---------------------------------------------------------------------------
# The layer
# ---------------------------------------------------------------------------


def forward(table_bits, hash_ids, w, w_scales, hidden_bits, q_bits, k_bits,
            token_mask, eps, clamp, block_tokens=2048, table_scales=None):
    """One Engram layer forward: gather -> (MXFP8 quantize) -> wkv -> gate.

    "vllm.models.deepseek_v4_1.common.engram", ``Engram.forward``:
    ``kv = wkv(embed(hash_ids).flatten(-2))``, then the fused gate / residual
    over ``[T, hc, dim]``. Every output row depends only on its own token's
    ids, hidden row and mask bit, so the work is done in token blocks (exact).
    With ``table_scales`` the table is fp8 (``table_bits`` holds e4m3fn codes)
    and the gather dequantizes (``gather_rows_fp8``).
    Returns dict(rows, kv, gate, out, err).
    """
    hidden_bits = np.asarray(hidden_bits, dtype=np.uint16)
    T, hc, dim = hidden_bits.shape
    ids = np.asarray(hash_ids)
    C = ids.shape[1]
    hd = table_bits.shape[1]
    N = (hc + 1) * dim
    rows = np.empty((T, C, hd), np.uint16)
    kv = np.empty((T, N), np.uint16)
    g = np.empty((T, hc))
    out = np.empty_like(hidden_bits)
    err = False
    wa = None
    if w_scales is not None:
        wa = mx_dequantize_weight(w, w_scales)
    for t0 in range(0, T, block_tokens):
        t1 = min(T, t0 + block_tokens)
        if table_scales is None:
            r, e = gather_rows(table_bits, ids[t0:t1])
        else:
            r, e = gather_rows_fp8(table_bits, table_scales, ids[t0:t1])
        err |= e
        rows[t0:t1] = r
        x = r.reshape(t1 - t0, C * hd)
        if w_scales is None:
            kvb, _ = wkv(x, w)
        else:
            codes, sb = mx_quantize(x)
            kv64 = mx_dequantize_activations(codes, sb) @ wa.T
            kvb = round_to_bf16(kv64)
        kv[t0:t1] = kvb
        m = None if token_mask is None else np.asarray(token_mask)[t0:t1]
        o, gg = gate(hidden_bits[t0:t1], kvb, q_bits, k_bits, m, eps, clamp)
        out[t0:t1] = o
        g[t0:t1] = gg
    return {"rows": rows, "kv": kv, "gate": g, "out": out, "err": err}


# ---------------------------------------------------------------------------
# Table layout
# ---------------------------------------------------------------------------


def _is_prime(n):
    if n < 2:
        return False
    if n % 2 == 0:
        return n == 2
    f = 3
    while f * f <= n:
        if n % f == 0:
            return False
        f += 2
    return True


def layout_primes(vocab_size, max_ngram_size, n_heads, n_layers=1):
    """Per-column table row counts of each layer, in (n-gram order, head) order.

    "vllm.models.deepseek_v4_1.common.engram", ``EngramLayout``: for every
    layer and every n-gram order 2..max, the search restarts just below the
    vocab size and takes, for each head, the next prime not already used by
    any earlier (layer, order, head); ``offsets`` is the exclusive running sum
    of a layer's sizes. Returns (sizes per layer, offsets per layer).
    """
    seen = set()
    layers = []
    for _ in range(n_layers):
        sizes = []
        for _ in range(max_ngram_size - 1):
            current = vocab_size - 1
            for _ in range(n_heads):
                current += 1
                while not _is_prime(current) or current in seen:
                    current += 1
                seen.add(current)
                sizes.append(current)
        layers.append(sizes)
    offsets = [[sum(s[:i]) for i in range(len(s))] for s in layers]
    return layers, offsets
