"""Pins of the CPU oracle to facts outside itself.

Each test checks the oracle against something the pages, the mathematics or a
published format definition fixes: library conversions, brute-force searches
on tiny inputs, closed forms, a second route to the same number, and
invariants. No GPU needed.
"""

import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import engram_oracle as o

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
EPS = 1e-6
CLAMP = 1e-6


def _bf16_bits(a):
    """float array -> bf16 bits via torch's cast (a library routine)."""
    t = torch.as_tensor(np.asarray(a, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def _sigmoid(x):
    return 1.0 / (1.0 + math.exp(-x))


# ---------------------------------------------------------------- bf16 ----


def test_bf16_widen_known_patterns():
    bits = np.array([0x3F80, 0xC000, 0x7F7F, 0x0001, 0x8000, 0x3FC0], np.uint16)
    want = [1.0, -2.0, float.fromhex("0x1.fep127"), 2.0 ** -133, -0.0, 1.5]
    got = o.bf16_to_f64(bits)
    assert list(got) == want
    assert math.copysign(1.0, got[4]) == -1.0


def test_bf16_round_matches_library_cast_on_fp32_inputs():
    rng = np.random.default_rng(1)
    x = rng.standard_normal(200000) * np.exp(rng.standard_normal(200000) * 8)
    x32 = x.astype(np.float32)
    # add exact ties: bf16 value + half a quantum
    base = o.bf16_to_f64(_bf16_bits(x32[:5000]))
    _, e = np.frexp(np.abs(base))
    ties = base + np.copysign(np.ldexp(1.0, e - 9), base)
    x32 = np.concatenate([x32, ties.astype(np.float32)])
    assert np.array_equal(o.round_to_bf16(x32.astype(np.float64)), _bf16_bits(x32))


def test_bf16_round_is_nearest_even_by_brute_force():
    rng = np.random.default_rng(2)
    x = rng.standard_normal(3000) * np.exp(rng.standard_normal(3000) * 4)
    got = o.round_to_bf16(x)
    for xi, b in zip(x, got):
        cands = np.array([b - 1, b, b + 1], dtype=np.int64) & 0xFFFF
        vals = o.bf16_to_f64(cands.astype(np.uint16))
        dist = np.abs(vals - xi)
        assert dist[1] <= dist[0] and dist[1] <= dist[2]
        if dist[1] == dist[0] or dist[1] == dist[2]:
            assert b % 2 == 0


def test_bf16_round_ties_to_even_worked():
    # around 1.0 the bf16 spacing is 2**-7
    x = np.array([1 + 2.0 ** -8, 1 + 3 * 2.0 ** -8, -(1 + 2.0 ** -8), 0.0, -0.0])
    assert list(o.round_to_bf16(x)) == [0x3F80, 0x3F82, 0xBF80, 0x0000, 0x8000]


# ---------------------------------------------------------------- e4m3 ----


def test_e4m3_decode_matches_spec_values():
    spec = json.load(open(os.path.join(GOLDEN, "e4m3fn_spec_values.json")))
    for code, val in spec["codes"].items():
        got = o.e4m3fn_decode(np.array([int(code, 16)], np.uint8))[0]
        assert got == val and math.copysign(1, got) == math.copysign(1, val), code
    for code in spec["nan_codes"]:
        assert np.isnan(o.e4m3fn_decode(np.array([int(code, 16)], np.uint8))[0])


def test_e4m3_decode_matches_library_all_codes():
    c = np.arange(256, dtype=np.uint8)
    lib = torch.from_numpy(c).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    ours = o.e4m3fn_decode(c)
    assert np.array_equal(np.isnan(ours), np.isnan(lib))
    fin = ~np.isnan(ours)
    assert np.array_equal(ours[fin], lib[fin])


def test_e4m3_encode_matches_library_in_range():
    rng = np.random.default_rng(3)
    v = np.concatenate([
        rng.standard_normal(100000) * 30,
        rng.uniform(-448, 448, 50000),
        rng.standard_normal(20000) * 2.0 ** -7,
    ])
    # exact midpoints between neighbouring magnitudes exercise the tie rule
    mags = o.e4m3fn_decode(np.arange(127, dtype=np.uint8))
    mids = (mags[1:] + mags[:-1]) / 2
    v = np.concatenate([v, mids, -mids])
    lib = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(o.e4m3fn_encode(v), lib)


def test_e4m3_encode_saturates_and_keeps_sign():
    v = np.array([448.0, 449.0, 464.0, 500.0, 1e9, -1e9, -0.0, -1e-30, np.nan])
    got = o.e4m3fn_encode(v)
    assert list(got[:6]) == [0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0xFE]
    assert got[6] == 0x80 and got[7] == 0x80 and got[8] == 0x7F


def test_e4m3_encode_decode_roundtrip_all_finite_codes():
    c = np.array([x for x in range(256) if (x & 0x7F) != 0x7F], np.uint8)
    assert np.array_equal(o.e4m3fn_encode(o.e4m3fn_decode(c)), c)


# -------------------------------------------------------------- MX rule ----


def test_mx_quantize_worked_blocks():
    K = 32 * 5
    x = np.zeros((1, K))
    x[0, 0] = 1.0
    x[0, 1] = 0.5  # amax 1 -> X = 0 - 8 -> byte 119; 1*2**8 = 256 -> 0x78
    x[0, 32:64] = 0.0  # all zero -> byte 0, zero codes
    x[0, 64] = 448.0 * 4  # amax = 448 * 2**2 -> X = 8+2-8 = 2 -> byte 129, code 0x7E
    x[0, 65] = -3.0  # -3 / 4 = -0.75 -> 0.75 = 1.5 * 2**-1 -> exp 6 mant 4 -> 0xB4
    x[0, 96] = 2.0 ** -20  # amax 2**-20 -> X = -28 -> byte 99; code 0x78
    x[0, 128] = 1.0
    x[0, 129] = 1.0 + 2.0 ** -7  # 256 + 2 -> between 256 and 288: nearest 256
    codes, sb = o.mx_quantize(o.round_to_bf16(x))
    assert list(sb[0]) == [119, 0, 129, 99, 119]
    assert codes[0, 0] == 0x78 and codes[0, 1] == 0x70 and codes[0, 2] == 0
    assert not codes[0, 32:64].any()
    assert codes[0, 64] == 0x7E and codes[0, 65] == 0xB4
    assert codes[0, 96] == 0x78
    assert codes[0, 128] == 0x78 and codes[0, 129] == 0x78


def test_mx_quantize_error_bound_and_idempotence():
    rng = np.random.default_rng(4)
    T, K = 16, 256
    x = o.round_to_bf16(rng.standard_normal((T, K)) * np.exp(rng.standard_normal((T, 1)) * 3))
    codes, sb = o.mx_quantize(x)
    xa = o.bf16_to_f64(x)
    deq = o.mx_dequantize_activations(codes, sb)
    # MX element error: at most half a quantum, the quantum being 2**-3 of the
    # element's own binade, or 2**(X-9) (e4m3's subnormal step times the block
    # scale 2**X) when that is larger
    X = sb.astype(np.int64) - 127
    Xf = np.repeat(X, 32, axis=1)
    _, e = np.frexp(np.abs(xa))
    q = np.maximum(np.ldexp(1.0, e - 1 - 3), np.ldexp(1.0, Xf - 9))
    sat = np.abs(xa) > np.ldexp(448.0, Xf)
    assert np.all(np.abs(deq - xa)[~sat] <= q[~sat] / 2)
    # elements above 448 * 2**X (only possible in a block's top binade) saturate
    assert np.array_equal(deq[sat], np.copysign(np.ldexp(448.0, Xf[sat]), xa[sat]))
    # the block maximum itself never saturates below 256 * 2**X
    amax = np.abs(xa).reshape(T, K // 32, 32).max(2)
    assert np.all(amax >= np.ldexp(256.0, X)) and np.all(amax < np.ldexp(512.0, X))
    # quantizing the dequantized values again gives the same codes and scales
    codes2, sb2 = o.mx_quantize(o.round_to_bf16(deq))
    assert np.array_equal(codes2, codes) and np.array_equal(sb2, sb)


def test_mx_quantize_non_finite_blocks_become_nan_blocks():
    """A block holding +inf, -inf or a NaN (any payload, either sign) is the
    E8M0 NaN scale 255 with every code 0x7F, the e4m3fn NaN; blocks of the
    same token without one are quantized as if it were not there (here the
    worked values of the rule: amax 1 -> byte 119, code 0x78), and the
    dequantized non-finite block is NaN throughout."""
    K = 32 * 4
    bits = np.zeros((3, K), np.uint16)
    bits[0, 5] = 0x7F80            # +inf
    bits[0, 6] = 0x3F80            # 1.0 beside it: still a NaN block
    bits[1, 40] = 0xFF80           # -inf in block 1
    bits[2, 127] = 0xFFC1          # a negative NaN with a payload, in block 3
    bits[2, 126] = 0x7FC0
    for t in range(3):
        fin = [b for b in range(4) if not ((t, b) in [(0, 0), (1, 1), (2, 3)])]
        for b in fin:
            bits[t, 32 * b] = 0x3F80                  # 1.0
            bits[t, 32 * b + 1] = 0xBF00              # -0.5
    codes, sb = o.mx_quantize(bits)
    nan_blocks = [(0, 0), (1, 1), (2, 3)]
    for t in range(3):
        for b in range(4):
            blk = codes[t, 32 * b:32 * b + 32]
            if (t, b) in nan_blocks:
                assert sb[t, b] == 255
                assert np.all(blk == 0x7F)
            else:
                assert sb[t, b] == 119
                assert blk[0] == 0x78 and blk[1] == 0xF0 and not blk[2:].any()
    deq = o.mx_dequantize_activations(codes, sb)
    assert np.all(np.isnan(deq[0, 0:32])) and np.all(np.isnan(deq[2, 96:128]))
    assert deq[0, 32] == 1.0 and deq[0, 33] == -0.5


# --------------------------------------------------------------- gather ----


def test_gather_equals_direct_indexing_and_flags_bad_ids():
    rng = np.random.default_rng(5)
    table = rng.integers(0, 65536, size=(97, 8), dtype=np.uint16)
    ids = rng.integers(0, 97, size=(11, 3))
    rows, err = o.gather_rows(table, ids)
    assert not err
    for t in range(11):
        for c in range(3):
            assert np.array_equal(rows[t, c], table[ids[t, c]])
    ids[2, 1] = 97
    ids[5, 0] = -1
    rows, err = o.gather_rows(table, ids)
    assert err and not rows[2, 1].any() and not rows[5, 0].any()
    assert np.array_equal(rows[2, 0], table[ids[2, 0]])


# ------------------------------------------------------------ fp8 tables ----


def test_fp8_table_dequant_worked_values():
    """Hand-worked e4m3 x 2^(b-127) -> bf16 cases, incl. the range edges
    (tests/golden/fp8_table_dequant.json states the source and each step)."""
    cases = json.load(open(os.path.join(GOLDEN, "fp8_table_dequant.json")))["cases"]
    for c in cases:
        codes = np.full((1, 32), int(c["code"], 16), np.uint8)
        sb = np.array([[c["byte"]]], np.uint8)
        got = o.dequant_table_rows(codes, sb)
        assert np.all(got == int(c["bf16"], 16)), (c, hex(int(got[0, 0])))


def test_fp8_table_dequant_matches_library_fp8_cast():
    """Every e4m3 code under scale bytes 100..167, a different byte for each
    32-element block of a row (so a wrong block-to-scale mapping shows):
    torch's float8_e4m3fn decode, times the power of two in float32 (exact
    there), cast to bfloat16 by torch."""
    codes = np.tile(np.arange(256, dtype=np.uint8), (61, 1))           # [61, 256]: 8 blocks a row
    sb = (np.arange(100, 161)[:, None] + np.arange(8)[None, :]).astype(np.uint8)   # [61, 8]
    got = o.dequant_table_rows(codes, sb)
    per_elem = np.repeat(sb.astype(np.int64), 32, axis=1)              # element j uses block j // 32
    f = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float32)
    f = f * torch.from_numpy(np.ldexp(1.0, per_elem - 127).astype(np.float32))
    want = f.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    nan = np.isnan(f.numpy())
    assert np.array_equal(got[~nan], want[~nan])
    assert np.all(got[nan] == 0x7FC0)


def test_gather_rows_fp8_commutes_with_dequant_and_flags_bad_ids():
    rng = np.random.default_rng(15)
    codes = rng.integers(0, 256, size=(61, 64), dtype=np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0x11                                # no NaN codes
    scales = rng.integers(110, 135, size=(61, 2), dtype=np.uint8)
    ids = rng.integers(0, 61, size=(9, 3))
    ids[4, 2] = 61
    ids[7, 0] = -3
    rows, err = o.gather_rows_fp8(codes, scales, ids)
    assert err
    full = o.dequant_table_rows(codes, scales)
    for t in range(9):
        for c in range(3):
            if 0 <= ids[t, c] < 61:
                assert np.array_equal(rows[t, c], full[ids[t, c]])
            else:
                assert not rows[t, c].any()


def test_forward_fp8_table_equals_forward_on_dequantized_table():
    rng = np.random.default_rng(16)
    T, hc, dim, C, hd, R = 19, 2, 64, 4, 32, 173
    codes = torch.from_numpy(rng.standard_normal((R, hd))).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    scales = rng.integers(119, 124, size=(R, hd // 32)).astype(np.uint8)
    ids = rng.integers(0, R, size=(T, C))
    w = o.round_to_bf16(rng.standard_normal(((hc + 1) * dim, C * hd)) * 0.02)
    hidden, _, q, k = _rand_gate_inputs(rng, T, hc, dim)
    mask = rng.random(T) > 0.2
    a = o.forward(codes, ids, w, None, hidden, q, k, mask, EPS, CLAMP, table_scales=scales)
    b = o.forward(o.dequant_table_rows(codes, scales), ids, w, None, hidden, q, k, mask, EPS, CLAMP)
    for key in ("rows", "kv", "out", "gate"):
        assert np.array_equal(a[key], b[key]), key


# ------------------------------------------------------------------ wkv ----


def test_wkv_bf16_matches_brute_force_loops():
    rng = np.random.default_rng(6)
    T, K, N = 3, 48, 40
    x = o.round_to_bf16(rng.standard_normal((T, K)))
    w = o.round_to_bf16(rng.standard_normal((N, K)) * 0.1)
    kv_bits, kv64 = o.wkv(x, w)
    for t in range(T):
        for n in range(N):
            acc = 0.0
            for k in range(K):
                acc += float(o.bf16_to_f64(x[t, k])) * float(o.bf16_to_f64(w[n, k]))
            assert abs(acc - kv64[t, n]) <= 1e-12 * max(1.0, abs(acc))
    assert np.array_equal(kv_bits, o.round_to_bf16(kv64))


def test_wkv_mxfp8_one_hot_probes_pick_the_right_block_scale():
    # distinct E8M0 byte per 32x32 block; one-hot weight code 1.0 at (n0, k0)
    # and a one-hot activation at k0 read back exactly 2**(S[n0/32, k0/32]-127)
    N, K = 96, 128
    S = (100 + np.arange(N // 32)[:, None] * 4 + np.arange(K // 32)[None, :]).astype(np.uint8)
    for n0, k0 in [(0, 0), (31, 31), (32, 0), (5, 40), (70, 127), (95, 64)]:
        w = np.zeros((N, K), np.uint8)
        w[n0, k0] = 0x38  # 1.0
        x = np.zeros((1, K))
        x[0, k0] = 1.0
        _, kv64 = o.wkv(o.round_to_bf16(x), w, S)
        want = np.zeros(N)
        want[n0] = 2.0 ** (int(S[n0 // 32, k0 // 32]) - 127)
        assert np.array_equal(kv64[0], want), (n0, k0)


def test_wkv_mxfp8_matches_brute_force_loops():
    rng = np.random.default_rng(7)
    T, K, N = 2, 64, 64
    x = o.round_to_bf16(rng.standard_normal((T, K)))
    w = torch.from_numpy(rng.standard_normal((N, K))).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    S = rng.integers(119, 128, size=(N // 32, K // 32)).astype(np.uint8)
    _, kv64 = o.wkv(x, w, S)
    codes, sb = o.mx_quantize(x)
    lib_dec = lambda c: float(torch.tensor([int(c)], dtype=torch.uint8).view(torch.float8_e4m3fn).double())
    for t in range(T):
        for n in range(N):
            acc = 0.0
            for k in range(K):
                xv = lib_dec(codes[t, k]) * 2.0 ** (int(sb[t, k // 32]) - 127)
                wv = lib_dec(w[n, k]) * 2.0 ** (int(S[n // 32, k // 32]) - 127)
                acc += xv * wv
            assert abs(acc - kv64[t, n]) <= 1e-12 * max(1.0, abs(acc))


# ----------------------------------------------------------------- gate ----


def _pattern(name, dim):
    if name == "ones":
        return np.ones(dim)
    if name == "minus_ones":
        return -np.ones(dim)
    if name == "alternating":
        return np.where(np.arange(dim) % 2 == 0, 1.0, -1.0)
    if name == "zeros":
        return np.zeros(dim)
    if name == "ones_times_1e-3":
        return np.full(dim, 1e-3)
    raise KeyError(name)


@pytest.mark.parametrize("case", json.load(open(os.path.join(GOLDEN, "gate_closed_forms.json")))["cases"],
                         ids=lambda c: f"{c['name']}-{c['dim']}")
def test_gate_closed_forms(case):
    dim = case["dim"]
    hid = _pattern(case["hidden"], dim)
    key = _pattern(case["key"], dim)
    value = np.full(dim, 0.5)
    hidden_bits = o.round_to_bf16(hid)[None, None, :]
    if case["hidden"] == "ones_times_1e-3":
        # bf16(1e-3) is not 1e-3: feed exact fp64 values through the sums
        hs, ks, dot = dim * 1e-6, float(dim), dim * 1e-3
        g = o._gate_from_sums(np.array([hs]), np.array([ks]), np.array([dot]), dim, EPS, CLAMP)[0]
        assert abs(g - case["expected"]) < 1e-9
        return
    kv_bits = o.round_to_bf16(np.concatenate([key, value]))[None, :]
    ones = o.round_to_bf16(np.ones((1, dim)))
    out, g = o.gate(hidden_bits, kv_bits, ones, ones, None, EPS, CLAMP)
    assert abs(g[0, 0] - case["expected"]) < 1e-9
    want = o.round_to_bf16(hid + case["expected"] * 0.5)
    assert np.array_equal(out[0, 0], want)


def _rand_gate_inputs(rng, T, hc, dim, scale_h=1.0):
    hidden = o.round_to_bf16(rng.standard_normal((T, hc, dim)) * scale_h)
    kv = o.round_to_bf16(rng.standard_normal((T, (hc + 1) * dim)) * 0.02)
    q = o.round_to_bf16(1 + 0.1 * rng.standard_normal((hc, dim)))
    k = o.round_to_bf16(1 + 0.1 * rng.standard_normal((hc, dim)))
    return hidden, kv, q, k


def test_gate_key_blocks_and_value_block_are_the_right_columns():
    # copy h's key is +-(its own hidden row); the value block is constant
    rng = np.random.default_rng(8)
    T, hc, dim = 2, 3, 64
    hid = rng.standard_normal((T, hc, dim))
    hidden = o.round_to_bf16(hid)
    hf = o.bf16_to_f64(hidden)
    signs = np.array([1.0, -1.0, 1.0])
    kv = np.concatenate([signs[h] * hf[:, h, :] for h in range(hc)] + [np.full((T, dim), 0.25)], axis=1)
    ones = o.round_to_bf16(np.ones((hc, dim)))
    out, g = o.gate(hidden, o.round_to_bf16(kv), ones, ones, None, EPS, CLAMP)
    # key = +-hidden: d = +-sqrt(dim)/(1+eps/ms)... |d| close to sqrt(dim)
    for t in range(T):
        for h in range(hc):
            ms = np.mean(hf[t, h] ** 2)
            d = signs[h] * math.sqrt(dim) * ms / (ms + EPS)
            want = _sigmoid(math.copysign(math.sqrt(abs(d)), d))
            assert abs(g[t, h] - want) < 1e-12
            assert np.array_equal(out[t, h], o.round_to_bf16(hf[t, h] + want * 0.25))


def test_gate_q_and_k_enter_only_the_dot():
    # scaling q by c scales only the dot; with the norms unchanged d scales by c
    rng = np.random.default_rng(9)
    hidden, kv, q, k = _rand_gate_inputs(rng, 4, 2, 128)
    ones = o.round_to_bf16(np.ones((2, 128)))
    two = o.round_to_bf16(2 * np.ones((2, 128)))
    _, g1 = o.gate(hidden, kv, ones, ones, None, EPS, CLAMP)
    _, g4 = o.gate(hidden, kv, two, two, None, EPS, CLAMP)
    s1 = np.log(g1 / (1 - g1))
    s4 = np.log(g4 / (1 - g4))
    big = np.abs(s1) > 0.05
    assert np.allclose(s4[big], 2 * s1[big], rtol=1e-9)


def test_gate_two_routes_agree():
    # the shard route (partials + finish) with 2, 4, 8 shards equals one shard
    rng = np.random.default_rng(10)
    T, hc, dim = 5, 4, 256
    hidden, kv, q, k = _rand_gate_inputs(rng, T, hc, dim)
    mask = np.array([True, False, True, True, False])
    out1, g1 = o.gate(hidden, kv, q, k, mask, EPS, CLAMP)
    kv3 = kv.reshape(T, hc + 1, dim)
    for shards in (1, 2, 4, 8):
        width = dim // shards
        parts = []
        for r in range(shards):
            sl = kv3[:, :, r * width:(r + 1) * width].reshape(T, (hc + 1) * width)
            parts.append(o.gate_partials(hidden, sl, q, k, r * width))
        out2, g2 = o.gate_finish(hidden, parts, mask, EPS, CLAMP)
        assert np.max(np.abs(g2 - g1)) < 1e-12
        act = mask
        assert np.array_equal(out2[act], out1[act])


def test_gate_invariants():
    rng = np.random.default_rng(11)
    T, hc, dim = 64, 2, 256
    hidden, kv, q, k = _rand_gate_inputs(rng, T, hc, dim)
    mask = rng.random(T) > 0.2
    out, g = o.gate(hidden, kv, q, k, mask, EPS, CLAMP)
    act = g[mask]
    assert np.all((act > 0) & (act < 1))
    assert np.all(np.abs(act - 0.5) >= _sigmoid(1e-3) - 0.5 - 1e-15)
    assert np.all(g[~mask] == 0)
    assert np.array_equal(out[~mask], hidden[~mask])
    # mask None == all True
    o1, g1 = o.gate(hidden, kv, q, k, None, EPS, CLAMP)
    o2, g2 = o.gate(hidden, kv, q, k, np.ones(T, bool), EPS, CLAMP)
    assert np.array_equal(o1, o2) and np.array_equal(g1, g2)
    # sign symmetry: negating the hidden stream maps g -> 1 - g
    neg = hidden ^ np.uint16(0x8000)
    _, gn = o.gate(neg, kv, q, k, None, EPS, CLAMP)
    assert np.max(np.abs(gn - (1 - g1))) < 1e-12
    # negating only the keys does the same
    kvn = kv.reshape(T, hc + 1, dim).copy()
    kvn[:, :hc] ^= np.uint16(0x8000)
    _, gk = o.gate(hidden, kvn.reshape(T, -1), q, k, None, EPS, CLAMP)
    assert np.max(np.abs(gk - (1 - g1))) < 1e-12
    # zero value -> out == hidden (by value)
    kvz = kv.reshape(T, hc + 1, dim).copy()
    kvz[:, hc] = 0
    oz, _ = o.gate(hidden, kvz.reshape(T, -1), q, k, None, EPS, CLAMP)
    assert np.array_equal(o.bf16_to_f64(oz), o.bf16_to_f64(hidden))
    # scale invariance of the gate in the hidden stream (mean square >> eps)
    h8 = o.round_to_bf16(8 * o.bf16_to_f64(hidden))
    _, g8 = o.gate(h8, kv, q, k, None, EPS, CLAMP)
    assert np.max(np.abs(g8 - g1)) < 1e-5


# -------------------------------------------------------------- forward ----


def test_forward_composes_the_steps_and_blocks_exactly():
    rng = np.random.default_rng(12)
    T, hc, dim, C, hd = 37, 2, 64, 4, 32
    R = 301
    table = o.round_to_bf16(rng.standard_normal((R, hd)) * 0.02)
    ids = rng.integers(0, R, size=(T, C))
    w = o.round_to_bf16(rng.standard_normal(((hc + 1) * dim, C * hd)) * 0.02)
    hidden, _, q, k = _rand_gate_inputs(rng, T, hc, dim)
    mask = rng.random(T) > 0.1
    res = o.forward(table, ids, w, None, hidden, q, k, mask, EPS, CLAMP, block_tokens=8)
    rows, _ = o.gather_rows(table, ids)
    kv, _ = o.wkv(rows.reshape(T, C * hd), w)
    out, g = o.gate(hidden, kv, q, k, mask, EPS, CLAMP)
    assert np.array_equal(res["rows"], rows) and np.array_equal(res["kv"], kv)
    assert np.array_equal(res["out"], out) and np.array_equal(res["gate"], g)
    assert np.array_equal(res["out"][~mask], hidden[~mask])
    # MXFP8 weights
    wq = torch.from_numpy(rng.standard_normal(((hc + 1) * dim, C * hd))).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    S = rng.integers(119, 128, size=((hc + 1) * dim // 32, C * hd // 32)).astype(np.uint8)
    res = o.forward(table, ids, wq, S, hidden, q, k, None, EPS, CLAMP, block_tokens=16)
    kvq, _ = o.wkv(rows.reshape(T, C * hd), wq, S)
    assert np.array_equal(res["kv"], kvq)
    # empty input
    res = o.forward(table, ids[:0], w, None, hidden[:0], q, k, None, EPS, CLAMP)
    assert res["out"].shape == (0, hc, dim)


# --------------------------------------------------------------- layout ----


def test_layout_primes_are_the_next_unused_primes():
    for vocab, ngram, heads in [(10000, 3, 4), (262144, 3, 8), (2097152, 3, 8), (4194304, 4, 8)]:
        sizes, offsets = o.layout_primes(vocab, ngram, heads)
        s = sizes[0]
        C = (ngram - 1) * heads
        assert len(s) == C and len(set(s)) == C
        # one layer: every order restarts at vocab-1 but skips used primes, so
        # the sizes are exactly the first C primes >= vocab, in order
        n, want = vocab, []
        while len(want) < C:
            if all(n % f for f in range(2, int(n ** 0.5) + 1)):
                want.append(n)
            n += 1
        assert s == want
        assert offsets[0] == [int(v) for v in np.cumsum([0] + s[:-1])]
    sizes, _ = o.layout_primes(10000, 3, 4, n_layers=2)
    assert sizes[1][0] == 10091 and not set(sizes[0]) & set(sizes[1])
