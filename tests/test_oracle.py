"""Pins for the CPU oracle (no GPU): format definition, brute force, invariants,
closed forms and exact special cases. Each test names what it pins.

The oracle is test infrastructure; these tests are what let the GPU parity
tests trust it.
"""
from __future__ import annotations

import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import brute
import oracle
import workloads as wl

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _golden_lines(name):
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                yield line.split()


def _bf16(values) -> np.ndarray:
    return wl.f32_to_bf16_bits(np.asarray(values, dtype=np.float32))


# ---------------------------------------------------------------- E4M3 codec

def test_decode_matches_hand_table():
    """Pin: hand-worked code values from the E4M3 definition (golden file)."""
    table = oracle.e4m3_decode_table()
    for code_hex, val in _golden_lines("e4m3_decode_hand.txt"):
        code = int(code_hex, 16)
        if val == "nan":
            assert math.isnan(table[code])
        elif val == "-0":
            assert table[code] == 0.0 and math.copysign(1.0, table[code]) < 0
        else:
            assert table[code] == float(Fraction(val)), (code_hex, table[code], val)


def test_decode_matches_torch_float8_e4m3fn():
    """Pin: all 256 codes agree with torch's float8_e4m3fn (a library routine, OCP E4M3FN)."""
    table = oracle.e4m3_decode_table()
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    both_nan = np.isnan(table) & np.isnan(ref)
    assert np.array_equal(np.isnan(table), np.isnan(ref))
    assert np.array_equal(table[~both_nan], ref[~both_nan])
    assert np.array_equal(np.signbit(table[~both_nan]), np.signbit(ref[~both_nan]))


def test_decode_matches_brute_definition():
    """Pin: the oracle's decoder equals the independent Fraction definition on every finite code."""
    table = oracle.e4m3_decode_table()
    for code in range(256):
        if code & 0x7F == 0x7F:
            continue
        assert table[code] == float(brute.e4m3_value(code))


def test_round_trip_all_finite_codes():
    """Pin: encode(decode(c)) == c for all 254 finite codes (incl. 0x80), both encoders."""
    table = oracle.e4m3_decode_table()
    for code in range(256):
        if code & 0x7F == 0x7F:
            continue
        v = float(table[code])
        if code == 0x80:
            v = -0.0
        assert oracle.e4m3_encode(v, "bits") == code
        assert oracle.e4m3_encode(v, "search") == code


def test_encode_hand_ties():
    """Pin: hand-worked ties, carries, saturation and signed zeros (golden file)."""
    for row in _golden_lines("e4m3_encode_hand.txt"):
        v, code = float.fromhex(row[0]), int(row[1], 16)
        assert oracle.e4m3_encode(v, "bits") == code, row
        assert oracle.e4m3_encode(v, "search") == code, row


def test_encoders_agree_exhaustive_band():
    """Pin: the bit-arithmetic and table-search encoders agree on every binary32
    pattern with 2^-12 <= |v| <= 2^10 (everything that can round to a nonzero
    code below saturation), and on a strided sample of the rest."""
    lo, hi = 0x39800000, 0x44800000          # 2^-12 .. 2^10
    bad, first = oracle.encoders_disagree(lo, hi, 1)
    assert bad == 0, hex(first)
    bad, first = oracle.encoders_disagree(0, lo, 997)       # zero, subnormals, tiny
    assert bad == 0, hex(first)
    bad, first = oracle.encoders_disagree(hi, 0x7F7FFFFF, 991)  # up to FLT_MAX
    assert bad == 0, hex(first)


def test_encode_matches_torch_cast_below_saturation():
    """Pin: agreement with torch's float32 -> float8_e4m3fn cast (a library
    routine) for |v| < 464, where torch is defined; ties and random values."""
    rng = np.random.default_rng(1)
    vals = [rng.standard_normal(20000).astype(np.float32) * np.float32(s)
            for s in (1e-3, 1e-2, 0.1, 1, 10, 100)]
    table = oracle.e4m3_decode_table()
    finite = table[:0x7F]
    mids = ((finite[:-1] + finite[1:]) / 2).astype(np.float32)  # every midpoint (exact in fp32)
    vals.append(mids)
    vals.append(-mids)
    v = np.concatenate(vals)
    v = v[np.abs(v) < 464]
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    ours = np.array([oracle.e4m3_encode(float(x), "bits") for x in v], dtype=np.uint8)
    assert np.array_equal(ours, ref)


# -------------------------------------------------------------- quantizers

def test_hand_worked_tile():
    """Pin: a 1x128 tile worked by hand (golden file): s = 2^-3, q = E4M3(8x)."""
    x = np.zeros((1, 128), dtype=np.uint16)
    expect = np.zeros(128, dtype=np.uint8)
    scale = None
    with open(os.path.join(GOLDEN, "quant_tile_hand.txt")) as f:
        for line in f:
            if line.startswith("# scale"):
                scale = float(line.split()[2])
    for idx, b, code, *_ in _golden_lines("quant_tile_hand.txt"):
        x[0, int(idx)] = int(b, 16)
        expect[int(idx)] = int(code, 16)
    q, s = oracle.quant_act_1x128(x)
    assert s[0, 0] == np.float32(scale)
    assert np.array_equal(q[0], expect)


def _edge_tiles(rng) -> np.ndarray:
    """A few 128-wide rows of bf16 bits hitting the special cases."""
    rows = []
    rows.append(_bf16(rng.standard_normal(128)))                          # plain
    z = np.zeros(128, dtype=np.uint16); z[::3] = 0x8000; rows.append(z)  # all +-0
    r = _bf16(rng.standard_normal(128) * 1e-3); r[17] = _bf16([1000.0])[0]; rows.append(r)  # outlier
    sub = rng.integers(1, 0x80, 128).astype(np.uint16)                    # bf16 subnormals
    sub[::2] |= 0x8000; rows.append(sub)
    big = _bf16(rng.standard_normal(128)); big[5] = 0x7F7F; rows.append(big)  # amax = bf16 max
    tiny = _bf16(rng.standard_normal(128) * 1e-38); rows.append(tiny)       # subnormal fp32 scale
    one = np.zeros(128, dtype=np.uint16); one[77] = _bf16([-3.0])[0]; rows.append(one)  # single value
    ties = _bf16(np.full(128, 448.0 * 17 / 64)); ties[0] = _bf16([448.0])[0]; rows.append(ties)
    return np.stack(rows)


def test_quantizer_matches_exact_rational_brute_force():
    """Pin: 1x128 quantization equals the exact-rational brute force (hand
    binary32 rounding + linear nearest-code scan) on random and edge tiles."""
    rng = np.random.default_rng(2)
    x = _edge_tiles(rng)
    extra = wl.activation(0, "tiny_fprop", 7, 4, 128, 100.0)
    x = np.concatenate([x, extra])
    q, s = oracle.quant_act_1x128(x)
    for r in range(x.shape[0]):
        s_ref, codes = brute.quantize_group([int(b) for b in x[r]])
        assert Fraction(float(s[0, r])) == s_ref, r
        assert list(q[r]) == codes, r


def test_max_code_is_448_in_every_normal_tile():
    """Invariant: every tile with a normal scale has max |q| decoding to 448
    (the amax element maps to ~448); all-zero tiles have s = 0."""
    d = wl.dense_fprop(0, m=64, n=128, k=1024)
    q, s = oracle.quant_act_1x128(d["x"])
    table = oracle.e4m3_decode_table()
    mag = np.abs(table[q]).reshape(64, -1, 128).max(axis=2)  # [rows][slabs]
    assert np.all(mag == 448.0)
    assert np.all(s > np.float32(2.0 ** -126))


def test_power_of_two_scaling_invariance():
    """Invariant: quant(2^p X) gives the same codes and scales times 2^p."""
    x = wl.activation(0, "tiny_fprop", 3, 16, 256, 100.0)
    q0, s0 = oracle.quant_act_1x128(x)
    xf = wl.bf16_bits_to_f32(x)
    for p in (-20, -3, 5, 30):
        xp = wl.f32_to_bf16_bits(xf * np.float32(2.0 ** p))  # exact scaling
        q1, s1 = oracle.quant_act_1x128(xp)
        assert np.array_equal(q0, q1)
        assert np.array_equal(s1, s0 * np.float32(2.0 ** p))


def test_negation_flips_sign_bits_only():
    """Invariant: quant(-X) = quant(X) with the sign bit flipped, same scales."""
    x = wl.activation(0, "tiny_fprop", 4, 16, 256, 100.0)
    q0, s0 = oracle.quant_act_1x128(x)
    q1, s1 = oracle.quant_act_1x128(x ^ np.uint16(0x8000))
    assert np.array_equal(q1, q0 ^ np.uint8(0x80))
    assert np.array_equal(s0, s1)


def test_row_permutation_commutes():
    """Invariant: 1x128 quantization commutes with a row permutation (quantize
    before dispatch: page "Eliminate Deepseek Ai News For Good", passage on
    quantizing activations before the MoE up-projection dispatch)."""
    x = wl.activation(0, "tiny_fprop", 5, 64, 384, 100.0)
    perm = np.random.default_rng(3).permutation(64)
    q0, s0 = oracle.quant_act_1x128(x)
    q1, s1 = oracle.quant_act_1x128(x[perm])
    assert np.array_equal(q1, q0[perm])
    assert np.array_equal(s1, s0[:, perm])


def test_weight_blocks_commute_with_transpose():
    """Invariant: 128x128 block quantization of W^T is the transpose of that of W."""
    w = wl.weight(0, "tiny_fprop", 6, 256, 384)
    q0, s0 = oracle.quant_weight_128x128(w)
    q1, s1 = oracle.quant_weight_128x128(np.ascontiguousarray(w.T))
    assert np.array_equal(q1, q0.T)
    assert np.array_equal(s1, s0.T)


def test_weight_block_matches_brute_force():
    """Pin: one 128x128 block equals the brute-force group quantization of its 16384 values."""
    w = wl.weight(0, "tiny_fprop", 8, 128, 128)
    w[3, 4] = _bf16([-0.5])[0]
    q, s = oracle.quant_weight_128x128(w)
    s_ref, codes = brute.quantize_group([int(b) for b in w.reshape(-1)])
    assert Fraction(float(s[0, 0])) == s_ref
    assert list(q.reshape(-1)) == codes


def test_128x1_is_1x128_of_transpose():
    """Invariant: 128x1 token tiles on X equal 1x128 tiles on X^T (output is X^T-shaped)."""
    x = wl.activation(0, "wgrad", 9, 256, 200, 50.0)
    qt, s = oracle.quant_act_128x1(x)
    q_ref, s_ref = oracle.quant_act_1x128(np.ascontiguousarray(x.T))
    assert np.array_equal(qt, q_ref)
    assert np.array_equal(s, s_ref)


def test_scale_closed_form_power_of_two_amax():
    """Closed form: amax = 448 * 2^p gives s = 2^p exactly and q = E4M3(x * 2^-p)."""
    rng = np.random.default_rng(4)
    for p in (-10, 0, 3):
        v = rng.standard_normal(128).astype(np.float32)
        v[0] = 448.0
        v = np.clip(v, -448, 448) * np.float32(2.0 ** p)
        x = _bf16(v)[None, :]
        q, s = oracle.quant_act_1x128(x)
        assert s[0, 0] == np.float32(2.0 ** p)
        expect = [oracle.e4m3_encode(float(f) * 2.0 ** -p) for f in wl.bf16_bits_to_f32(x[0])]
        assert list(q[0]) == expect


def test_quant_pairs_matches_tile_quantizer():
    """The (x, amax) pair form equals the tile quantizer when amax is the tile's amax."""
    x = wl.activation(0, "tiny_fprop", 10, 8, 128, 100.0)
    q, _ = oracle.quant_act_1x128(x)
    amax_bits = (x & np.uint16(0x7FFF)).max(axis=1, keepdims=True)
    qp = oracle.quant_pairs(x, np.broadcast_to(amax_bits, x.shape).copy())
    assert np.array_equal(q, qp)


# -------------------------------------------------------------------- GEMM

def _expand_block(s, rows, k):
    return np.repeat(np.repeat(s, 128, 0), 128, 1)[:rows, :k]


def test_gemm_matches_exact_rational_brute_force():
    """Pin: tiny GEMM (M,N <= 6, K = 384) equals the exact rational sum."""
    x = wl.activation(0, "tiny_fprop", 11, 5, 384, 100.0)
    w = wl.weight(0, "tiny_fprop", 12, 128, 384)
    qa, sa = oracle.quant_act_1x128(x)
    qb, sb = oracle.quant_weight_128x128(w)
    c = oracle.gemm(qa, sa, qb, sb, "block")
    a_sc = np.repeat(sa.T, 128, axis=1)
    b_sc = _expand_block(sb, 128, 384)
    exact = brute.gemm_exact(qa.tolist(), a_sc.tolist(), qb[:6].tolist(), b_sc[:6].tolist())
    for m in range(5):
        for n in range(6):
            e = exact[m][n]
            assert abs(Fraction(c[m, n]) - e) <= abs(e) * Fraction(1, 2 ** 45) + Fraction(1, 2 ** 200)


def test_gemm_row_kind_matches_brute_force():
    """Pin: the Wgrad form (per-row scales on both operands) against the exact sum."""
    dy = wl.activation(0, "wgrad", 13, 256, 4, None)
    x = wl.activation(0, "wgrad", 14, 256, 5, 50.0)
    qa, sa = oracle.quant_act_128x1(dy)   # [4][256], [2][4]
    qb, sb = oracle.quant_act_128x1(x)    # [5][256], [2][5]
    c = oracle.gemm(qa, sa, qb, sb, "row")
    a_sc = np.repeat(sa.T, 128, axis=1)
    b_sc = np.repeat(sb.T, 128, axis=1)
    exact = brute.gemm_exact(qa.tolist(), a_sc.tolist(), qb.tolist(), b_sc.tolist())
    for m in range(4):
        for n in range(5):
            e = exact[m][n]
            assert abs(Fraction(c[m, n]) - e) <= abs(e) * Fraction(1, 2 ** 45) + Fraction(1, 2 ** 200)


def test_gemm_k128_is_scaled_integer_gemm():
    """Special case: with K = 128 the result is sA[m] * sB * (textbook GEMM of the
    decoded values), and the decoded values times 2^9 are integers."""
    x = wl.activation(0, "tiny_fprop", 15, 32, 128, 100.0)
    w = wl.weight(0, "tiny_fprop", 16, 128, 128)
    qa, sa = oracle.quant_act_1x128(x)
    qb, sb = oracle.quant_weight_128x128(w)
    table = oracle.e4m3_decode_table()
    ia = (table[qa] * 512).astype(np.int64)
    ib = (table[qb] * 512).astype(np.int64)
    assert np.array_equal(ia / 512.0, table[qa])
    scale = sa[0].astype(np.float64)[:, None] * float(sb[0, 0]) / 2.0 ** 18
    ref = (ia @ ib.T).astype(np.float64) * scale          # one rounding
    mag = (np.abs(ia) @ np.abs(ib).T).astype(np.float64) * scale
    c = oracle.gemm(qa, sa, qb, sb, "block")
    # float64 dot-product error bound: K * 2^-53 * sum |terms| (+ ref's own rounding)
    bound = 128 * 2.0 ** -53 * mag + 2.0 ** -52 * np.abs(ref)
    assert np.all(np.abs(c - ref) <= bound)


def test_gemm_exact_power_of_two_case():
    """Exact case: integer-valued codes (|q| <= 16) and power-of-two scales make
    every partial sum an integer times a power of two, so the float64 result
    must equal the integer GEMM bit for bit."""
    rng = np.random.default_rng(5)
    M, N, K = 24, 256, 512
    ints = [0, 1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11, 12, 13, 14, 15, 16]
    int_codes = {int(v): oracle.e4m3_encode(float(v)) for v in ints}
    va = rng.integers(-16, 17, (M, K))
    vb = rng.integers(-16, 17, (N, K))
    enc = lambda v: np.vectorize(lambda t: int_codes[abs(int(t))] | (0x80 if t < 0 else 0))(v).astype(np.uint8)
    qa, qb = enc(va), enc(vb)
    sa = (2.0 ** rng.integers(-4, 5, (K // 128, M))).astype(np.float32)
    sb = (2.0 ** rng.integers(-4, 5, (N // 128, K // 128))).astype(np.float32)
    c = oracle.gemm(qa, sa, qb, sb, "block")
    ref = np.zeros((M, N))
    for j in range(K // 128):
        part = va[:, 128 * j:128 * j + 128] @ vb[:, 128 * j:128 * j + 128].T
        ref += part * (sa[j].astype(np.float64)[:, None] * np.repeat(sb[:, j], 128)[None, :N])
    assert np.array_equal(c, ref)


def test_gemm_linearity_and_zero():
    """Invariants: zero operand -> zero output; doubling A's scales doubles C; negating B's codes negates C."""
    x = wl.activation(0, "tiny_fprop", 17, 16, 256, 100.0)
    w = wl.weight(0, "tiny_fprop", 18, 128, 256)
    qa, sa = oracle.quant_act_1x128(x)
    qb, sb = oracle.quant_weight_128x128(w)
    c = oracle.gemm(qa, sa, qb, sb)
    assert np.array_equal(oracle.gemm(np.zeros_like(qa), sa, qb, sb), np.zeros_like(c))
    assert np.array_equal(oracle.gemm(qa, sa * np.float32(2), qb, sb), 2 * c)
    assert np.array_equal(oracle.gemm(qa, sa, qb ^ np.uint8(0x80), sb), -c)


def test_grouped_is_per_expert_gemm_with_zero_padding():
    """Invariant: grouped GEMM equals per-expert GEMM on each segment; padding rows are 0."""
    rows = np.array([0, 1, 127, 128, 129, 5])
    g = wl.grouped_fprop(0, n=256, k=256, experts=len(rows), rows=rows)
    qa, sa = oracle.quant_act_1x128(g["x"])
    qb = np.empty(g["w"].shape, dtype=np.uint8)
    sb = np.empty((len(rows), 2, 2), dtype=np.float32)
    for e in range(len(rows)):
        qb[e], sb[e] = oracle.quant_weight_128x128(g["w"][e])
    c = oracle.grouped_gemm(g["offsets"], rows, qa, sa, qb, sb)
    off = g["offsets"]
    for e in range(len(rows)):
        r0, r = off[e], rows[e]
        if r:
            ref = oracle.gemm(qa[r0:r0 + r], np.ascontiguousarray(sa[:, r0:r0 + r]), qb[e], sb[e])
            assert np.array_equal(c[r0:r0 + r], ref)
        assert np.all(c[r0 + r:off[e + 1]] == 0)


def test_grouped_brute_force_tiny():
    """oracle.grouped_gemm against exact rationals on a tiny grouped problem.
    The segment of each expert is found here from the real row counts alone
    (each expert's rows rounded up to a multiple of 128, in expert order), and
    every real output row is the exact sum over K of the dequantized codes of
    its own A row and its own expert's weight; padding rows are zero."""
    rows = [0, 1, 2, 1]
    n, k = 256, 256
    rng = np.random.default_rng(77)
    seg = [128 * ((r + 127) // 128) for r in rows]
    m_total = sum(seg)
    offsets = np.concatenate([[0], np.cumsum(seg)]).astype(np.int64)
    finite = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], np.uint8)
    qa = rng.choice(finite, size=(m_total, k)).astype(np.uint8)
    sa = rng.uniform(0.01, 3.0, (k // 128, m_total)).astype(np.float32)
    E = len(rows)
    qb = rng.choice(finite, size=(E, n, k)).astype(np.uint8)
    sb = rng.uniform(0.01, 3.0, (E, n // 128, k // 128)).astype(np.float32)
    c = oracle.grouped_gemm(offsets, np.array(rows), qa, sa, qb, sb)
    start = 0
    for e, r in enumerate(rows):
        real = list(range(start, start + r))
        if real:
            a_codes = [[int(v) for v in qa[i]] for i in real]
            a_sc = [[float(sa[kk // 128][i]) for kk in range(k)] for i in real]
            b_codes = [[int(v) for v in qb[e][j]] for j in range(n)]
            b_sc = [[float(sb[e][j // 128][kk // 128]) for kk in range(k)] for j in range(n)]
            exact = brute.gemm_exact(a_codes, a_sc, b_codes, b_sc)
            # float64 dot products of K terms are within K * 2^-53 * sum |terms|
            # of the exact value (the dequantized operands themselves are exact)
            abs_sum = brute.gemm_exact(a_codes, a_sc, b_codes, b_sc, absolute=True)
            got = c[start:start + r]
            for ii in range(r):
                for j in range(n):
                    ref = exact[ii][j]
                    bound = k * 2.0 ** -53 * float(abs_sum[ii][j])
                    assert abs(Fraction(float(got[ii, j])) - ref) <= bound, (e, ii, j, got[ii, j], float(ref))
        pad_end = start + 128 * ((r + 127) // 128)
        assert np.all(c[start + r:pad_end] == 0), "expert %d padding rows" % e
        start = pad_end
    assert start == m_total


def test_grouped_experts_take_their_own_weight():
    """Invariant: if expert e's weight is 2^e times expert 0's (exact in bf16,
    and quantizing 2^e W gives W's codes with scales times 2^e), every real
    row of expert e equals 2^e times the dense GEMM of that row with W; with
    equal weights, the grouped output on the real rows is the dense GEMM of
    the gathered rows. A segment read from the wrong offset, or an expert
    paired with the wrong weight, breaks one of the two."""
    rows = np.array([3, 0, 130, 1, 64])
    n, k = 128, 384
    g = wl.grouped_fprop(2, n=n, k=k, experts=len(rows), rows=rows)
    qa, sa = oracle.quant_act_1x128(g["x"])
    w0 = g["w"][0]
    E = len(rows)
    qb = np.empty((E, n, k), np.uint8)
    sb = np.empty((E, n // 128, k // 128), np.float32)
    for e in range(E):
        we = wl.f32_to_bf16_bits(wl.bf16_bits_to_f32(w0) * np.float32(2.0 ** e))
        qb[e], sb[e] = oracle.quant_weight_128x128(we)
    q0, s0 = oracle.quant_weight_128x128(w0)
    for e in range(E):
        assert np.array_equal(qb[e], q0)
        assert np.array_equal(sb[e], s0 * np.float32(2.0 ** e))
    off = g["offsets"]
    c = oracle.grouped_gemm(off, rows, qa, sa, qb, sb)
    real = np.concatenate([np.arange(off[e], off[e] + rows[e]) for e in range(E)]).astype(np.int64)
    expert_of = np.concatenate([np.full(rows[e], e) for e in range(E)])
    ga, gs = np.ascontiguousarray(qa[real]), np.ascontiguousarray(sa[:, real])
    dense = oracle.gemm(ga, gs, q0, s0)
    # the float64 sums may round differently in a different row batch: allow
    # K * 2^-53 of the sum of the terms' magnitudes
    tol = k * 2.0 ** -53 * (np.abs(oracle.dequant_rows_1x128(ga, gs)) @
                            np.abs(oracle.dequant_block_128x128(q0, s0)).T)
    scale = (2.0 ** expert_of)[:, None]
    assert np.all(np.abs(c[real] - dense * scale) <= tol * scale)
    same = oracle.grouped_gemm(off, rows, qa, sa, np.repeat(q0[None], E, 0), np.repeat(s0[None], E, 0))
    assert np.all(np.abs(same[real] - dense) <= tol)
    # and the pairing is visible: expert e's rows are not those of any other scaling
    for e in range(E):
        sel = expert_of == e
        if sel.any() and e > 0:
            assert np.max(np.abs(c[real][sel] - dense[sel])) > 1e-3
    pad = np.setdiff1d(np.arange(qa.shape[0]), real)
    assert np.all(c[pad] == 0) and np.all(same[pad] == 0)


def test_bf16_round_diagnostic():
    """The bf16 rounding helper (diagnostic only) matches torch's float32 -> bf16 cast."""
    v = np.random.default_rng(6).standard_normal(10000) * 10
    ref = torch.from_numpy(v.astype(np.float32)).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(oracle.bf16_round(v), ref)


# ------------------------------------------------- tile placement (closed form)

def _planted(rng, shape, tile_r, tile_c):
    """Values in [-1, 1] with each (tile_r x tile_c) tile's amax planted at 448 * 2^p,
    p distinct per tile; returns (bf16 bits, p per tile)."""
    R, C = shape
    tr, tc = R // tile_r, C // tile_c
    p = rng.permutation(tr * tc).reshape(tr, tc) - 20
    v = rng.uniform(-1, 1, shape).astype(np.float32) * np.float32(448.0 * 0.99)
    for i in range(tr):
        for j in range(tc):
            blk = v[i * tile_r:(i + 1) * tile_r, j * tile_c:(j + 1) * tile_c]
            blk[rng.integers(tile_r), rng.integers(tile_c)] = 448.0
            blk *= np.float32(2.0 ** p[i, j])
    return wl.f32_to_bf16_bits(v), p


def test_1x128_scale_placement_closed_form():
    """Closed form: tile (row r, slab j) with amax 448 * 2^p has s[j][r] = 2^p and
    codes E4M3(x * 2^-p) -- pins the slab-major scale layout and tile indexing."""
    rng = np.random.default_rng(7)
    x, p = _planted(rng, (6, 512), 1, 128)
    q, s = oracle.quant_act_1x128(x)
    assert np.array_equal(s, (2.0 ** p.T).astype(np.float32))
    xf = wl.bf16_bits_to_f32(x).astype(np.float64)
    for r in range(6):
        for j in range(4):
            expect = [oracle.e4m3_encode(float(v) * 2.0 ** -p[r, j]) for v in xf[r, 128 * j:128 * j + 128]]
            assert list(q[r, 128 * j:128 * j + 128]) == expect


def test_128x1_scale_placement_closed_form():
    """Closed form for 128x1 token tiles: s[j][c] = 2^p(j, c); output is token-contiguous."""
    rng = np.random.default_rng(8)
    x, p = _planted(rng, (384, 5), 128, 1)
    qt, s = oracle.quant_act_128x1(x)
    assert np.array_equal(s, (2.0 ** p).astype(np.float32))
    xf = wl.bf16_bits_to_f32(x).astype(np.float64)
    for c in range(5):
        for j in range(3):
            expect = [oracle.e4m3_encode(float(v) * 2.0 ** -p[j, c]) for v in xf[128 * j:128 * j + 128, c]]
            assert list(qt[c, 128 * j:128 * j + 128]) == expect


def test_128x128_scale_placement_closed_form():
    """Closed form for 128x128 blocks: s[bn][bk] = 2^p(bn, bk)."""
    rng = np.random.default_rng(9)
    w, p = _planted(rng, (256, 384), 128, 128)
    q, s = oracle.quant_weight_128x128(w)
    assert np.array_equal(s, (2.0 ** p).astype(np.float32))
    xf = wl.bf16_bits_to_f32(w).astype(np.float64)
    for bn in range(2):
        for bk in range(3):
            blk = xf[128 * bn:128 * bn + 128, 128 * bk:128 * bk + 128].reshape(-1)[::37]
            got = q[128 * bn:128 * bn + 128, 128 * bk:128 * bk + 128].reshape(-1)[::37]
            assert list(got) == [oracle.e4m3_encode(float(v) * 2.0 ** -p[bn, bk]) for v in blk]


def test_scatter_identity_route_is_the_tile_quantizer():
    """Special case: one route per token to its own row is plain 1x128 quantization."""
    x = wl.activation(0, "grouped_fprop", 50, 37, 256, 50.0)
    dst = np.arange(37, dtype=np.int32)[:, None]
    q, s, written = oracle.quant_act_scatter(x, dst, 37)
    q_ref, s_ref = oracle.quant_act_1x128(x)
    assert written.all()
    assert np.array_equal(q, q_ref) and np.array_equal(s.view(np.uint32), s_ref.view(np.uint32))


def test_scatter_rows_are_quantized_source_rows():
    """Invariant (quantization commutes with row moves): each destination row
    equals the 1x128 quantization of the bf16 row of its source token; a token
    routed twice gives two identical rows; -1 and out-of-range routes write
    nothing. Checked against quantizing the gathered bf16 rows directly."""
    x = wl.activation(0, "grouped_fprop", 51, 6, 384, 50.0)
    dst = np.array([[4, -1], [0, 7], [-1, -1], [2, 99], [5, 1], [-1, 3]], dtype=np.int32)
    m_total = 9
    q, s, written = oracle.quant_act_scatter(x, dst, m_total)
    src = {4: 0, 0: 1, 7: 1, 2: 3, 5: 4, 1: 4, 3: 5}
    assert sorted(np.nonzero(written)[0].tolist()) == sorted(src)
    rows = sorted(src)
    q_g, s_g = oracle.quant_act_1x128(np.stack([x[src[r]] for r in rows]))
    assert np.array_equal(q[rows], q_g)
    assert np.array_equal(s[:, rows].view(np.uint32), s_g.view(np.uint32))
    assert np.array_equal(q[0], q[7]) and not q[6].any() and not q[8].any()


def test_moe_dispatch_map_is_a_valid_layout():
    """The seeded routing fills every real row of every expert segment exactly
    once, in token order, with at most top_k routes per token."""
    d = wl.moe_dispatch(0, k=128)
    dst, rows, off = d["dst_rows"], d["rows"], d["offsets"]
    v = dst[dst >= 0]
    assert len(v) == rows.sum() and len(np.unique(v)) == len(v)
    real = np.concatenate([np.arange(off[e], off[e] + rows[e]) for e in range(len(rows))])
    assert np.array_equal(np.sort(v), real)
    assert (dst >= 0).sum(axis=1).max() <= dst.shape[1]
    t_idx, k_idx = np.nonzero(dst >= 0)
    d = dst[t_idx, k_idx]
    order = np.argsort(d)
    tok_by_row, row_sorted = t_idx[order], d[order]
    seg = np.searchsorted(off, row_sorted, side="right") - 1
    same = seg[1:] == seg[:-1]
    assert np.all(np.diff(tok_by_row)[same] > 0)      # token order inside each segment


def _packed_tokens(rows, cols, tensor_id, grad=False):
    """Expert-sorted bf16 rows (128-padded segments, zero padding rows)."""
    rows = np.asarray(rows, dtype=np.int64)
    off = wl.pad_offsets(rows)
    real = (wl.grad_rowscaled(0, "grouped_fprop", tensor_id, int(rows.sum()), cols) if grad
            else wl.activation(0, "grouped_fprop", tensor_id, int(rows.sum()), cols, 50.0))
    out = np.zeros((int(off[-1]), cols), np.uint16)
    src = 0
    for e in range(len(rows)):
        out[off[e]:off[e] + rows[e]] = real[src:src + rows[e]]
        src += int(rows[e])
    return out, off


def test_grouped_wgrad_sums_to_dense_wgrad():
    """Invariant: with zero padding tokens, the expert gradients add up to the
    dense Wgrad over all tokens (the pinned row-scale GEMM): every 128-token
    slab belongs to one expert, so the sum regroups the same slab terms."""
    rows = [5, 0, 130, 128, 1]
    dy, off = _packed_tokens(rows, 256, 90, grad=True)
    x, _ = _packed_tokens(rows, 384, 91)
    a_q, a_s = oracle.quant_act_128x1(dy)
    b_q, b_s = oracle.quant_act_128x1(x)
    per = oracle.grouped_gemm_wgrad(off, a_q, a_s, b_q, b_s)
    dense = oracle.gemm(a_q, a_s, b_q, b_s, "row")
    assert per.shape == (5, 256, 384)
    assert not per[1].any()                                  # empty segment: zero gradient
    np.testing.assert_allclose(per.sum(axis=0), dense, rtol=1e-12, atol=1e-12 * np.abs(dense).max())


def test_grouped_wgrad_single_expert_is_dense_wgrad():
    """Special case: one expert owning every token is the dense Wgrad GEMM."""
    dy, off = _packed_tokens([256], 128, 92, grad=True)
    x, _ = _packed_tokens([256], 256, 93)
    a_q, a_s = oracle.quant_act_128x1(dy)
    b_q, b_s = oracle.quant_act_128x1(x)
    per = oracle.grouped_gemm_wgrad(off, a_q, a_s, b_q, b_s)
    assert np.array_equal(per[0], oracle.gemm(a_q, a_s, b_q, b_s, "row"))


# ------------------------------------------------------------- microscaling

def test_mx_hand_worked_block():
    """A block worked by hand under the OCP-MX reading: amax = 3 gives
    floor(log2 3) - 8 = -7 (E8M0 byte 120, X = 2^-7); 3 -> 384 = 1.5 * 2^8
    (0x7C); 1 -> 128 = 2^7 (0x70); bf16(0.1) = 0.10009765625 -> 12.8125,
    rounded to 13 = 1.625 * 2^3 (0x55); bf16(-0.001) -> -0.12805..., rounded
    to -0.125 = -2^-3 (0xA0); zeros stay +0."""
    bits = np.zeros(32, np.uint16)
    bits[:4] = wl.f32_to_bf16_bits(np.array([3.0, 1.0, 0.1, -0.001], np.float32))
    q, e = oracle.quant_mx_1x32(bits[None, :])
    assert e[0, 0] == 120
    assert list(q[0, :4]) == [0x7C, 0x70, 0x55, 0xA0]
    assert not q[0, 4:].any()


def _mx_special_rows(rng):
    rows = [wl.f32_to_bf16_bits(rng.standard_normal(64).astype(np.float32))]
    z = np.zeros(64, np.uint16)
    z[::5] = 0x8000
    rows.append(z)                                                    # zero blocks, signed zeros
    rows.append(rng.integers(1, 0x80, 64).astype(np.uint16) | np.uint16(0x8000))  # bf16 subnormals
    big = wl.f32_to_bf16_bits(rng.standard_normal(64).astype(np.float32) * 1e37)
    big[3] = 0x7F7F                                                   # bf16 max: e = 127 - 8
    rows.append(big)
    rows.append(wl.f32_to_bf16_bits(rng.standard_normal(64).astype(np.float32) * 1e-37))  # e below -127 -> clamp
    ties = wl.f32_to_bf16_bits(np.full(64, 448.0 * 17 / 64, np.float32))
    rows.append(ties)
    return np.stack(rows)


def test_mx_matches_exact_rational_brute_force():
    """Pin: every 32-element block equals the exact-rational MX quantization."""
    rng = np.random.default_rng(21)
    x = _mx_special_rows(rng)
    q, e = oracle.quant_mx_1x32(x)
    for r in range(x.shape[0]):
        for b in range(x.shape[1] // 32):
            be, bq = brute.quantize_mx_block([int(v) for v in x[r, 32 * b:32 * b + 32]])
            assert e[r, b] == be + 127, (r, b)
            assert list(q[r, 32 * b:32 * b + 32]) == bq, (r, b)


def test_mx_invariants():
    """Invariants: a nonzero block with an unclamped exponent has max |q| in
    [256, 448] (amax / 2^e lies in [256, 512)); scaling X by 2^p keeps the
    codes and adds p to every exponent; negation flips sign bits only."""
    x = wl.activation(0, "tiny_fprop", 91, 64, 256, 50.0)
    q, e = oracle.quant_mx_1x32(x)
    dec = np.abs(oracle.e4m3_decode_table()[q]).reshape(64, 8, 32).max(axis=2)
    assert np.all((dec >= 256) & (dec <= 448))
    xf = wl.bf16_bits_to_f32(x)
    for p in (-5, 3):
        q2, e2 = oracle.quant_mx_1x32(wl.f32_to_bf16_bits(xf * np.float32(2.0 ** p)))
        assert np.array_equal(q2, q) and np.array_equal(e2.astype(int), e.astype(int) + p)
    qn, en = oracle.quant_mx_1x32(x ^ np.uint16(0x8000))
    assert np.array_equal(en, e) and np.array_equal(qn, q ^ np.uint8(0x80))


def test_gemm_mx_matches_exact_rational_brute_force():
    """Pin: tiny MX GEMM (M, N <= 5, K = 96) equals the exact rational sum."""
    rng = np.random.default_rng(22)
    a = wl.f32_to_bf16_bits(rng.standard_normal((4, 96)).astype(np.float32) * 3)
    b = wl.f32_to_bf16_bits(rng.standard_normal((5, 96)).astype(np.float32) * 0.02)
    aq, ae = oracle.quant_mx_1x32(a)
    bq, be = oracle.quant_mx_1x32(b)
    got = oracle.gemm_mx(aq, ae, bq, be)
    exp_a = [[2.0 ** (int(ae[m, k // 32]) - 127) for k in range(96)] for m in range(4)]
    exp_b = [[2.0 ** (int(be[n, k // 32]) - 127) for k in range(96)] for n in range(5)]
    ref = brute.gemm_exact(aq.tolist(), exp_a, bq.tolist(), exp_b)
    for m in range(4):
        for n in range(5):
            assert got[m, n] == float(ref[m][n])


# ------------------------------------------------- FP8 activation cache re-tile

def _cached_activation(rng, tokens, cols):
    """1x128 codes and scales of a bf16 activation with special token rows:
    zero rows (scale 0), a row with only signed zeros, rows of tiny values
    (subnormal fp32 scales), an outlier row and negative-only rows."""
    x = wl.f32_to_bf16_bits(rng.standard_normal((tokens, cols)).astype(np.float32))
    x[3] = 0
    x[4] = 0x8000
    x[5] = wl.f32_to_bf16_bits(rng.standard_normal(cols).astype(np.float32) * 1e-39)
    x[6] = wl.f32_to_bf16_bits(rng.standard_normal(cols).astype(np.float32) * 3e3)
    x[7] = wl.f32_to_bf16_bits(-np.abs(rng.standard_normal(cols)).astype(np.float32))
    if tokens > 128:
        x[128:256, 5] = 0                                  # an all-zero 128x1 group
    return oracle.quant_act_1x128(x)


def test_retile_matches_exact_rational_brute_force():
    """Pin: sampled 128x1 groups of the re-tiled cache equal the exact-rational
    dequantize (rn32(dec(q) * s)) and requantize of brute force."""
    rng = np.random.default_rng(31)
    q, s = _cached_activation(rng, 256, 256)
    qt, st = oracle.retile_128x1(q, s)
    for c in (0, 1, 5, 127, 128, 200, 255):
        for j in range(2):
            toks = range(128 * j, 128 * j + 128)
            codes = [int(q[t, c]) for t in toks]
            scales = [Fraction(float(s[c // 128, t])) for t in toks]
            bs, bq = brute.retile_group(codes, scales)
            assert Fraction(float(st[j, c])) == bs, (c, j)
            assert list(qt[c, 128 * j:128 * j + 128]) == bq, (c, j)


def test_retile_power_of_two_rows_reproduce_the_codes():
    """Closed form: when every token's 1x128 scale is the same 2^p and every
    128x1 group holds the code 448, v = dec(q) * 2^p exactly, the new scale is
    448 * 2^p / 448 = 2^p and each code comes back unchanged (transposed)."""
    rng = np.random.default_rng(32)
    finite = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], np.uint8)
    q = rng.choice(finite, size=(256, 384)).astype(np.uint8)
    q[rng.integers(0, 128, 384), np.arange(384)] = 0x7E         # +448 in every group
    q[128 + rng.integers(0, 128, 384), np.arange(384)] = 0xFE   # -448
    for p in (-20, 0, 7):
        s = np.full((3, 256), 2.0 ** p, np.float32)
        qt, st = oracle.retile_128x1(q, s)
        assert np.array_equal(qt, q.T)
        assert np.all(st == np.float32(2.0 ** p))


def test_retile_error_within_one_half_e4m3_step():
    """Bound: each re-tiled value differs from the cached value v by at most
    half an E4M3 step at the new scale (rounding v / s' to nearest), plus the
    binary32 rounding of the quotient."""
    rng = np.random.default_rng(33)
    q, s = _cached_activation(rng, 256, 512)
    qt, st = oracle.retile_128x1(q, s)
    dec = oracle.e4m3_decode_table()
    v = (dec[q].astype(np.float32) * np.repeat(s.T, 128, axis=1)).astype(np.float64)   # [t][c]
    back = dec[qt].T * np.repeat(st.astype(np.float64), 128, axis=0)
    y = np.abs(v) / np.repeat(np.where(st == 0, 1, st).astype(np.float64), 128, axis=0)
    expo = np.floor(np.log2(np.maximum(y, 2.0 ** -6)))
    step = 2.0 ** (expo - 3)                                  # E4M3 spacing at y (2^-9 below 2^-6)
    bound = (0.5 * step * (1 + 2 ** -20) + y * 2 ** -24) * np.repeat(st.astype(np.float64), 128, axis=0)
    assert np.all(np.abs(back - v) <= bound)


def test_retile_sign_and_zero_groups():
    """Special cases: an all-zero group stores scale 0 and keeps signed zeros;
    negating the cache flips only the sign bits of the re-tiled codes."""
    rng = np.random.default_rng(34)
    q, s = _cached_activation(rng, 256, 256)
    qt, st = oracle.retile_128x1(q, s)
    assert st[1, 5] == 0 and np.all((qt[5, 128:256] & 0x7F) == 0)
    qn, stn = oracle.retile_128x1(q ^ np.uint8(0x80), s)
    assert np.array_equal(stn, st)
    assert np.array_equal(qn, qt ^ np.uint8(0x80))


# ---------------------------------------------- per-tensor GEMM (study arm)

def test_gemm_tensor_matches_exact_rational_brute_force():
    """Pin: tiny per-tensor GEMM equals the exact rational sum times sA * sB."""
    rng = np.random.default_rng(35)
    finite = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], np.uint8)
    a = rng.choice(finite, size=(3, 160)).astype(np.uint8)
    b = rng.choice(finite, size=(4, 160)).astype(np.uint8)
    sa, sb = np.float32(0.375), np.float32(3.1e-3)
    c = oracle.gemm_tensor(a, sa, b, sb)
    ex = brute.gemm_exact([[int(v) for v in r] for r in a], [[Fraction(float(sa))] * 160] * 3,
                          [[int(v) for v in r] for r in b], [[Fraction(float(sb))] * 160] * 4)
    for i in range(3):
        for j in range(4):
            assert c[i, j] == float(ex[i][j])


def test_gemm_tensor_is_exact_at_k4096():
    """Pin: at the study's K = 4096 the oracle sum is exact: it equals the
    integer GEMM of the codes' values times 2^9 (exact in int64), scaled by
    2^-18, bit for bit."""
    rng = np.random.default_rng(36)
    finite = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], np.uint8)
    a = rng.choice(finite, size=(24, 4096)).astype(np.uint8)
    b = rng.choice(finite, size=(20, 4096)).astype(np.uint8)
    ints = np.array([int(brute.e4m3_value(c) * 512) if (c & 0x7F) != 0x7F else 0
                     for c in range(256)], np.int64)
    exact = ints[a] @ ints[b].T                                # int64, no rounding
    c = oracle.gemm_tensor(a, 1.0, b, 1.0)
    assert np.array_equal(c * 2.0 ** 18, exact.astype(np.float64))
    assert np.all(np.abs(exact) < 2 ** 53)


def test_retile_dequantizes_to_binary32_before_requantizing():
    """Pin of the reading that the cached value is first rounded to binary32:
    token 0 holds 448 at scale 1 (so the new scale is exactly 1) and token 1
    holds 1.125 at scale s = the smallest binary32 above 17/18. The exact
    product lies just above the E4M3 tie 1.0625 (-> 1.125, code 0x39), but
    rn32 of it is the tie itself, which goes to the even code 1.0 (0x38)."""
    s1 = np.float32(17 / 18)
    if Fraction(float(s1)) <= Fraction(17, 18):
        s1 = np.nextafter(s1, np.float32(1))
    assert np.float32(1.125) * s1 == np.float32(1.0625)
    assert Fraction(9, 8) * Fraction(float(s1)) > Fraction(17, 16)
    q = np.zeros((128, 128), np.uint8)
    s = np.ones((1, 128), np.float32)
    q[0, 0], q[1, 0], s[0, 1] = 0x7E, 0x39, s1
    qt, st = oracle.retile_128x1(q, s)
    assert st[0, 0] == 1.0 and qt[0, 0] == 0x7E and qt[0, 1] == 0x38
    bs, bq = brute.retile_group([int(v) for v in q[:, 0]], [Fraction(float(v)) for v in s[0]])
    assert bs == 1 and bq[:2] == [0x7E, 0x38]


def test_oracle_refuses_non_finite_inputs():
    """Non-finite inputs are outside the method's contract: every oracle entry
    that reads bf16 values, E4M3 codes or scales refuses them."""
    x = wl.activation(0, "tiny_fprop", 99, 128, 256, 50.0)
    q, s = oracle.quant_act_1x128(x)
    for bad in (0x7F80, 0xFF80, 0x7FC1):                       # +Inf, -Inf, a NaN
        xb = x.copy()
        xb[5, 200] = bad
        for fn in (oracle.quant_act_1x128, oracle.quant_act_128x1, oracle.quant_weight_128x128,
                   oracle.quant_mx_1x32):
            with pytest.raises(oracle.OutOfContract):
                fn(xb)
    qn = q.copy()
    qn[3, 3] = 0xFF                                            # E4M3 NaN
    with pytest.raises(oracle.OutOfContract):
        oracle.retile_128x1(qn, s)
    with pytest.raises(oracle.OutOfContract):
        oracle.gemm(qn, s, q[:128], np.ones((1, 2), np.float32), "block")
    sn = s.copy()
    sn[1, 7] = np.inf
    with pytest.raises(oracle.OutOfContract):
        oracle.retile_128x1(q, sn)
    with pytest.raises(oracle.OutOfContract):
        oracle.gemm_tensor(q, np.float32("nan"), q, 1.0)
