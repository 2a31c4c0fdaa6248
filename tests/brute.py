"""Exact-rational brute force used to pin the oracle on tiny inputs.

Written independently of ``oracle/``: every value is a ``fractions.Fraction``,
binary32 rounding is done by hand (nearest, ties to even, with subnormals), and
E4M3 encoding is a linear scan over all finite codes. Slow by design; only for
a few tiles or a few-by-few GEMM.
"""
from __future__ import annotations

from fractions import Fraction


def bf16_value(bits: int) -> Fraction:
    """Exact value of a finite bf16 bit pattern (sign bit 15, 8 exponent bits, 7 fraction bits)."""
    bits &= 0xFFFF
    sign = -1 if bits >> 15 else 1
    exp = (bits >> 7) & 0xFF
    frac = bits & 0x7F
    if exp == 0xFF:
        raise ValueError("non-finite bf16 is out of contract")
    if exp == 0:
        mag = Fraction(frac, 1 << 7) * Fraction(1, 1 << 126)
    else:
        mag = (1 + Fraction(frac, 1 << 7)) * (Fraction(2) ** (exp - 127))
    return sign * mag


def bf16_is_negative(bits: int) -> bool:
    return bool((bits >> 15) & 1)


def _floor_log2(a: Fraction) -> int:
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    return e


def _round_half_even(v: Fraction) -> int:
    fl = v.numerator // v.denominator
    rem = v - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        return fl + 1
    return fl


def round_binary32(v: Fraction) -> Fraction:
    """Nearest binary32 value (ties to even), subnormals included; no overflow expected."""
    if v == 0:
        return Fraction(0)
    sign = -1 if v < 0 else 1
    a = abs(v)
    e = max(_floor_log2(a), -126)
    ulp = Fraction(2) ** (e - 23)
    n = _round_half_even(a / ulp)
    out = n * ulp
    assert out < Fraction(2) ** 128, "binary32 overflow"
    return sign * out


def e4m3_finite_values() -> list[tuple[int, Fraction]]:
    """(code, value) for the non-negative finite E4M3FN codes 0x00..0x7E."""
    out = []
    for code in range(0x7F):
        e, m = code >> 3, code & 7
        if e == 0:
            val = Fraction(m, 8) * Fraction(1, 64)          # m/8 * 2^-6
        else:
            val = Fraction(8 + m, 8) * Fraction(2) ** (e - 7)
        out.append((code, val))
    return out


_E4M3 = e4m3_finite_values()


def e4m3_nearest(v: Fraction, negative: bool) -> int:
    """Nearest finite E4M3 code to |v| (ties to the even code), sign bit from ``negative``."""
    a = abs(v)
    best_code, best_d = None, None
    for code, val in _E4M3:
        d = abs(val - a)
        if best_d is None or d < best_d or (d == best_d and code % 2 == 0):
            best_code, best_d = code, d
    return (0x80 if negative else 0) | best_code


def quantize_group(bits: list[int]) -> tuple[Fraction, list[int]]:
    """One quantization group: s = rn32(amax/448); q = E4M3(rn32(x/s)); all-zero group -> s = 0."""
    vals = [bf16_value(b) for b in bits]
    amax = max(abs(v) for v in vals)
    s = round_binary32(amax / 448)
    codes = []
    for b, v in zip(bits, vals):
        if amax == 0:
            codes.append(0x80 if bf16_is_negative(b) else 0x00)
        else:
            codes.append(e4m3_nearest(round_binary32(v / s), bf16_is_negative(b)))
    return s, codes


def e4m3_value(code: int) -> Fraction:
    sign = -1 if code & 0x80 else 1
    for c, v in _E4M3:
        if c == code & 0x7F:
            return sign * v
    raise ValueError("NaN code")


def gemm_exact(a_codes, a_scales, b_codes, b_scales, absolute=False) -> list[list[Fraction]]:
    """C[m][n] = sum_k (dec(a[m][k]) * a_scales[m][k]) * (dec(b[n][k]) * b_scales[n][k]), exactly.

    Scales are given per element (already expanded from their tiles/blocks).
    absolute: the sum of the terms' magnitudes instead (for error bounds).
    """
    M, K = len(a_codes), len(a_codes[0])
    N = len(b_codes)
    out = []
    for m in range(M):
        row = []
        for n in range(N):
            acc = Fraction(0)
            for k in range(K):
                term = (e4m3_value(a_codes[m][k]) * Fraction(a_scales[m][k])) * \
                       (e4m3_value(b_codes[n][k]) * Fraction(b_scales[n][k]))
                acc += abs(term) if absolute else term
            row.append(acc)
        out.append(row)
    return out


def quantize_mx_block(bits: list[int]) -> tuple[int, list[int]]:
    """One microscaling block (OCP MX, E4M3 elements): e = floor(log2(amax)) - 8
    clamped to [-127, 127] (all-zero block: -127); q = nearest E4M3 of x / 2^e
    (exact rational, ties to the even code, largest finite code beyond 448).
    Returns (e, codes)."""
    vals = [bf16_value(b) for b in bits]
    amax = max(abs(v) for v in vals)
    e = -127 if amax == 0 else max(-127, min(127, _floor_log2(amax) - 8))
    scale = Fraction(2) ** e
    return e, [e4m3_nearest(v / scale, bf16_is_negative(b)) for b, v in zip(bits, vals)]


def retile_group(codes: list[int], scales: list[Fraction]) -> tuple[Fraction, list[int]]:
    """One 128x1 group of a cached 1x128 activation: v = rn32(dec(q) * s) per
    element (s: the element's 1x128 scale), then the group quantization of
    :func:`quantize_group` on the v (sign of each code = sign of its q)."""
    vals = [round_binary32(e4m3_value(c) * s) for c, s in zip(codes, scales)]
    neg = [bool(c & 0x80) for c in codes]
    amax = max(abs(v) for v in vals)
    s_new = round_binary32(amax / 448)
    out = []
    for v, ng in zip(vals, neg):
        if amax == 0:
            out.append(0x80 if ng else 0x00)
        else:
            out.append(e4m3_nearest(round_binary32(v / s_new), ng))
    return s_new, out
