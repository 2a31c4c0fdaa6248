"""CPU oracle for fine-grained FP8 quantization and the block-scaled FP8 GEMM.

TEST INFRASTRUCTURE ONLY: the tests, ``__graft_entry__.smoke()`` and the
benchmark's CPU-baseline leg may use it; the GPU library never does, and the
two share no code.

Quantization runs in the scalar C file ``fp8_oracle.c`` (binary32 IEEE, see
its header for the readings). The GEMM is its plain definition: dequantize both
FP8 operands exactly in float64 (E4M3 value times its FP32 scale) and multiply
them with numpy's float64 matmul:

    C[m][n] = sum_k (dec(qA[m,k]) * sA(m,k)) * (dec(qB[n,k]) * sB(n,k))

which is what the FP8 GEMM of the pages computes up to rounding order: FP8
operands in, per-group scales applied during accumulation, BF16 or FP32 out
(page "Deepseek Ai News Expert Interview", passages on promotion to FP32
registers and on BF16/FP32 GEMM outputs; page "Is aI Hitting a Wall?",
passage on the dequantization overhead).
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

from . import build as _build

_LIB = None


def lib() -> ctypes.CDLL:
    """Load (building if needed) the C oracle; FP8Q_ORACLE_LIBRARY names
    another build of it (the sanitizer build of the CPU suites)."""
    global _LIB
    if _LIB is None:
        path = os.environ.get("FP8Q_ORACLE_LIBRARY") or _build.build(force=False)
        L = ctypes.CDLL(path)
        u8p = ctypes.POINTER(ctypes.c_uint8)
        u16p = ctypes.POINTER(ctypes.c_uint16)
        f32p = ctypes.POINTER(ctypes.c_float)
        i64 = ctypes.c_int64
        L.oracle_bf16_to_f32.argtypes = [ctypes.c_uint16]
        L.oracle_bf16_to_f32.restype = ctypes.c_float
        L.oracle_e4m3_decode.argtypes = [ctypes.c_uint8]
        L.oracle_e4m3_decode.restype = ctypes.c_double
        L.oracle_e4m3_encode_bits.argtypes = [ctypes.c_float]
        L.oracle_e4m3_encode_bits.restype = ctypes.c_uint8
        L.oracle_e4m3_encode_search.argtypes = [ctypes.c_float]
        L.oracle_e4m3_encode_search.restype = ctypes.c_uint8
        for name in ("oracle_quant_act_1x128", "oracle_quant_act_128x1",
                     "oracle_quant_weight_128x128"):
            getattr(L, name).argtypes = [u16p, i64, i64, i64, u8p, i64, f32p, i64]
            getattr(L, name).restype = None
        L.oracle_encoders_disagree.argtypes = [ctypes.c_uint32, ctypes.c_uint32, ctypes.c_uint32,
                                               ctypes.POINTER(ctypes.c_uint32)]
        L.oracle_encoders_disagree.restype = ctypes.c_int64
        L.oracle_quant_pairs.argtypes = [u16p, u16p, i64, u8p]
        L.oracle_quant_pairs.restype = None
        L.oracle_quant_mx_1x32.argtypes = [u16p, i64, i64, i64, u8p, i64, u8p, i64]
        L.oracle_quant_mx_1x32.restype = None
        L.oracle_retile_128x1.argtypes = [u8p, i64, i64, i64, f32p, i64, u8p, i64, f32p, i64]
        L.oracle_retile_128x1.restype = None
        _LIB = L
    return _LIB


class OutOfContract(ValueError):
    """A non-finite input (NaN/Inf bf16 value, NaN E4M3 code 0x7F/0xFF, NaN
    E8M0 byte 0xFF, or a non-finite scale): the method's numbers are defined
    for finite values only, so the oracle refuses rather than guess."""


def _finite_bf16(x: np.ndarray, what: str) -> None:
    if np.any((np.asarray(x, dtype=np.uint16) & 0x7F80) == 0x7F80):
        raise OutOfContract("%s holds a NaN or infinite bf16 value" % what)


def _finite_codes(q: np.ndarray, what: str) -> None:
    if np.any((np.asarray(q, dtype=np.uint8) & 0x7F) == 0x7F):
        raise OutOfContract("%s holds a NaN E4M3 code" % what)


def _finite_scales(s, what: str) -> None:
    if not np.all(np.isfinite(np.asarray(s, dtype=np.float64))):
        raise OutOfContract("%s holds a non-finite scale" % what)


def _p(a: np.ndarray, ctype):
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(ctypes.POINTER(ctype))


# ------------------------------------------------------------------ formats

def e4m3_decode_table() -> np.ndarray:
    """float64[256]: the value of every E4M3 code (NaN for 0x7F and 0xFF)."""
    L = lib()
    return np.array([L.oracle_e4m3_decode(c) for c in range(256)], dtype=np.float64)


def e4m3_encode(v: float, method: str = "bits") -> int:
    L = lib()
    f = L.oracle_e4m3_encode_bits if method == "bits" else L.oracle_e4m3_encode_search
    return int(f(ctypes.c_float(v)))


def encoders_disagree(lo_bits: int, hi_bits: int, stride: int = 1) -> tuple[int, int]:
    """Count fp32 patterns lo, lo+stride, ... <= hi (both signs) where the two encoders differ."""
    first = ctypes.c_uint32(0)
    n = lib().oracle_encoders_disagree(lo_bits, hi_bits, stride, ctypes.byref(first))
    return int(n), int(first.value)


# --------------------------------------------------------------- quantizers

def quant_act_1x128(x: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """bf16 bits X[rows][cols] -> (Q uint8[rows][cols], S float32[cols/128][rows])."""
    x = np.ascontiguousarray(x, dtype=np.uint16)
    _finite_bf16(x, "x")
    rows, cols = x.shape
    assert cols % 128 == 0
    q = np.empty((rows, cols), dtype=np.uint8)
    s = np.empty((cols // 128, rows), dtype=np.float32)
    lib().oracle_quant_act_1x128(_p(x, ctypes.c_uint16), rows, cols, cols,
                                 _p(q, ctypes.c_uint8), cols, _p(s, ctypes.c_float), rows)
    return q, s


def quant_act_scatter(x: np.ndarray, dst_rows: np.ndarray, m_total: int):
    """Quantize before dispatch (page "Eliminate Deepseek Ai News For Good",
    passage on quantizing activations before the MoE dispatch): every token
    row of bf16 X[tokens][cols] gets its 1x128 quantization, and the codes and
    scales of token t go to each destination row dst_rows[t][k] in
    [0, m_total). Returns (Q uint8[m_total][cols], S float32[cols/128][m_total],
    written bool[m_total]); unwritten rows hold zeros."""
    q_tok, s_tok = quant_act_1x128(x)
    dst = np.asarray(dst_rows, dtype=np.int64)
    tokens, cols = q_tok.shape
    q = np.zeros((m_total, cols), dtype=np.uint8)
    s = np.zeros((cols // 128, m_total), dtype=np.float32)
    written = np.zeros(m_total, dtype=bool)
    t_idx, k_idx = np.nonzero((dst >= 0) & (dst < m_total))
    d = dst[t_idx, k_idx]
    q[d] = q_tok[t_idx]
    s[:, d] = s_tok[:, t_idx]
    written[d] = True
    return q, s, written


def quant_mx_1x32(x: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """Microscaling (OCP MX, E4M3 elements): bf16 bits X[rows][cols] ->
    (Q uint8[rows][cols], E uint8[rows][cols/32] E8M0 exponent bytes)."""
    x = np.ascontiguousarray(x, dtype=np.uint16)
    _finite_bf16(x, "x")
    rows, cols = x.shape
    assert cols % 32 == 0
    q = np.empty((rows, cols), dtype=np.uint8)
    e = np.empty((rows, cols // 32), dtype=np.uint8)
    lib().oracle_quant_mx_1x32(_p(x, ctypes.c_uint16), rows, cols, cols,
                               _p(q, ctypes.c_uint8), cols, _p(e, ctypes.c_uint8), cols // 32)
    return q, e


def dequant_mx(q: np.ndarray, e: np.ndarray) -> np.ndarray:
    """float64 value of MX codes: dec(q) * 2^(E - 127) per 32-element block."""
    rows, cols = q.shape
    scale = np.ldexp(1.0, e.astype(np.int64) - 127)
    return _dec()[q] * np.repeat(scale, 32, axis=1)


def gemm_mx(a_q: np.ndarray, a_e: np.ndarray, b_q: np.ndarray, b_e: np.ndarray) -> np.ndarray:
    """float64 C[m][n] = deq_mx(A)[m][:] . deq_mx(B)[n][:], unrounded (both
    operands K-contiguous, 32-element blocks along K)."""
    for q, e, what in ((a_q, a_e, "a"), (b_q, b_e, "b")):
        _finite_codes(q, what)
        if np.any(np.asarray(e, dtype=np.uint8) == 0xFF):
            raise OutOfContract("%s holds the NaN E8M0 byte 0xFF" % what)
    return dequant_mx(a_q, a_e) @ dequant_mx(b_q, b_e).T


def quant_act_128x1(x: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """bf16 bits X[tokens][cols] -> (QT uint8[cols][tokens], S float32[tokens/128][cols])."""
    x = np.ascontiguousarray(x, dtype=np.uint16)
    _finite_bf16(x, "x")
    rows, cols = x.shape
    assert rows % 128 == 0
    qt = np.empty((cols, rows), dtype=np.uint8)
    s = np.empty((rows // 128, cols), dtype=np.float32)
    lib().oracle_quant_act_128x1(_p(x, ctypes.c_uint16), rows, cols, cols,
                                 _p(qt, ctypes.c_uint8), rows, _p(s, ctypes.c_float), cols)
    return qt, s


def retile_128x1(q: np.ndarray, s: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """Cached FP8 activation re-tiled for Wgrad: 1x128 codes Q uint8[tokens][cols]
    with scales S float32[cols/128][tokens] -> (QT uint8[cols][tokens],
    ST float32[tokens/128][cols]). Every value is dequantized to binary32,
    v = fl32(dec(q) * s), and quantized again in 128x1 tiles along tokens
    (page "Is aI Hitting a Wall?", passage on keeping activations in FP8 for
    the backward pass)."""
    q = np.ascontiguousarray(q, dtype=np.uint8)
    rows, cols = q.shape
    assert rows % 128 == 0 and cols % 128 == 0
    s = np.ascontiguousarray(s[:, :rows], dtype=np.float32)
    _finite_codes(q, "q")
    _finite_scales(s, "scale")
    assert s.shape == (cols // 128, rows)
    qt = np.empty((cols, rows), dtype=np.uint8)
    st = np.empty((rows // 128, cols), dtype=np.float32)
    lib().oracle_retile_128x1(_p(q, ctypes.c_uint8), rows, cols, cols, _p(s, ctypes.c_float), rows,
                              _p(qt, ctypes.c_uint8), rows, _p(st, ctypes.c_float), cols)
    return qt, st


def quant_weight_128x128(w: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """bf16 bits W[n][k] -> (Q uint8[n][k], S float32[n/128][k/128])."""
    w = np.ascontiguousarray(w, dtype=np.uint16)
    _finite_bf16(w, "w")
    n, k = w.shape
    assert n % 128 == 0 and k % 128 == 0
    q = np.empty((n, k), dtype=np.uint8)
    s = np.empty((n // 128, k // 128), dtype=np.float32)
    lib().oracle_quant_weight_128x128(_p(w, ctypes.c_uint16), n, k, k,
                                      _p(q, ctypes.c_uint8), k, _p(s, ctypes.c_float), k // 128)
    return q, s


def quant_pairs(x: np.ndarray, amax: np.ndarray) -> np.ndarray:
    """E4M3(fl32(x / fl32(|amax| / 448))) element-wise on bf16 bit arrays."""
    x = np.ascontiguousarray(x, dtype=np.uint16)
    amax = np.ascontiguousarray(amax, dtype=np.uint16)
    _finite_bf16(x, "x")
    _finite_bf16(amax, "amax")
    assert x.shape == amax.shape
    q = np.empty(x.shape, dtype=np.uint8)
    lib().oracle_quant_pairs(_p(x, ctypes.c_uint16), _p(amax, ctypes.c_uint16), x.size,
                             _p(q, ctypes.c_uint8))
    return q


# ---------------------------------------------------------- dequantization

_DEC = None


def _dec() -> np.ndarray:
    global _DEC
    if _DEC is None:
        _DEC = e4m3_decode_table()
    return _DEC


def dequant_rows_1x128(q: np.ndarray, s: np.ndarray) -> np.ndarray:
    """float64 operand from K-contiguous codes q[r][k] with slab-major scales s[k/128][r]."""
    rows, k = q.shape
    assert s.shape[0] == k // 128 and s.shape[1] >= rows
    scale = np.repeat(s[:, :rows].astype(np.float64).T, 128, axis=1)
    return _dec()[q] * scale


def dequant_block_128x128(q: np.ndarray, s: np.ndarray) -> np.ndarray:
    """float64 operand from codes q[n][k] with block scales s[n/128][k/128]."""
    n, k = q.shape
    scale = np.repeat(np.repeat(s.astype(np.float64), 128, axis=0), 128, axis=1)[:n, :k]
    return _dec()[q] * scale


# -------------------------------------------------------------------- GEMM

def gemm(a_q: np.ndarray, a_s: np.ndarray, b_q: np.ndarray, b_s: np.ndarray,
         b_scale_kind: str = "block") -> np.ndarray:
    """float64 C[m][n] = deq(A)[m][:] . deq(B)[n][:], unrounded.

    A: codes [m][k] (K contiguous) with slab-major 1x128 scales [k/128][m].
    B: codes [n][k] (K contiguous) with scales either 128x128 blocks
    [n/128][k/128] (``"block"``) or one per (slab, row) [k/128][n] (``"row"``,
    the Wgrad case where both operands were quantized in 128x1 token tiles).
    """
    _finite_codes(a_q, "a")
    _finite_codes(b_q, "b")
    _finite_scales(a_s, "a_scale")
    _finite_scales(b_s, "b_scale")
    A = dequant_rows_1x128(a_q, a_s)
    if b_scale_kind == "block":
        B = dequant_block_128x128(b_q, b_s)
    elif b_scale_kind == "row":
        B = dequant_rows_1x128(b_q, b_s)
    else:
        raise ValueError(b_scale_kind)
    return A @ B.T


def gemm_rows(row_idx: np.ndarray, a_q: np.ndarray, a_s: np.ndarray, b_q: np.ndarray,
              b_s: np.ndarray, b_scale_kind: str = "block") -> np.ndarray:
    """Selected rows of :func:`gemm` (float64 [len(row_idx)][n])."""
    row_idx = np.asarray(row_idx)
    return gemm(np.ascontiguousarray(a_q[row_idx]), np.ascontiguousarray(a_s[:, row_idx]),
                b_q, b_s, b_scale_kind)


def gemm_tensor(a_q: np.ndarray, a_s: float, b_q: np.ndarray, b_s: float) -> np.ndarray:
    """Per-tensor scaled FP8 GEMM, the accumulation-study arm whose whole K
    sum stays inside the matrix core (page "Eliminate Deepseek Ai News For
    Good", passage on limited accumulation precision at K = 4096):

        C[m][n] = sA * sB * sum_k dec(qA[m,k]) * dec(qB[n,k])

    E4M3 values are multiples of 2^-9 below 2^9, so every product is a
    multiple of 2^-18 below 2^18 and, for K <= 131072, every partial sum is
    exact in float64 in any order: the matmul is the exact sum, and the one
    rounding is the final multiplication by sA * sB (itself exact)."""
    assert a_q.shape[1] <= 131072
    _finite_codes(a_q, "a")
    _finite_codes(b_q, "b")
    _finite_scales([a_s, b_s], "per-tensor scale")
    d = _dec()
    return (float(a_s) * float(b_s)) * (d[a_q] @ d[b_q].T)


def grouped_gemm(offsets: np.ndarray, rows: np.ndarray, a_q: np.ndarray, a_s: np.ndarray,
                 b_q: np.ndarray, b_s: np.ndarray) -> np.ndarray:
    """Per expert e: C[off_e : off_e + rows_e] = GEMM(A segment, W_e); padding rows are 0.

    a_q [m_total][k], a_s [k/128][m_total], b_q [E][n][k], b_s [E][n/128][k/128].
    """
    m_total = a_q.shape[0]
    n = b_q.shape[1]
    out = np.zeros((m_total, n), dtype=np.float64)
    for e in range(len(rows)):
        r0, r = int(offsets[e]), int(rows[e])
        if r == 0:
            continue
        out[r0:r0 + r] = gemm(np.ascontiguousarray(a_q[r0:r0 + r]),
                              np.ascontiguousarray(a_s[:, r0:r0 + r]), b_q[e], b_s[e], "block")
    return out


def grouped_gemm_wgrad(offsets: np.ndarray, a_q: np.ndarray, a_s: np.ndarray, b_q: np.ndarray,
                       b_s: np.ndarray) -> np.ndarray:
    """MoE expert Wgrad: dW_e = GEMM over expert e's token slice [off_e, off_e+1)
    of A = dY^T codes [m][k_total] and B = X^T codes [n][k_total], both with
    per-(slab, row) scales [k_total/128][rows] (the Wgrad GEMM of page
    dssusan.co.kr Q&A board, Figure 6, per expert). Returns float64 [E][m][n]."""
    m, n = a_q.shape[0], b_q.shape[0]
    E = len(offsets) - 1
    out = np.zeros((E, m, n), dtype=np.float64)
    for e in range(E):
        t0, t1 = int(offsets[e]), int(offsets[e + 1])
        if t1 == t0:
            continue
        out[e] = gemm(np.ascontiguousarray(a_q[:, t0:t1]), np.ascontiguousarray(a_s[t0 // 128:t1 // 128]),
                      np.ascontiguousarray(b_q[:, t0:t1]), np.ascontiguousarray(b_s[t0 // 128:t1 // 128]),
                      "row")
    return out


def bf16_round(a: np.ndarray) -> np.ndarray:
    """Round float64 values to bf16 (via float32, nearest-even each step) as float64.

    Diagnostic only: the pass criteria compare against the unrounded result.
    """
    f = a.astype(np.float32)
    u = f.view(np.uint32)
    r = ((u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)) << np.uint32(16)
    return r.view(np.float32).astype(np.float64)
