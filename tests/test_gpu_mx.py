"""GPU parity of the microscaling variant (fp8_quantize_mx, fp8_gemm_mx).

Codes and E8M0 exponent bytes must equal the oracle's bit for bit; the
scaled-MFMA GEMM must match the unrounded float64 oracle GEMM of the same MX
operands to the same tolerance as the block-scaled GEMM.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import fine_grained_fp8_quantize_amd as fq
import oracle
import workloads as wl
from gpu_util import assert_bits_equal, assert_gemm_close, dev_bf16, host_codes, host_out, nan_out

pytestmark = pytest.mark.gpu


def _words_to_bytes(words: torch.Tensor, rows: int) -> np.ndarray:
    """GPU scale words [cols/128][rows] (byte b = block 4j + b) -> [rows][cols/32]."""
    w = words.contiguous().cpu().numpy().view(np.uint8).reshape(words.shape[0], words.shape[1], 4)
    return np.ascontiguousarray(w[:, :rows].transpose(1, 0, 2).reshape(rows, -1))


def _check_quant(bits: np.ndarray, what: str):
    q, s = fq.fp8_quantize_mx(dev_bf16(bits))
    torch.cuda.synchronize()
    q_ref, e_ref = oracle.quant_mx_1x32(bits)
    assert_bits_equal(_words_to_bytes(s, bits.shape[0]), e_ref, what + " E8M0 bytes")
    assert_bits_equal(host_codes(q), q_ref, what + " codes")


@pytest.mark.parametrize("which", ["x", "w"])
def test_mx_quant_dense_full_size(which):
    _check_quant(wl.dense_fprop()[which], "dense " + which)


@pytest.mark.parametrize("rows", [1, 15, 17, 129])
def test_mx_quant_ragged_rows(rows):
    _check_quant(wl.activation(2, "tiny_fprop", 95, rows, 384, 50.0), "rows=%d" % rows)


def test_mx_quant_special_blocks():
    rng = np.random.default_rng(31)
    rows = []
    z = np.zeros(128, np.uint16)
    z[::7] = 0x8000
    rows.append(z)                                                               # all zero
    rows.append(rng.integers(1, 0x80, 128).astype(np.uint16))                   # bf16 subnormals
    big = wl.f32_to_bf16_bits(rng.standard_normal(128).astype(np.float32) * 1e37)
    big[9] = 0x7F7F
    rows.append(big)                                                             # largest exponents
    rows.append(wl.f32_to_bf16_bits(rng.standard_normal(128).astype(np.float32) * 1e-37))  # clamp at -127
    rows.append(wl.f32_to_bf16_bits(np.full(128, 448.0 * 17 / 64, np.float32)))   # ties
    one = np.zeros(128, np.uint16)
    one[40] = wl.f32_to_bf16_bits(np.array([-5.0], np.float32))[0]
    rows.append(one)                                                             # single value
    mixed = wl.f32_to_bf16_bits(rng.standard_normal(128).astype(np.float32))
    mixed[32:64] = 0                                                             # one zero block among others
    rows.append(mixed)
    _check_quant(np.stack(rows), "special blocks")


def _gemm_case(m, n, k, out_dtype=torch.bfloat16, seed=0):
    a = wl.activation(seed, "tiny_fprop", 96, m, k, 50.0)
    b = wl.weight(seed, "tiny_fprop", 97, n, k)
    aq, asc = fq.fp8_quantize_mx(dev_bf16(a))
    bq, bsc = fq.fp8_quantize_mx(dev_bf16(b))
    c = fq.fp8_gemm_mx(aq, asc, bq, bsc, out_dtype, out=nan_out((m, n), out_dtype))
    torch.cuda.synchronize()
    got = host_out(c)
    a_q, a_e = oracle.quant_mx_1x32(a)
    b_q, b_e = oracle.quant_mx_1x32(b)
    assert_gemm_close(got, oracle.gemm_mx(a_q, a_e, b_q, b_e), "mx gemm %dx%dx%d" % (m, n, k))


def test_mx_gemm_tiny_all_elements():
    _gemm_case(128, 256, 512)


def test_mx_gemm_ragged_and_f32():
    _gemm_case(300, 200, 384, out_dtype=torch.float32)


def test_mx_gemm_dense_fprop_full():
    _gemm_case(4096, 4096, 7168)


def test_mx_gemm_k0_writes_zeros():
    a = torch.empty((64, 0), dtype=torch.uint8, device="cuda")
    s = torch.empty((0, 64), dtype=torch.int32, device="cuda")
    c = torch.full((64, 128), 3.0, dtype=torch.float32, device="cuda")
    b = torch.empty((128, 0), dtype=torch.uint8, device="cuda")
    sb = torch.empty((0, 128), dtype=torch.int32, device="cuda")
    fq.fp8_gemm_mx(a, s, b, sb, torch.float32, out=c)
    torch.cuda.synchronize()
    assert torch.all(c == 0)


def test_mx_gemm_224_wide_tiles():
    """N = 7168 makes the launcher pick 224-wide n tiles (32 x 224)."""
    _gemm_case(512, 7168, 256, seed=3)


def test_mx_gemm_padded_leading_dims():
    """Operands and output as row-padded views (lda, ldb > k; ldc > n)."""
    m, n, k = 200, 136, 256
    a = wl.activation(4, "tiny_fprop", 98, m, k, 50.0)
    b = wl.weight(4, "tiny_fprop", 99, n, k)
    aq, asc = fq.fp8_quantize_mx(dev_bf16(a))
    bq, bsc = fq.fp8_quantize_mx(dev_bf16(b))
    ap = torch.zeros((m, k + 32), dtype=torch.uint8, device="cuda")
    bp = torch.zeros((n, k + 64), dtype=torch.uint8, device="cuda")
    ap[:, :k] = aq.view(torch.uint8)
    bp[:, :k] = bq.view(torch.uint8)
    c = torch.full((m, n + 8), float("nan"), dtype=torch.bfloat16, device="cuda")
    fq.fp8_gemm_mx(ap[:, :k], asc, bp[:, :k], bsc, torch.bfloat16, out=c[:, :n])
    torch.cuda.synchronize()
    got = host_out(c)
    assert np.all(np.isnan(got[:, n:])), "columns past n written"
    a_q, a_e = oracle.quant_mx_1x32(a)
    b_q, b_e = oracle.quant_mx_1x32(b)
    assert_gemm_close(got[:, :n], oracle.gemm_mx(a_q, a_e, b_q, b_e), "mx gemm padded")


# ----------------------------------------- both GEMM operands in one launch

def test_mx_pair_equals_separate_launches_full_size():
    """X and W of the Dense Fprop shapes in one launch: byte-identical to two
    fp8_quantize_mx launches (each pinned to the oracle at full size above)."""
    d = wl.dense_fprop()
    x, w = dev_bf16(d["x"]), dev_bf16(d["w"])
    got = fq.fp8_quantize_mx_pair(x, w)
    ref = fq.fp8_quantize_mx(x) + fq.fp8_quantize_mx(w)
    torch.cuda.synchronize()
    for a, b, tag in zip(got, ref, ("q0", "scale0", "q1", "scale1")):
        assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), tag


@pytest.mark.parametrize("r0,c0,r1,c1", [(17, 384, 130, 256), (1, 128, 0, 128), (0, 256, 33, 512)])
def test_mx_pair_against_the_oracle(r0, c0, r1, c1):
    x0 = wl.activation(2, "tiny_fprop", 96, max(r0, 1), c0, 50.0)[:r0]
    x1 = wl.weight(2, "tiny_fprop", 97, max(r1, 1), c1)[:r1]
    d0 = dev_bf16(x0) if r0 else torch.empty((0, c0), dtype=torch.bfloat16, device="cuda")
    d1 = dev_bf16(x1) if r1 else torch.empty((0, c1), dtype=torch.bfloat16, device="cuda")
    q0, s0, q1, s1 = fq.fp8_quantize_mx_pair(d0, d1)
    torch.cuda.synchronize()
    for rows, x, q, s, tag in ((r0, x0, q0, s0, "x0"), (r1, x1, q1, s1, "x1")):
        if rows == 0:
            continue
        q_ref, e_ref = oracle.quant_mx_1x32(np.ascontiguousarray(x))
        assert_bits_equal(_words_to_bytes(s, rows), e_ref, tag + " E8M0 bytes")
        assert_bits_equal(host_codes(q), q_ref, tag + " codes")
