"""GPU parity of the FP8 activation-cache re-tile (fp8_retile_act_128x1).

The forward pass keeps X as 1x128 codes and scales; Wgrad needs 128x1 token
tiles. The re-tile must equal the oracle's dequantize-to-binary32 and
requantize bit for bit (codes and scales). Its inputs are the oracle's own
1x128 quantization of seeded activations, or seeded random codes and scales,
never GPU output. End to end, the Wgrad GEMM on the re-tiled cache must
match the oracle GEMM of the oracle's re-tiled codes.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import fine_grained_fp8_quantize_amd as fq
import oracle
import workloads as wl
from gpu_util import (assert_bits_equal, assert_gemm_close, dev_bf16, dev_codes, dev_f32, host_codes,
                      host_f32, host_out)

pytestmark = pytest.mark.gpu


def _retile(q: np.ndarray, s: np.ndarray, pad_q=0, pad_s=0, pad_qt=0, pad_st=0):
    """Run the GPU re-tile on host inputs, optionally with padded leading
    dimensions on every operand; returns the host codes and scales."""
    tokens, cols = q.shape
    qd = torch.zeros((tokens, cols + pad_q), dtype=torch.uint8, device="cuda")
    qd[:, :cols] = dev_codes(q)
    sd = torch.zeros((cols // 128, tokens + pad_s), dtype=torch.float32, device="cuda")
    sd[:, :tokens] = dev_f32(s[:, :tokens])
    qt = torch.full((cols, tokens + pad_qt), 0x5A, dtype=torch.uint8, device="cuda")
    st = torch.full((tokens // 128, cols + pad_st), 7.0, dtype=torch.float32, device="cuda")
    fq.fp8_retile_act_128x1(qd[:, :cols], sd[:, :tokens], q_t=qt[:, :tokens], scale_t=st[:, :cols])
    torch.cuda.synchronize()
    got_q, got_s = host_codes(qt), host_f32(st)
    assert np.all(got_q[:, tokens:] == 0x5A) and np.all(got_s[:, cols:] == 7.0), "padding written"
    return got_q[:, :tokens], got_s[:, :cols]


def _check(q, s, what, **pads):
    qt, st = _retile(q, s, **pads)
    qt_ref, st_ref = oracle.retile_128x1(q, s)
    assert_bits_equal(st, st_ref, what + " scales")
    assert_bits_equal(qt, qt_ref, what + " codes")


def test_retile_wgrad_x_full_size():
    """X of the Wgrad config (8192 tokens x 7168), cached 1x128 by the oracle."""
    q, s = oracle.quant_act_1x128(wl.wgrad()["x"])
    _check(q, s, "Wgrad X cache")


@pytest.mark.parametrize("tokens,cols", [(128, 128), (384, 256), (256, 1152)])
def test_retile_shapes_and_padded_leading_dims(tokens, cols):
    x = wl.activation(3, "wgrad", 80 + tokens // 128, tokens, cols, 50.0)
    q, s = oracle.quant_act_1x128(x)
    _check(q, s, "%dx%d" % (tokens, cols))
    _check(q, s, "%dx%d padded" % (tokens, cols), pad_q=16, pad_s=4, pad_qt=32, pad_st=8)


def test_retile_special_token_rows():
    """Zero rows (scale 0), signed zeros, subnormal-scale rows, outliers,
    one-signed rows and an all-zero 128x1 group."""
    rng = np.random.default_rng(41)
    x = wl.f32_to_bf16_bits(rng.standard_normal((256, 384)).astype(np.float32))
    x[3] = 0
    x[4] = 0x8000
    x[5] = wl.f32_to_bf16_bits(rng.standard_normal(384).astype(np.float32) * 1e-39)
    x[6] = wl.f32_to_bf16_bits(rng.standard_normal(384).astype(np.float32) * 3e3)
    x[7] = wl.f32_to_bf16_bits(-np.abs(rng.standard_normal(384)).astype(np.float32))
    x[128:256, 5] = 0
    x[130] = wl.f32_to_bf16_bits(rng.standard_normal(384).astype(np.float32) * 1e-30)
    q, s = oracle.quant_act_1x128(x)
    _check(q, s, "special rows")


def test_retile_random_codes_and_scales():
    """Every finite code with scales over many binades, including groups
    whose new scale is below 2^-60 (the division path) and zero scales."""
    rng = np.random.default_rng(42)
    finite = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], np.uint8)
    q = rng.choice(finite, size=(512, 640)).astype(np.uint8)
    s = (2.0 ** rng.uniform(-80, 20, size=(5, 512))).astype(np.float32)
    s[:, 128:256] = (2.0 ** rng.uniform(-120, -70, size=(5, 128))).astype(np.float32)
    s[:, 300] = 0
    q[300] = q[300] & 0x80                                  # a zero-scale token holds signed zeros
    _check(q, s, "random codes")


def test_wgrad_from_the_fp8_cache():
    """Wgrad with X taken from its forward-pass FP8 cache: dY quantized 128x1,
    X re-tiled, then the row-scaled GEMM (fp32 out), against the oracle GEMM
    of the oracle's own codes."""
    tokens, n_out, k_in = 1024, 256, 384
    dy = wl.grad_rowscaled(1, "wgrad", 90, tokens, n_out)
    x = wl.activation(1, "wgrad", 91, tokens, k_in, 50.0)
    xq, xs = oracle.quant_act_1x128(x)                       # the forward-pass cache
    aq, as_ = fq.fp8_quantize_act(dev_bf16(dy), "128x1")
    bq, bs = fq.fp8_retile_act_128x1(dev_codes(xq), dev_f32(xs))
    c = fq.fp8_gemm(aq, as_, bq, bs, "row", torch.float32)
    torch.cuda.synchronize()
    aq_ref, as_ref = oracle.quant_act_128x1(dy)
    bq_ref, bs_ref = oracle.retile_128x1(xq, xs)
    assert_bits_equal(host_codes(bq), bq_ref, "re-tiled X codes")
    ref = oracle.gemm(aq_ref, as_ref, bq_ref, bs_ref, "row")
    assert_gemm_close(host_out(c), ref, "Wgrad from the FP8 cache")


def test_retile_empty_is_noop():
    q = torch.empty((0, 256), dtype=torch.uint8, device="cuda")
    s = torch.empty((2, 0), dtype=torch.float32, device="cuda")
    qt, st = fq.fp8_retile_act_128x1(q, s)
    assert qt.shape == (256, 0) and st.shape == (0, 256)


# ---------------------------- dY quantized and the X cache re-tiled, one launch

def test_quant_retile_one_launch_equals_separate_full_size():
    """The Wgrad config from the cache: dY [8192][2048] quantized 128x1 and
    the cached X [8192][7168] re-tiled, in one launch, byte-identical to the
    two separate launches (each pinned to the oracle above)."""
    g = wl.wgrad()
    dy = dev_bf16(g["dy"])
    xq_h, xs_h = oracle.quant_act_1x128(g["x"])
    xq, xs = dev_codes(xq_h), dev_f32(xs_h)
    got = fq.fp8_quantize_act_128x1_retile(dy, xq, xs)
    ref = fq.fp8_quantize_act(dy, "128x1") + fq.fp8_retile_act_128x1(xq, xs)
    torch.cuda.synchronize()
    for a, b, tag in zip(got, ref, ("q0", "scale0", "q1", "scale1")):
        assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), tag


@pytest.mark.parametrize("cols0,cols1", [(136, 256), (8, 128), (0, 384), (264, 0)])
def test_quant_retile_one_launch_against_the_oracle(cols0, cols1):
    tokens = 384
    dy = wl.activation(3, "wgrad", 90, tokens, max(cols0, 8), None)[:, :cols0]
    x = wl.activation(3, "wgrad", 91, tokens, max(cols1, 128), 50.0)[:, :cols1]
    xq_h, xs_h = oracle.quant_act_1x128(np.ascontiguousarray(x)) if cols1 else (
        np.zeros((tokens, 0), np.uint8), np.zeros((0, tokens), np.float32))
    d0 = dev_bf16(dy) if cols0 else torch.empty((tokens, 0), dtype=torch.bfloat16, device="cuda")
    xq = dev_codes(xq_h) if cols1 else torch.empty((tokens, 0), dtype=torch.uint8, device="cuda")
    xs = dev_f32(xs_h) if cols1 else torch.empty((0, tokens), dtype=torch.float32, device="cuda")
    q0, s0, q1, s1 = fq.fp8_quantize_act_128x1_retile(d0, xq, xs)
    torch.cuda.synchronize()
    if cols0:
        q_ref, s_ref = oracle.quant_act_128x1(np.ascontiguousarray(dy))
        assert_bits_equal(host_f32(s0), s_ref, "dY scales")
        assert_bits_equal(host_codes(q0), q_ref, "dY codes")
    if cols1:
        qt_ref, st_ref = oracle.retile_128x1(xq_h, xs_h)
        assert_bits_equal(host_f32(s1), st_ref, "X re-tile scales")
        assert_bits_equal(host_codes(q1), qt_ref, "X re-tile codes")
