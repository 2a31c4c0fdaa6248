"""GPU parity of the MoE expert Wgrad (fp8_grouped_gemm_wgrad).

dY and X in the expert-sorted layout (128-padded segments, zero padding
rows) are quantized on the GPU in 128x1 token tiles; each expert's gradient
contracts over its own token segment. Compared with the oracle's per-expert
row-scale GEMM on the oracle's codes.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import fine_grained_fp8_quantize_amd as fq
import oracle
import workloads as wl
from gpu_util import assert_bits_equal, assert_gemm_close, dev_bf16, host_codes, host_f32, host_out, nan_out

pytestmark = pytest.mark.gpu


def _packed(rows, cols, tensor_id, grad):
    rows = np.asarray(rows, dtype=np.int64)
    off = wl.pad_offsets(rows)
    real = (wl.grad_rowscaled(1, "grouped_fprop", tensor_id, int(rows.sum()), cols) if grad
            else wl.activation(1, "grouped_fprop", tensor_id, int(rows.sum()), cols, 50.0))
    out = np.zeros((int(off[-1]), cols), np.uint16)
    src = 0
    for e in range(len(rows)):
        out[off[e]:off[e] + rows[e]] = real[src:src + rows[e]]
        src += int(rows[e])
    return out, off


def _wgrad_case(rows, m, n, out_dtype=torch.float32):
    dy, off = _packed(rows, m, 100, grad=True)
    x, _ = _packed(rows, n, 101, grad=False)
    aq, as_ = fq.fp8_quantize_act(dev_bf16(dy), "128x1")
    bq, bs = fq.fp8_quantize_act(dev_bf16(x), "128x1")
    off_d = torch.from_numpy(off.astype(np.int32)).cuda()
    out = fq.fp8_grouped_gemm_wgrad(off_d, aq, as_, bq, bs, out_dtype,
                                    out=nan_out((len(rows), m, n), out_dtype))
    torch.cuda.synchronize()
    a_q, a_s = oracle.quant_act_128x1(dy)
    b_q, b_s = oracle.quant_act_128x1(x)
    assert_bits_equal(host_codes(aq), a_q, "dY^T codes")
    assert_bits_equal(host_f32(as_), a_s, "dY^T scales")
    _compare_experts(out, off, rows, a_q, a_s, b_q, b_s, "wgrad")


def _compare_experts(out, off, rows, a_q, a_s, b_q, b_s, what):
    """Every dW_e in full against the oracle's row-scale GEMM over expert e's
    token segment (rms over that dW_e); an empty segment must give zeros."""
    for e in range(len(rows)):
        t0, t1 = int(off[e]), int(off[e + 1])
        got = host_out(out[e])
        if t1 == t0:
            assert np.all(got == 0), "%s expert %d: empty segment must give zeros" % (what, e)
            continue
        ref = oracle.gemm(np.ascontiguousarray(a_q[:, t0:t1]), np.ascontiguousarray(a_s[t0 // 128:t1 // 128]),
                          np.ascontiguousarray(b_q[:, t0:t1]), np.ascontiguousarray(b_s[t0 // 128:t1 // 128]),
                          "row")
        assert_gemm_close(got, ref, "%s expert %d (%d tokens)" % (what, e, rows[e]))


def test_grouped_wgrad_edge_segments():
    # empty expert, 1 token, exact 128, 129 (two slabs), a 2-slab expert
    _wgrad_case([0, 1, 128, 129, 256], m=256, n=384)


def test_grouped_wgrad_ragged_output_and_bf16():
    _wgrad_case([3, 200, 64], m=320, n=200, out_dtype=torch.bfloat16)


def test_grouped_wgrad_all_empty():
    _wgrad_case([0, 0, 0], m=256, n=256)


def test_grouped_wgrad_moe_config_full():
    """MoE up-projection Wgrad: 32 experts, dW_e [4096][7168] over each expert's
    tokens (8192 routed rows, 10112 padded); every dW_e compared in full."""
    _wgrad_case(wl.moe_rows(0), m=4096, n=7168)


def _wgrad_from_dispatch_cache(rows, m, k, tokens, top_k):
    """MoE Wgrad with X taken from the FP8 cache the dispatch quantizer wrote:
    the expert-sorted 1x128 codes and scales (padding rows zeroed before the
    scatter) re-tiled to 128x1 token tiles, then the grouped-over-K GEMM.
    Segments are 128-aligned, so no 128-token tile straddles two experts."""
    rows = np.asarray(rows, dtype=np.int64)
    d = wl.moe_dispatch(0, k=k, tokens=tokens, top_k=top_k, rows=rows)
    off = d["offsets"]
    m_total = int(off[-1])
    q = torch.zeros((m_total, k), dtype=torch.uint8, device="cuda")         # padding rows stay zero
    s = torch.zeros((k // 128, m_total), dtype=torch.float32, device="cuda")
    fq.fp8_quantize_act_scatter(dev_bf16(d["x"]), torch.from_numpy(d["dst_rows"]).cuda(), m_total, q=q, scale=s)
    bq, bs = fq.fp8_retile_act_128x1(q, s)
    dy, _ = _packed(rows, m, 102, grad=True)
    aq, as_ = fq.fp8_quantize_act(dev_bf16(dy), "128x1")
    off_d = torch.from_numpy(off.astype(np.int32)).cuda()
    out = fq.fp8_grouped_gemm_wgrad(off_d, aq, as_, bq, bs, torch.float32,
                                    out=nan_out((len(rows), m, k), torch.float32))
    torch.cuda.synchronize()
    xq_ref, xs_ref, _ = oracle.quant_act_scatter(d["x"], d["dst_rows"], m_total)
    b_q, b_s = oracle.retile_128x1(xq_ref, xs_ref)
    assert_bits_equal(host_codes(bq), b_q, "re-tiled cache codes")
    assert_bits_equal(host_f32(bs), b_s, "re-tiled cache scales")
    a_q, a_s = oracle.quant_act_128x1(dy)
    _compare_experts(out, off, rows, a_q, a_s, b_q, b_s, "cached-X wgrad")


def test_grouped_wgrad_from_dispatch_cache_small():
    _wgrad_from_dispatch_cache([5, 0, 130, 64, 1], m=256, k=384, tokens=200, top_k=2)


def test_grouped_wgrad_from_dispatch_cache_moe_full():
    """The MoE config: 8192 tokens x 7168, top-8 routes into 32 local experts,
    dW [32][4096][7168]; every dW_e compared in full."""
    _wgrad_from_dispatch_cache(wl.moe_rows(0), m=4096, k=7168, tokens=8192, top_k=8)


def test_grouped_wgrad_padded_output_and_operand_views():
    """Operands as padded views (lda, ldb past the token count; scale rows past
    m and n) and dW as a padded [E][m][n] view (ldc > n, expert stride >
    m * ldc): every expert matches the oracle and nothing outside the
    windows is written."""
    rows = [5, 0, 300]
    m, n = 256, 136
    dy, off = _packed(rows, m, 102, grad=True)
    x, _ = _packed(rows, n, 103, grad=False)
    a_q, a_s = oracle.quant_act_128x1(dy)
    b_q, b_s = oracle.quant_act_128x1(x)
    kt = a_q.shape[1]
    ap = torch.zeros((m, kt + 32), dtype=torch.uint8, device="cuda")
    ap[:, :kt] = torch.from_numpy(a_q).cuda()
    bp = torch.zeros((n, kt + 64), dtype=torch.uint8, device="cuda")
    bp[:, :kt] = torch.from_numpy(b_q).cuda()
    asp = torch.full((kt // 128, m + 8), 7.0, device="cuda")
    asp[:, :m] = torch.from_numpy(a_s).cuda()
    bsp = torch.full((kt // 128, n + 12), 7.0, device="cuda")
    bsp[:, :n] = torch.from_numpy(b_s).cuda()
    E = len(rows)
    c = torch.full((E, m + 3, n + 8), float("nan"), dtype=torch.float32, device="cuda")
    off_d = torch.from_numpy(off.astype(np.int32)).cuda()
    fq.fp8_grouped_gemm_wgrad(off_d, ap[:, :kt], asp[:, :m], bp[:, :kt], bsp[:, :n], torch.float32,
                              out=c[:, :m, :n])
    torch.cuda.synchronize()
    got = c.cpu().numpy().astype(np.float64)
    assert np.all(np.isnan(got[:, m:, :])) and np.all(np.isnan(got[:, :, n:])), "written outside the windows"
    for e in range(E):
        t0, t1 = int(off[e]), int(off[e + 1])
        if t1 == t0:
            assert np.all(got[e, :m, :n] == 0), "expert %d: empty segment must give zeros" % e
            continue
        ref = oracle.gemm(np.ascontiguousarray(a_q[:, t0:t1]), np.ascontiguousarray(a_s[t0 // 128:t1 // 128]),
                          np.ascontiguousarray(b_q[:, t0:t1]), np.ascontiguousarray(b_s[t0 // 128:t1 // 128]), "row")
        assert_gemm_close(got[e, :m, :n], ref, "padded wgrad expert %d" % e)
