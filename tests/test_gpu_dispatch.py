"""GPU parity of quantize-before-dispatch (fp8_quantize_act_scatter).

Every token row is quantized once (1x128) and its codes and scales land in
each expert-sorted destination row the routing names. Codes and scales must
equal the oracle's bit for bit; rows no route names are left untouched; the
grouped GEMM on the scattered layout, with poisoned padding rows, must match
the oracle GEMM on the gathered rows.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import fine_grained_fp8_quantize_amd as fq
import oracle
import workloads as wl
from gpu_util import assert_bits_equal, assert_gemm_close, dev_bf16, dev_codes, dev_f32, host_codes, host_f32, host_out

pytestmark = pytest.mark.gpu

SENTINEL_CODE = 0x5A
SENTINEL_SCALE = 7.0


def _scatter(x_bits, dst, m_total, fill_code=SENTINEL_CODE, fill_scale=SENTINEL_SCALE):
    cols = x_bits.shape[1]
    q = torch.full((m_total, cols), fill_code, dtype=torch.uint8, device="cuda")
    s = torch.full((cols // 128, m_total), fill_scale, dtype=torch.float32, device="cuda")
    d = torch.from_numpy(np.ascontiguousarray(dst, dtype=np.int32)).cuda()
    fq.fp8_quantize_act_scatter(dev_bf16(x_bits), d, m_total, q=q, scale=s)
    torch.cuda.synchronize()
    return host_codes(q), host_f32(s)


def _check(x_bits, dst, m_total, what):
    q, s = _scatter(x_bits, dst, m_total)
    q_ref, s_ref, written = oracle.quant_act_scatter(x_bits, dst, m_total)
    assert_bits_equal(q[written], q_ref[written], what + " codes")
    assert_bits_equal(s[:, written], s_ref[:, written], what + " scales")
    assert np.all(q[~written] == SENTINEL_CODE), what + ": unrouted rows were written"
    assert np.all(s[:, ~written] == SENTINEL_SCALE), what + ": unrouted scales were written"


def test_scatter_moe_config_full_size():
    """8192 tokens x 7168, top-8 slots, 32 local experts, 10112 padded rows."""
    d = wl.moe_dispatch(0)
    _check(d["x"], d["dst_rows"], int(d["offsets"][-1]), "MoE dispatch")


@pytest.mark.parametrize("tokens,topk", [(1, 1), (15, 3), (17, 8), (100, 2)])
def test_scatter_ragged_tokens_and_routes(tokens, topk):
    rng = np.random.default_rng(tokens * 10 + topk)
    x = wl.activation(1, "grouped_fprop", 60 + topk, tokens, 384, 50.0)
    m_total = 2 * tokens * topk + 5
    rows = rng.permutation(m_total)[:tokens * topk].reshape(tokens, topk).astype(np.int32)
    rows[rng.random(rows.shape) < 0.3] = -1                  # routes to other layouts
    rows[rng.random(rows.shape) < 0.05] = m_total + 3         # out of range: ignored
    _check(x, rows, m_total, "tokens=%d topk=%d" % (tokens, topk))


def test_scatter_identity_equals_tile_quantizer():
    x = wl.activation(1, "grouped_fprop", 70, 300, 512, 50.0)
    dst = np.arange(300, dtype=np.int32)[:, None]
    q, s = _scatter(x, dst, 300)
    qa, sa = fq.fp8_quantize_act(dev_bf16(x))
    torch.cuda.synchronize()
    assert_bits_equal(q, host_codes(qa), "identity scatter codes")
    assert_bits_equal(s, host_f32(sa), "identity scatter scales")


def test_scatter_edge_tiles_duplicated():
    """Special tiles (all zero, subnormal scales, single values) routed twice."""
    rng = np.random.default_rng(5)
    base = wl.activation(1, "grouped_fprop", 71, 8, 256, 50.0)
    base[1] = 0
    base[2, :128] = 0x8000
    base[3] = wl.f32_to_bf16_bits(rng.standard_normal(256).astype(np.float32) * 1e-38)
    base[4] = 0
    base[4, 77] = wl.f32_to_bf16_bits(np.array([-3.0], np.float32))[0]
    dst = np.stack([np.arange(8) * 2, np.arange(8) * 2 + 1], axis=1).astype(np.int32)
    _check(base, dst, 16, "duplicated edge tiles")


def test_scatter_then_grouped_gemm_ignores_padding_rows():
    """End to end: scatter into a layout whose padding rows hold NaN codes and
    NaN scales, then the grouped GEMM: real rows match the oracle GEMM of the
    gathered rows and padding rows come out zero."""
    n, k = 256, 384
    rows = np.array([5, 0, 130, 64, 1], dtype=np.int64)
    d = wl.moe_dispatch(0, k=k, tokens=200, top_k=2, rows=rows)
    off = d["offsets"]
    m_total = int(off[-1])
    cols = k
    q = torch.full((m_total, cols), 0x7F, dtype=torch.uint8, device="cuda")          # E4M3 NaN
    s = torch.full((cols // 128, m_total), float("nan"), dtype=torch.float32, device="cuda")
    fq.fp8_quantize_act_scatter(dev_bf16(d["x"]), torch.from_numpy(d["dst_rows"]).cuda(), m_total,
                                q=q, scale=s)
    w = wl.weight(0, "grouped_fprop", 1, len(rows), n, k)
    b_q = np.empty((len(rows), n, k), np.uint8)
    b_s = np.empty((len(rows), n // 128, k // 128), np.float32)
    for e in range(len(rows)):
        b_q[e], b_s[e] = oracle.quant_weight_128x128(w[e])
    c = fq.fp8_grouped_gemm(torch.from_numpy(off.astype(np.int32)).cuda(),
                            torch.from_numpy(rows.astype(np.int32)).cuda(), q, s,
                            dev_codes(b_q), dev_f32(b_s), torch.bfloat16)
    torch.cuda.synchronize()
    got = host_out(c)
    a_q, a_s, written = oracle.quant_act_scatter(d["x"], d["dst_rows"], m_total)
    ref = oracle.grouped_gemm(off, rows, a_q, a_s, b_q, b_s)
    for e in range(len(rows)):
        r0, r, end = int(off[e]), int(rows[e]), int(off[e + 1])
        assert written[r0:r0 + r].all() and not written[r0 + r:end].any()
        assert np.all(got[r0 + r:end] == 0), "expert %d padding rows not zero" % e
        if r:
            assert_gemm_close(got[r0:r0 + r], ref[r0:r0 + r], "expert %d" % e)


def test_scatter_empty_is_noop():
    x = torch.empty((0, 256), dtype=torch.bfloat16, device="cuda")
    d = torch.empty((0, 8), dtype=torch.int32, device="cuda")
    q, s = fq.fp8_quantize_act_scatter(x, d, 0)
    assert q.shape == (0, 256) and s.shape == (2, 0)
