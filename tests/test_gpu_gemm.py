"""GPU parity of the block-scaled FP8 GEMM (Fprop, Dgrad, Wgrad, grouped MoE).

Both sides consume the same FP8 operands: the oracle quantizes the seeded
bf16 inputs, the codes and scales are uploaded unchanged, and the GPU GEMM is
compared with the oracle's unrounded float64 GEMM of the dequantized
operands. Pass criteria: normwise error <= 2e-3 and every element within
1e-2 * (|ref| + rms(ref)), with rms over the whole compared output (for the
grouped GEMM, all real rows of all experts). Every case, the full-size
configs included, compares every element of the output; outputs start as
NaN, so a tile the kernel leaves unwritten fails. An exact case (integer
codes, power-of-two scales) must be bit-exact in FP32. End-to-end cases run
the GPU quantizers too.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import fine_grained_fp8_quantize_amd as fq
import oracle
import workloads as wl
from gpu_util import (assert_bits_equal, assert_gemm_close, assert_grouped_close, cached, dev_bf16,
                      dev_codes, dev_f32, host_codes, host_f32, host_out, nan_out)

pytestmark = pytest.mark.gpu

OUT = {"bf16": torch.bfloat16, "f32": torch.float32}


def _gpu_gemm(a_q, a_s, b_q, b_s, kind, out):
    c = nan_out((a_q.shape[0], b_q.shape[0]), OUT[out])
    fq.fp8_gemm(dev_codes(a_q), dev_f32(a_s), dev_codes(b_q), dev_f32(b_s), kind, OUT[out], out=c)
    torch.cuda.synchronize()
    return host_out(c)


def _check_full(a_q, a_s, b_q, b_s, kind, out, what):
    got = _gpu_gemm(a_q, a_s, b_q, b_s, kind, out)
    ref = oracle.gemm(a_q, a_s, b_q, b_s, kind)
    return assert_gemm_close(got, ref, what)


# ------------------------------------------------------------ config shapes

@pytest.mark.parametrize("out", ["bf16", "f32"])
def test_tiny_fprop_all_elements(out):
    d = wl.tiny_fprop()
    a_q, a_s = oracle.quant_act_1x128(d["x"])
    b_q, b_s = oracle.quant_weight_128x128(d["w"])
    _check_full(a_q, a_s, b_q, b_s, "block", out, "tiny fprop " + out)


def test_dense_fprop_full_size():
    d = wl.dense_fprop()
    a_q, a_s = oracle.quant_act_1x128(d["x"])
    b_q, b_s = oracle.quant_weight_128x128(d["w"])
    e = _check_full(a_q, a_s, b_q, b_s, "block", "bf16", "dense fprop")
    print("dense fprop errors", e)


def test_dgrad_full_size():
    d = wl.dgrad()
    a_q, a_s = oracle.quant_act_1x128(d["dy"])               # [4096][2048]
    w_q, w_s = oracle.quant_weight_128x128(d["w"])            # [2048][7168]
    b_q = np.ascontiguousarray(w_q.T)                         # W^T codes [7168][2048]
    b_s = np.ascontiguousarray(w_s.T)                         # [56][16]
    e = _check_full(a_q, a_s, b_q, b_s, "block", "bf16", "dgrad")
    print("dgrad errors", e)


def test_wgrad_full_size():
    d = wl.wgrad()
    a_q, a_s = oracle.quant_act_128x1(d["dy"])                # dY^T [2048][8192], [64][2048]
    b_q, b_s = oracle.quant_act_128x1(d["x"])                 # X^T [7168][8192], [64][7168]
    e = _check_full(a_q, a_s, b_q, b_s, "row", "f32", "wgrad")
    print("wgrad errors", e)


# ------------------------------------------------------------ ragged / edge

@pytest.mark.parametrize("m,n,k", [(1, 128, 128), (17, 384, 384), (300, 256, 256), (257, 640, 640),
                                   (513, 128, 1024), (4000, 3968, 256)])
@pytest.mark.parametrize("out", ["bf16", "f32"])
def test_block_scaled_ragged(m, n, k, out):
    x = wl.activation(2, "tiny_fprop", 30, m, k, 100.0)
    w = wl.weight(2, "tiny_fprop", 31, n, k)
    a_q, a_s = oracle.quant_act_1x128(x)
    b_q, b_s = oracle.quant_weight_128x128(w)
    _check_full(a_q, a_s, b_q, b_s, "block", out, "block m=%d n=%d k=%d %s" % (m, n, k, out))


@pytest.mark.parametrize("m,n,tokens", [(1, 8, 128), (200, 72, 256), (130, 264, 384), (256, 512, 512),
                                        (4000, 3992, 256)])
@pytest.mark.parametrize("out", ["bf16", "f32"])
def test_row_scaled_ragged(m, n, tokens, out):
    dy = wl.activation(2, "wgrad", 32, tokens, m, None)
    x = wl.activation(2, "wgrad", 33, tokens, n, 50.0)
    a_q, a_s = oracle.quant_act_128x1(dy)
    b_q, b_s = oracle.quant_act_128x1(x)
    _check_full(a_q, a_s, b_q, b_s, "row", out, "row m=%d n=%d k=%d %s" % (m, n, tokens, out))


@pytest.mark.parametrize("kind", ["block", "row"])
def test_padded_leading_dims_and_scale_strides(kind):
    """Operands, scales and output as padded views (lda, ldb > k; ld_as > m;
    ld_bs past the scale row; ldc > n): the result matches the oracle and
    nothing outside the output window is written."""
    m, n, k = 200, 256, 384
    if kind == "block":
        a_q, a_s = oracle.quant_act_1x128(wl.activation(4, "tiny_fprop", 96, m, k, 50.0))
        b_q, b_s = oracle.quant_weight_128x128(wl.weight(4, "tiny_fprop", 97, n, k))
    else:
        a_q, a_s = oracle.quant_act_128x1(wl.activation(4, "wgrad", 96, k, m + 56, None))
        b_q, b_s = oracle.quant_act_128x1(wl.activation(4, "wgrad", 97, k, n, 50.0))
        a_q, a_s = a_q[:m], a_s[:, :m]   # rows 0..m-1 of the transposed operand
    ap = torch.zeros((m, k + 32), dtype=torch.uint8, device="cuda")
    bp = torch.zeros((n, k + 64), dtype=torch.uint8, device="cuda")
    ap[:, :k] = dev_codes(np.ascontiguousarray(a_q)).view(torch.uint8)
    bp[:, :k] = dev_codes(b_q).view(torch.uint8)
    asp = torch.full((a_s.shape[0], m + 24), 7.0, device="cuda")
    asp[:, :m] = dev_f32(np.ascontiguousarray(a_s))
    bsp = torch.full((b_s.shape[0], b_s.shape[1] + 5), 7.0, device="cuda")
    bsp[:, :b_s.shape[1]] = dev_f32(b_s)
    c = torch.full((m, n + 8), float("nan"), dtype=torch.bfloat16, device="cuda")
    fq.fp8_gemm(ap[:, :k], asp[:, :m], bp[:, :k], bsp[:, :b_s.shape[1]], kind, torch.bfloat16, out=c[:, :n])
    torch.cuda.synchronize()
    got = host_out(c)
    assert np.all(np.isnan(got[:, n:])), "columns past n written"
    assert_gemm_close(got[:, :n], oracle.gemm(np.ascontiguousarray(a_q), np.ascontiguousarray(a_s), b_q, b_s, kind),
                      "padded %s" % kind)


def test_operand_pitch_at_the_limit():
    """lda = ldb = FP8Q_MAX_GEMM_LD (2^23 - 128 bytes), the largest pitch the
    host accepts: a tile's last row then sits 255 pitches (just under 2^31
    bytes) past the tile origin, the most its 31-bit lane offsets reach. Two
    m-tiles (the second ragged) over 2.5 GB and 2.1 GB operand buffers."""
    ld = 8388480
    m, n, k = 296, 256, 256
    a_q, a_s = oracle.quant_act_1x128(wl.activation(6, "tiny_fprop", 98, m, k, 50.0))
    b_q, b_s = oracle.quant_weight_128x128(wl.weight(6, "tiny_fprop", 99, n, k))
    ap = torch.zeros((m, ld), dtype=torch.uint8, device="cuda")
    bp = torch.zeros((n, ld), dtype=torch.uint8, device="cuda")
    ap[:, :k] = dev_codes(a_q).view(torch.uint8)
    bp[:, :k] = dev_codes(b_q).view(torch.uint8)
    c = nan_out((m, n), torch.bfloat16)
    fq.fp8_gemm(ap[:, :k], dev_f32(a_s), bp[:, :k], dev_f32(b_s), "block", torch.bfloat16, out=c)
    torch.cuda.synchronize()
    del ap, bp
    assert_gemm_close(host_out(c), oracle.gemm(a_q, a_s, b_q, b_s, "block"), "pitch at the limit")


def test_scale_pitches_at_the_limit():
    """The A scales' and the 128x128 B block scales' row pitches at the
    largest values the host accepts for 2 rows (a span just under
    FP8Q_MAX_SCALE_SPAN = 2^29 floats): the second n-block's scales sit
    almost 1 GiB past the first, the most a lane offset of the block-scale
    copy reaches. Two 2 GB scale buffers."""
    ld = (1 << 28) - 16
    m, n, k = 256, 256, 256
    a_q, a_s = oracle.quant_act_1x128(wl.activation(6, "tiny_fprop", 100, m, k, 50.0))
    b_q, b_s = oracle.quant_weight_128x128(wl.weight(6, "tiny_fprop", 101, n, k))
    asp = torch.zeros((k // 128, ld), dtype=torch.float32, device="cuda")
    bsp = torch.zeros((n // 128, ld), dtype=torch.float32, device="cuda")
    asp[:, :m] = dev_f32(a_s)
    bsp[:, :k // 128] = dev_f32(b_s)
    c = nan_out((m, n), torch.bfloat16)
    fq.fp8_gemm(dev_codes(a_q), asp[:, :m], dev_codes(b_q), bsp[:, :k // 128], "block", torch.bfloat16, out=c)
    torch.cuda.synchronize()
    del asp, bsp
    assert_gemm_close(host_out(c), oracle.gemm(a_q, a_s, b_q, b_s, "block"), "scale pitches at the limit")


def test_k_zero_writes_zeros():
    """K = 0: the product is the zero matrix; every element of the window is
    written and nothing is read from the (unused) operands."""
    lib = fq._load()
    a = torch.zeros(16, dtype=torch.uint8, device="cuda")      # valid, never read
    b = torch.zeros(16, dtype=torch.uint8, device="cuda")
    out = torch.full((40, 136), 3.0, dtype=torch.float32, device="cuda")
    st = lib.fp8_gemm(40, 130, 0, a.data_ptr(), 16, None, 40, b.data_ptr(), 16, None, 1, 0,
                      out.data_ptr(), 136, 1, None)
    assert st == 0
    torch.cuda.synchronize()
    assert torch.all(out[:, :130] == 0)
    assert torch.all(out[:, 130:] == 3.0)


def test_exact_power_of_two_case():
    """Integer codes (|q| <= 16) and scales in {1, 2}: every partial sum is an
    integer below 2^24, so the FP32 result is exact and must equal the oracle
    bit for bit; the bf16 output must be its nearest-even rounding."""
    rng = np.random.default_rng(40)
    m, n, k = 300, 384, 512
    ints = list(range(17))
    code = {v: oracle.e4m3_encode(float(v)) for v in ints}
    va = rng.integers(-16, 17, (m, k))
    vb = rng.integers(-16, 17, (n, k))
    enc = np.vectorize(lambda t: code[abs(int(t))] | (0x80 if t < 0 else 0))
    a_q = enc(va).astype(np.uint8)
    b_q = enc(vb).astype(np.uint8)
    a_s = rng.choice([1.0, 2.0], (k // 128, m)).astype(np.float32)
    b_s = rng.choice([1.0, 2.0], (n // 128, k // 128)).astype(np.float32)
    ref = oracle.gemm(a_q, a_s, b_q, b_s, "block")
    got32 = _gpu_gemm(a_q, a_s, b_q, b_s, "block", "f32")
    assert_bits_equal(got32.astype(np.float32), ref.astype(np.float32), "exact fp32")
    assert np.array_equal(got32, ref)
    got16 = _gpu_gemm(a_q, a_s, b_q, b_s, "block", "bf16")
    assert np.array_equal(got16, oracle.bf16_round(ref))
    # the row-scaled form on the same integers
    a_r = rng.choice([1.0, 2.0], (k // 128, m)).astype(np.float32)
    b_r = rng.choice([1.0, 2.0], (k // 128, n)).astype(np.float32)
    ref_r = oracle.gemm(a_q, a_r, b_q, b_r, "row")
    got_r = _gpu_gemm(a_q, a_r, b_q, b_r, "row", "f32")
    assert np.array_equal(got_r, ref_r)


# ------------------------------------------------------------------ grouped

def _moe_expert_weights(n, k, rows, seed=0):
    """Oracle quantization of the grouped config's expert weights (cached:
    the 32 MoE experts take seconds on the host)."""
    def make():
        g = wl.grouped_fprop(seed, n=n, k=k, experts=len(rows), rows=np.asarray(rows, dtype=np.int64))
        E = len(rows)
        b_q = np.empty((E, n, k), np.uint8)
        b_s = np.empty((E, n // 128, k // 128), np.float32)
        for e in range(E):
            b_q[e], b_s[e] = oracle.quant_weight_128x128(g["w"][e])
        return g, b_q, b_s
    return cached(("moe_w", n, k, tuple(int(r) for r in rows), seed), make)


def _grouped_case(rows, n, k, seed=0, group_rows=True, out="bf16", pad_extra=None, workspace=None,
                  return_out=False):
    rows = np.asarray(rows, dtype=np.int64)
    key = (tuple(int(r) for r in rows), n, k, seed, group_rows,
           None if pad_extra is None else tuple(int(p) for p in pad_extra))
    g, b_q, b_s = _moe_expert_weights(n, k, rows, seed)
    offsets = g["offsets"].copy()
    if pad_extra is not None:   # enlarge some segments beyond the 128-padding
        seg = np.diff(offsets) + np.asarray(pad_extra, dtype=np.int64)
        offsets = np.concatenate([[0], np.cumsum(seg)])
        x = np.zeros((int(offsets[-1]), k), np.uint16)
        for e in range(len(rows)):
            x[offsets[e]:offsets[e] + rows[e]] = g["x"][g["offsets"][e]:g["offsets"][e] + rows[e]]
    else:
        x = g["x"]
    a_q, a_s = cached(("grouped_a",) + key, lambda: oracle.quant_act_1x128(x))
    off_d = torch.from_numpy(offsets.astype(np.int32)).cuda()
    rows_d = torch.from_numpy(rows.astype(np.int32)).cuda() if group_rows else None
    c = nan_out((a_q.shape[0], n), OUT[out])
    fq.fp8_grouped_gemm(off_d, rows_d, dev_codes(a_q), dev_f32(a_s), dev_codes(b_q), dev_f32(b_s), OUT[out],
                        out=c, workspace=workspace)
    torch.cuda.synchronize()
    got = host_out(c)
    real = rows if group_rows else np.diff(offsets)
    ref = cached(("grouped_ref",) + key, lambda: oracle.grouped_gemm(offsets, real, a_q, a_s, b_q, b_s))
    e = assert_grouped_close(got, ref, offsets, real, "grouped %d experts n=%d k=%d" % (len(rows), n, k))
    return (e, got) if return_out else e


def test_grouped_edge_row_counts():
    _grouped_case([0, 1, 127, 128, 129, 255, 256, 257, 3], n=256, k=384)


def test_grouped_all_rows_real_and_f32():
    _grouped_case([128, 256, 384], n=384, k=256, group_rows=False, out="f32")


def test_grouped_wide_padding_segments():
    # segments larger than the 128-rounding: real rows, then >= 128 padding rows
    _grouped_case([5, 0, 300], n=256, k=256, pad_extra=[256, 128, 128])


def test_grouped_more_experts_than_a_wave():
    # 70 experts: the tile scan takes them in chunks of 64
    rows = np.random.default_rng(7).integers(0, 300, 70)
    rows[[3, 64, 69]] = 0
    _grouped_case(rows, n=256, k=256)


@pytest.mark.parametrize("out", ["bf16", "f32"])
def test_grouped_split_last_round(out):
    # 7 m-tiles x 2 n-tiles = 14 tiles, one partial round: each tile is cut
    # into 4 K pieces of 4 or 5 slabs (18 slabs) and summed by the fix-up
    # kernel; N = 384 leaves the second n-tile half outside C, and the
    # segments hold padding rows and an empty expert
    _grouped_case([300, 5, 0, 128, 257, 40], n=384, k=18 * 128, out=out)


def test_grouped_split_last_round_wide_padding_and_all_real():
    # 5 m-tiles in one partial round, split into 2 K pieces (8 slabs): one
    # tail tile holds padding only (its pieces do no MFMA work and the fix-up
    # writes zeros), one expert is empty; then every row real, fp32 out
    _grouped_case([5, 0, 300], n=256, k=8 * 128, pad_extra=[256, 128, 128])
    _grouped_case([128, 256, 384], n=512, k=8 * 128, group_rows=False, out="f32")


def test_grouped_operand_pitch_at_the_limit():
    """The grouped kernel (which recomputes its copy offsets every step) at
    the largest operand pitch the host accepts: lda = ldb = 2^23 - 128 bytes,
    two experts (one a full 256-row tile, one ragged), 3.2 GB of activation
    rows and 4.3 GB of expert weights."""
    ld = 8388480
    rows = np.array([100, 256])
    n, k = 256, 256
    offsets = wl.pad_offsets(rows)
    m_total = int(offsets[-1])
    x = wl.activation(6, "grouped_fprop", 102, m_total, k, 50.0)
    a_q, a_s = oracle.quant_act_1x128(x)
    w = wl.weight(6, "grouped_fprop", 103, 2, n, k)
    b_q = np.stack([oracle.quant_weight_128x128(w[e])[0] for e in range(2)])
    b_s = np.stack([oracle.quant_weight_128x128(w[e])[1] for e in range(2)])
    ap = torch.zeros((m_total, ld), dtype=torch.uint8, device="cuda")
    bp = torch.zeros((2, n, ld), dtype=torch.uint8, device="cuda")
    ap[:, :k] = dev_codes(a_q).view(torch.uint8)
    bp[:, :, :k] = dev_codes(b_q).view(torch.uint8)
    c = nan_out((m_total, n), torch.bfloat16)
    fq.fp8_grouped_gemm(torch.from_numpy(offsets.astype(np.int32)).cuda(),
                        torch.from_numpy(rows.astype(np.int32)).cuda(),
                        ap[:, :k], dev_f32(a_s), bp[:, :, :k], dev_f32(b_s), torch.bfloat16, out=c)
    torch.cuda.synchronize()
    del ap, bp
    ref = oracle.grouped_gemm(offsets, rows, a_q, a_s, b_q, b_s)
    assert_grouped_close(host_out(c), ref, offsets, rows, "grouped pitch at the limit")


def test_grouped_moe_config_full():
    """The MoE config: 32 experts, Zipf(1.1) routing of 8192 tokens, N=4096,
    K=7168; every real row of every expert compared."""
    e = _grouped_case(wl.moe_rows(0), n=4096, k=7168)
    print("grouped MoE errors", e)


def test_grouped_moe_config_workspace_sizes():
    """The MoE config's 816 tiles leave a last round of 48: with the full
    workspace each of them is cut into 5 K pieces, with room for 100 partial
    tiles into 2, and with no workspace not at all. Every result meets the bar
    against the oracle, and a second call with the full workspace gives the
    same bits (the pieces are added in a fixed order)."""
    full = torch.empty(fq.GROUPED_WORKSPACE_BYTES, dtype=torch.uint8, device="cuda")
    part = torch.empty(256 * 32 + 100 * 256 * 256 * 4, dtype=torch.uint8, device="cuda")
    none = torch.empty(0, dtype=torch.uint8, device="cuda")
    outs = {}
    for name, ws in (("full", full), ("100 partials", part), ("none", none), ("full again", full)):
        e, outs[name] = _grouped_case(wl.moe_rows(0), n=4096, k=7168, workspace=ws, return_out=True)
        print("workspace", name, e)
    assert np.array_equal(outs["full"], outs["full again"])


# --------------------------------------------------------------- end to end

@pytest.mark.parametrize("name", ["tiny_fprop", "dense_fprop"])
def test_end_to_end_fprop(name):
    """GPU quantizers + GPU GEMM against oracle quantizers + oracle GEMM."""
    d = wl.tiny_fprop() if name == "tiny_fprop" else wl.dense_fprop()
    xq, xs = fq.fp8_quantize_act(dev_bf16(d["x"]))
    wq, ws = fq.fp8_quantize_weight(dev_bf16(d["w"]))
    c = fq.fp8_gemm(xq, xs, wq, ws, "block", torch.bfloat16)
    torch.cuda.synchronize()
    got = host_out(c)
    a_q, a_s = oracle.quant_act_1x128(d["x"])
    b_q, b_s = oracle.quant_weight_128x128(d["w"])
    assert_bits_equal(host_codes(xq), a_q, name + " activation codes")
    assert_bits_equal(host_codes(wq), b_q, name + " weight codes")
    assert_gemm_close(got, oracle.gemm(a_q, a_s, b_q, b_s, "block"), name + " end to end")


def test_end_to_end_dgrad_uses_transposed_copy():
    d = wl.dgrad(m=512)
    dq, ds = fq.fp8_quantize_act(dev_bf16(d["dy"]))
    _, _, wqt, wst = fq.fp8_quantize_weight(dev_bf16(d["w"]), transposed=True)
    c = fq.fp8_gemm(dq, ds, wqt, wst, "block", torch.bfloat16)
    torch.cuda.synchronize()
    a_q, a_s = oracle.quant_act_1x128(d["dy"])
    w_q, w_s = oracle.quant_weight_128x128(d["w"])
    ref = oracle.gemm(a_q, a_s, np.ascontiguousarray(w_q.T), np.ascontiguousarray(w_s.T), "block")
    assert_gemm_close(host_out(c), ref, "dgrad end to end")


def test_end_to_end_wgrad():
    d = wl.wgrad(tokens=1024, n_out=384, k_in=640)
    aq, as_ = fq.fp8_quantize_act(dev_bf16(d["dy"]), "128x1")
    bq, bs = fq.fp8_quantize_act(dev_bf16(d["x"]), "128x1")
    c = fq.fp8_gemm(aq, as_, bq, bs, "row", torch.float32)
    torch.cuda.synchronize()
    a_q, a_s = oracle.quant_act_128x1(d["dy"])
    b_q, b_s = oracle.quant_act_128x1(d["x"])
    assert_bits_equal(host_codes(aq), a_q, "wgrad dY^T codes")
    assert_bits_equal(host_f32(bs), b_s, "wgrad X^T scales")
    assert_gemm_close(host_out(c), oracle.gemm(a_q, a_s, b_q, b_s, "row"), "wgrad end to end")


# ------------------------------------------------------------ grouped Dgrad

def _grouped_dgrad_case(rows, n_out, k_in, one_launch=False):
    """dX_e = dY_e W_e for every expert: the grouped GEMM with each expert's
    transposed weight copy (W_e^T codes [k_in][n_out], transposed block
    scales) as B; dY in the expert-sorted layout, quantized 1x128.
    one_launch: all experts' W quantized as one [E*n_out][k_in] matrix; the
    transposed copy [k_in][E*n_out] is read in place, expert e at column
    e*n_out (interleaved rows: stride_b = n_out, ldb = E*n_out)."""
    rows = np.asarray(rows, dtype=np.int64)
    off = wl.pad_offsets(rows)
    m_total = int(off[-1])
    E = len(rows)
    dy = np.zeros((m_total, n_out), np.uint16)
    real = wl.grad_rowscaled(0, "grouped_fprop", 80, int(rows.sum()), n_out)
    src = 0
    for e in range(E):
        dy[off[e]:off[e] + rows[e]] = real[src:src + rows[e]]
        src += int(rows[e])
    w = wl.weight(0, "grouped_fprop", 81, E, n_out, k_in)
    if one_launch:
        flat_q = torch.empty((k_in, E * n_out), dtype=torch.uint8, device="cuda")
        flat_s = torch.empty((k_in // 128, E * n_out // 128), dtype=torch.float32, device="cuda")
        fq.fp8_quantize_weight(dev_bf16(w.reshape(E * n_out, k_in)), transposed=True, q_t=flat_q,
                               scale_t=flat_s)
        wt_q = flat_q.view(k_in, E, n_out).permute(1, 0, 2)            # strides (n_out, E*n_out, 1)
        wt_s = flat_s.view(k_in // 128, E, n_out // 128).permute(1, 0, 2)
    else:
        wt_q = torch.empty((E, k_in, n_out), dtype=torch.uint8, device="cuda")
        wt_s = torch.empty((E, k_in // 128, n_out // 128), dtype=torch.float32, device="cuda")
        for e in range(E):   # one launch per expert: codes, scales and the transposed copy
            fq.fp8_quantize_weight(dev_bf16(w[e]), transposed=True, q_t=wt_q[e], scale_t=wt_s[e])
    dq, ds = fq.fp8_quantize_act(dev_bf16(dy))
    c = nan_out((m_total, k_in), torch.bfloat16)
    fq.fp8_grouped_gemm(torch.from_numpy(off.astype(np.int32)).cuda(),
                        torch.from_numpy(rows.astype(np.int32)).cuda(), dq, ds, wt_q, wt_s,
                        torch.bfloat16, out=c)
    torch.cuda.synchronize()
    got = host_out(c)
    a_q, a_s = oracle.quant_act_1x128(dy)
    bt_q = np.empty((E, k_in, n_out), np.uint8)
    bt_s = np.empty((E, k_in // 128, n_out // 128), np.float32)
    for e in range(E):   # every expert's transposed copy, bit for bit
        w_q, w_s = oracle.quant_weight_128x128(w[e])
        bt_q[e], bt_s[e] = w_q.T, w_s.T
        assert_bits_equal(host_codes(wt_q[e].contiguous()), bt_q[e], "expert %d transposed codes" % e)
        assert_bits_equal(host_f32(wt_s[e].contiguous()), bt_s[e], "expert %d transposed scales" % e)
    ref = oracle.grouped_gemm(off, rows, a_q, a_s, bt_q, bt_s)
    return assert_grouped_close(got, ref, off, rows, "grouped dgrad %d experts" % E)


def test_grouped_dgrad_edge_rows():
    _grouped_dgrad_case([0, 1, 129, 256, 3], n_out=256, k_in=384)


def test_grouped_dgrad_edge_rows_one_weight_launch():
    _grouped_dgrad_case([0, 1, 129, 256, 3], n_out=256, k_in=384, one_launch=True)


def test_grouped_dgrad_moe_config_one_weight_launch_full():
    """The MoE Dgrad with all 32 experts' weights quantized in one launch and
    their transposed copies read in place (interleaved rows); every real row
    compared."""
    _grouped_dgrad_case(wl.moe_rows(0), n_out=4096, k_in=7168, one_launch=True)


def test_grouped_dgrad_moe_config_full():
    """MoE up-projection Dgrad: 32 experts, dY [rows][4096] -> dX [rows][7168];
    every real row compared."""
    e = _grouped_dgrad_case(wl.moe_rows(0), n_out=4096, k_in=7168)
    print("grouped dgrad errors", e)


def test_grouped_padded_views_and_strides():
    """Grouped Fprop with every operand a padded view: lda > k, ldb > k with
    expert stride > n * ldb, block scales with ld_bs > k/128 and a padded
    expert stride, ldc > n. Matches the oracle; nothing outside the output
    window is written."""
    rows = np.array([130, 0, 77, 256], dtype=np.int64)
    n, k = 256, 384
    g = wl.grouped_fprop(5, n=n, k=k, experts=len(rows), rows=rows)
    offsets = g["offsets"]
    a_q, a_s = oracle.quant_act_1x128(g["x"])
    E, m_total = len(rows), a_q.shape[0]
    b_q = np.empty((E, n, k), np.uint8)
    b_s = np.empty((E, n // 128, k // 128), np.float32)
    for e in range(E):
        b_q[e], b_s[e] = oracle.quant_weight_128x128(g["w"][e])
    ap = torch.zeros((m_total, k + 48), dtype=torch.uint8, device="cuda")
    ap[:, :k] = dev_codes(a_q)
    asp = torch.full((k // 128, m_total + 40), 7.0, device="cuda")
    asp[:, :m_total] = dev_f32(a_s)
    bp = torch.zeros((E, n + 16, k + 64), dtype=torch.uint8, device="cuda")
    bp[:, :n, :k] = dev_codes(b_q)
    bsp = torch.full((E, n // 128 + 1, k // 128 + 3), 7.0, device="cuda")
    bsp[:, :n // 128, :k // 128] = dev_f32(b_s)
    c = torch.full((m_total, n + 24), float("nan"), dtype=torch.bfloat16, device="cuda")
    off_d = torch.from_numpy(offsets.astype(np.int32)).cuda()
    rows_d = torch.from_numpy(rows.astype(np.int32)).cuda()
    fq.fp8_grouped_gemm(off_d, rows_d, ap[:, :k], asp[:, :m_total], bp[:, :n, :k], bsp[:, :n // 128, :k // 128],
                        torch.bfloat16, out=c[:, :n])
    torch.cuda.synchronize()
    got = host_out(c)
    assert np.all(np.isnan(got[:, n:])), "columns past n written"
    ref = oracle.grouped_gemm(offsets, rows, a_q, a_s, b_q, b_s)
    real = np.concatenate([np.arange(offsets[e], offsets[e] + rows[e]) for e in range(E)]).astype(np.int64)
    assert_gemm_close(got[real, :n], ref[real], "grouped padded views")
    pad = np.setdiff1d(np.arange(m_total), real)
    assert np.all(got[pad, :n] == 0), "padding rows not zero"


# ------------------------------------------------------------ looping grid

@pytest.mark.parametrize("m,n,k,out", [
    (4096, 7168, 256, "bf16"),    # 2 rounds of 224-wide tiles, the minimum 2 slabs
    (4096, 7168, 256, "f32"),
    (5120, 7168, 512, "bf16"),    # 640 tiles: some blocks run 3 tiles, others 2
    (6144, 7168, 256, "f32"),     # 3 rounds
    (8192, 3584, 256, "bf16"),    # N = 16 x 224
    (4096, 7168, 384, "bf16"),    # odd slab count: one tile per block instead
])
def test_block_scaled_several_rounds(m, n, k, out):
    """Shapes whose whole 224-wide tiles take several rounds of the CUs run
    one looping block per CU, which copies each next tile's first slab under
    the tile before; every element of every tile against the oracle."""
    x = wl.activation(5, "dgrad", 40, m, k, 50.0)
    w = wl.weight(5, "dgrad", 41, n, k)
    a_q, a_s = oracle.quant_act_1x128(x)
    b_q, b_s = oracle.quant_weight_128x128(w)
    _check_full(a_q, a_s, b_q, b_s, "block", out, "rounds block m=%d n=%d k=%d %s" % (m, n, k, out))


@pytest.mark.parametrize("out", ["f32", "bf16"])
def test_row_scaled_several_rounds(out):
    m, n, tokens = 4096, 7168, 256
    dy = wl.activation(5, "wgrad", 42, tokens, m, None)
    x = wl.activation(5, "wgrad", 43, tokens, n, 50.0)
    a_q, a_s = oracle.quant_act_128x1(dy)
    b_q, b_s = oracle.quant_act_128x1(x)
    _check_full(a_q, a_s, b_q, b_s, "row", out, "rounds row %s" % out)
