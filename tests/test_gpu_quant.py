"""GPU parity of the quantization kernels: FP8 codes and FP32 scales must be
bit-identical to the CPU oracle on the same seeded inputs.

Covers every config's quantized operands at full size, ragged row counts,
edge tiles (all-zero, signed zeros, bf16 subnormals, bf16 max, subnormal
fp32 scales, single values, ties), padded leading dimensions, and the
exhaustive sweep over every bf16 (x, amax) pair (both signs).
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import fine_grained_fp8_quantize_amd as fq
import oracle
import workloads as wl
from gpu_util import assert_bits_equal, dev_bf16, host_codes, host_f32

pytestmark = pytest.mark.gpu


def _gpu_act(bits: np.ndarray, tiling: str = "1x128"):
    x = dev_bf16(bits)
    q, s = fq.fp8_quantize_act(x, tiling)
    torch.cuda.synchronize()
    return host_codes(q), host_f32(s)


def _check_act_1x128(bits: np.ndarray, what: str):
    q, s = _gpu_act(bits)
    q_ref, s_ref = oracle.quant_act_1x128(bits)
    assert_bits_equal(s, s_ref, what + " scales")
    assert_bits_equal(q, q_ref, what + " codes")


def _check_act_128x1(bits: np.ndarray, what: str):
    q, s = _gpu_act(bits, "128x1")
    q_ref, s_ref = oracle.quant_act_128x1(bits)
    assert_bits_equal(s, s_ref, what + " scales")
    assert_bits_equal(q, q_ref, what + " codes")


def _edge_rows(rng) -> np.ndarray:
    def bf(v):
        return wl.f32_to_bf16_bits(np.asarray(v, dtype=np.float32))
    rows = [bf(rng.standard_normal(128))]
    z = np.zeros(128, np.uint16)
    z[::3] = 0x8000
    rows.append(z)                                            # all +-0: s = 0
    r = bf(rng.standard_normal(128) * 1e-3)
    r[17] = bf([1000.0])[0]
    rows.append(r)                                            # one outlier
    sub = rng.integers(1, 0x80, 128).astype(np.uint16)
    sub[::2] |= 0x8000
    rows.append(sub)                                          # bf16 subnormals only
    big = bf(rng.standard_normal(128))
    big[5] = 0x7F7F
    rows.append(big)                                          # amax = bf16 max
    rows.append(bf(rng.standard_normal(128) * 1e-38))         # subnormal fp32 scale
    rows.append(bf(rng.standard_normal(128) * 1e-20))         # scale below 2^-60
    one = np.zeros(128, np.uint16)
    one[77] = bf([-3.0])[0]
    rows.append(one)                                          # single nonzero value
    ties = bf(np.full(128, 448.0 * 17 / 64))
    ties[0] = bf([448.0])[0]
    rows.append(ties)                                         # exact E4M3 ties
    neg = bf(-np.abs(rng.standard_normal(128)) * 1e-6)
    neg[3] = 0x8000
    rows.append(neg)                                          # negatives rounding to -0
    return np.stack(rows)


# ------------------------------------------------------------------ 1x128

@pytest.mark.parametrize("name", ["tiny_fprop", "dense_fprop", "dgrad", "grouped_fprop"])
def test_act_1x128_configs_full_size(name):
    if name == "tiny_fprop":
        bits = wl.tiny_fprop()["x"]
    elif name == "dense_fprop":
        bits = wl.dense_fprop()["x"]
    elif name == "dgrad":
        bits = wl.dgrad()["dy"]
    else:
        bits = wl.grouped_fprop(with_weights=False)["x"]
    _check_act_1x128(bits, name)


@pytest.mark.parametrize("rows", [1, 3, 15, 16, 17, 63, 129, 1000])
def test_act_1x128_ragged_rows(rows):
    bits = wl.activation(1, "tiny_fprop", 20, rows, 384, 100.0)
    _check_act_1x128(bits, "rows=%d" % rows)


@pytest.mark.parametrize("rows,cols", [(9, 128), (1000, 640), (8, 256)])
def test_act_1x128_slab_pairs(rows, cols):
    """A wave takes two slabs of 8 rows: one slab (its pair half empty), an odd
    slab count, and exactly one unit."""
    _check_act_1x128(wl.activation(1, "tiny_fprop", 23, rows, cols, 100.0), "rows=%d cols=%d" % (rows, cols))


def test_act_1x128_edge_tiles():
    rng = np.random.default_rng(11)
    e = _edge_rows(rng)
    # two slabs per row: edge tile in slab 0, a plain tile in slab 1, so every
    # 16-lane group also sees its neighbours' special cases
    bits = np.concatenate([e, wl.activation(1, "tiny_fprop", 21, e.shape[0], 128, None)], axis=1)
    _check_act_1x128(bits, "edge tiles")


def test_act_1x128_padded_leading_dimension():
    bits = wl.activation(1, "tiny_fprop", 22, 70, 512, 100.0)
    x_full = dev_bf16(np.concatenate([bits, np.zeros((70, 128), np.uint16)], axis=1))
    x = x_full[:, :384]
    q = torch.full((70, 400), 0x5A, dtype=torch.uint8, device="cuda")[:, :384]
    s = torch.full((3, 80), 7.0, dtype=torch.float32, device="cuda")[:, :70]
    fq.fp8_quantize_act(x, "1x128", q=q, scale=s)
    torch.cuda.synchronize()
    q_ref, s_ref = oracle.quant_act_1x128(bits[:, :384])
    assert_bits_equal(host_codes(q.contiguous()), q_ref, "padded ld codes")
    assert_bits_equal(host_f32(s.contiguous()), s_ref, "padded ld scales")
    # bytes outside the logical window are untouched
    assert torch.all(q.as_strided((70, 16), (400, 1), q.storage_offset() + 384) == 0x5A)


def test_exhaustive_x_amax_sweep():
    """Every bf16 amax A > 0 with every bf16 |x| <= A, both signs: A sits in
    slot 0 of a 1x128 tile and 127 x values fill the rest. GPU codes must
    equal the oracle's for all ~1.07e9 pairs."""
    amax_bits = np.arange(1, 0x7F80, dtype=np.int64)          # positive finite bf16
    counts = amax_bits + 1                                    # |x| bits 0..A
    chunk_edges = np.searchsorted(np.cumsum(counts), np.linspace(0, counts.sum(), 17)[1:-1])
    total_pairs = 0
    for sign in (0, 0x8000):
        for chunk in np.split(amax_bits, chunk_edges):
            if chunk.size == 0:
                continue
            c = chunk + 1
            tiles_per = (c + 126) // 127
            n_tiles = int(tiles_per.sum())
            tile_amax = np.repeat(chunk, tiles_per)
            # x bit pattern for slot 1..127 of tile t: 127*(t - first tile of its A) + slot - 1
            first = np.repeat(np.cumsum(tiles_per) - tiles_per, tiles_per)
            local = (np.arange(n_tiles) - first)[:, None] * 127 + np.arange(127)[None, :]
            xb = np.where(local <= tile_amax[:, None], local, 0).astype(np.uint16) | np.uint16(sign)
            tiles = np.empty((n_tiles, 128), np.uint16)
            tiles[:, 0] = tile_amax.astype(np.uint16)
            tiles[:, 1:] = xb
            total_pairs += int(c.sum())
            _check_act_1x128(tiles, "sweep sign=%#x A in [%#x, %#x]" % (sign, chunk[0], chunk[-1]))
    assert total_pairs == 2 * int(counts.sum())


# ------------------------------------------------------------------ 128x1

@pytest.mark.parametrize("which", ["dy", "x"])
def test_act_128x1_wgrad_full_size(which):
    d = wl.wgrad()
    _check_act_128x1(d[which], "wgrad " + which)


@pytest.mark.parametrize("cols", [8, 120, 200, 264])
def test_act_128x1_ragged_columns(cols):
    bits = wl.activation(1, "wgrad", 23, 384, cols, 50.0)
    _check_act_128x1(bits, "cols=%d" % cols)


def test_act_128x1_edge_tiles():
    rng = np.random.default_rng(12)
    e = _edge_rows(rng)                                       # [10][128]: one tile per row
    bits = np.ascontiguousarray(np.concatenate([e, e[::-1]], axis=0)[:16].T)  # [128][16]
    bits = np.concatenate([bits, bits[::-1]], axis=0)         # [256][16]
    _check_act_128x1(bits, "edge tiles 128x1")


# ---------------------------------------------------------------- 128x128

@pytest.mark.parametrize("name", ["tiny_fprop", "dense_fprop", "dgrad"])
def test_weight_configs_full_size(name):
    w = {"tiny_fprop": wl.tiny_fprop, "dense_fprop": wl.dense_fprop, "dgrad": wl.dgrad}[name]()["w"]
    q, s, qt, st = fq.fp8_quantize_weight(dev_bf16(w), transposed=True)
    torch.cuda.synchronize()
    q_ref, s_ref = oracle.quant_weight_128x128(w)
    assert_bits_equal(host_f32(s), s_ref, name + " weight scales")
    assert_bits_equal(host_codes(q), q_ref, name + " weight codes")
    assert_bits_equal(host_f32(st), np.ascontiguousarray(s_ref.T), name + " transposed scales")
    assert_bits_equal(host_codes(qt), np.ascontiguousarray(q_ref.T), name + " transposed codes")


def test_weight_grouped_experts_all():
    """All 32 expert weights quantized on the GPU as one [32*4096][7168]
    matrix (the bench launch); every expert compared in full with the oracle."""
    g = wl.grouped_fprop()
    w = g["w"]
    E, n, k = w.shape
    dw = dev_bf16(w.reshape(E * n, k))
    q, s = fq.fp8_quantize_weight(dw)   # experts stacked along n: blocks never straddle
    torch.cuda.synchronize()
    q = host_codes(q).reshape(E, n, k)
    s = host_f32(s).reshape(E, n // 128, k // 128)
    for e in range(E):
        q_ref, s_ref = oracle.quant_weight_128x128(w[e])
        assert_bits_equal(s[e], s_ref, "expert %d scales" % e)
        assert_bits_equal(q[e], q_ref, "expert %d codes" % e)


def test_weight_edge_blocks():
    rng = np.random.default_rng(13)
    w = wl.weight(1, "tiny_fprop", 24, 384, 256)
    w[0:128, 0:128] = 0                                   # all-zero block
    w[0:128:3, 0:128:5] = 0x8000                          # with signed zeros
    w[128:256, 128:256] = rng.integers(1, 0x80, (128, 128)).astype(np.uint16)  # subnormals
    w[256, 7] = 0x7F7F                                    # bf16 max
    w[300:384, 128:256] = wl.f32_to_bf16_bits(rng.standard_normal((84, 128)).astype(np.float32) * 1e-39)
    w[256:300, 128:256] = 0
    q, s, qt, st = fq.fp8_quantize_weight(dev_bf16(w), transposed=True)
    torch.cuda.synchronize()
    q_ref, s_ref = oracle.quant_weight_128x128(w)
    assert_bits_equal(host_f32(s), s_ref, "edge weight scales")
    assert_bits_equal(host_codes(q), q_ref, "edge weight codes")
    assert_bits_equal(host_codes(qt), np.ascontiguousarray(q_ref.T), "edge transposed codes")


@pytest.mark.parametrize("n,k", [(256, 128), (384, 640), (128, 1152)])
def test_weight_odd_block_columns(n, k):
    """An odd number of 128-column blocks (1, 5, 9): the last work unit of
    each block row holds one block instead of two."""
    w = wl.weight(3, "tiny_fprop", 60, n, k)
    w[0:128, k - 128:k] = 0                               # all-zero last block
    q, s, qt, st = fq.fp8_quantize_weight(dev_bf16(w), transposed=True)
    torch.cuda.synchronize()
    q_ref, s_ref = oracle.quant_weight_128x128(w)
    tag = "odd blocks %dx%d" % (n, k)
    assert_bits_equal(host_f32(s), s_ref, tag + " scales")
    assert_bits_equal(host_codes(q), q_ref, tag + " codes")
    assert_bits_equal(host_f32(st), np.ascontiguousarray(s_ref.T), tag + " transposed scales")
    assert_bits_equal(host_codes(qt), np.ascontiguousarray(q_ref.T), tag + " transposed codes")


@pytest.mark.parametrize("experts", [8, 16])
def test_weight_grouped_staged_transpose_odd_blocks(experts):
    """Enough blocks for the LDS-staged transposed copy (experts x 8 x 33
    blocks: 2112 in single-block units, 4224 in pairs of blocks), with an odd
    number of block columns per expert."""
    w = np.stack([wl.weight(3, "tiny_fprop", 70 + e, 1024, 4224) for e in range(experts)])
    w[1, 128:256, 4096:4224] = 0                          # all-zero last (unpaired) block
    _check_grouped_weights(w, "staged odd %d" % experts)


@pytest.mark.parametrize("n,k", [(256, 384), (128, 128), (384, 1152)])
def test_act_weight_pairs_odd_block_columns(n, k):
    """X + W in one launch without the transposed copy (weights in pairs of
    blocks) and an odd number of block columns."""
    x = wl.activation(3, "tiny_fprop", 80, 17, k, 100.0)
    w = wl.weight(3, "tiny_fprop", 81, n, k)
    _check_act_weight(x, w, "pairs odd %dx%d" % (n, k), transposed=False)


def test_empty_inputs_are_noops():
    x = torch.empty((0, 256), dtype=torch.bfloat16, device="cuda")
    q, s = fq.fp8_quantize_act(x)
    assert q.shape == (0, 256) and s.shape == (2, 0)
    w = torch.empty((0, 128), dtype=torch.bfloat16, device="cuda")
    q, s = fq.fp8_quantize_weight(w)
    assert q.shape == (0, 128)


# ------------------------------------------------ grouped weight quantization

def _check_grouped_weights(w, what, experts=None, pad=False):
    """fp8_quantize_weight_grouped of w[E][n][k] (transposed copies too):
    every checked expert equals the oracle's 128x128 quantization bit for bit.
    pad: every operand has padded leading dimensions and group strides."""
    E, n, k = w.shape
    if pad:
        wd = torch.zeros((E, n + 3, k + 8), dtype=torch.bfloat16, device="cuda")
        wd[:, :n, :k] = dev_bf16(w)
        wd = wd[:, :n, :k]
        bufs = [torch.full((E, n + 1, k + 16), 0x5A, dtype=torch.uint8, device="cuda"),
                torch.full((E, n // 128 + 1, k // 128 + 2), 7.0, device="cuda"),
                torch.full((E, k + 2, n + 32), 0x5A, dtype=torch.uint8, device="cuda"),
                torch.full((E, k // 128 + 1, n // 128 + 3), 7.0, device="cuda")]
        q, s = bufs[0][:, :n, :k], bufs[1][:, :n // 128, :k // 128]
        qt, st = bufs[2][:, :k, :n], bufs[3][:, :k // 128, :n // 128]
        fq.fp8_quantize_weight_grouped(wd, transposed=True, q=q, scale=s, q_t=qt, scale_t=st)
    else:
        q, s, qt, st = fq.fp8_quantize_weight_grouped(dev_bf16(w), transposed=True)
    torch.cuda.synchronize()
    for e in (range(E) if experts is None else experts):
        q_ref, s_ref = oracle.quant_weight_128x128(w[e])
        tag = "%s expert %d" % (what, e)
        assert_bits_equal(host_f32(s[e].contiguous()), s_ref, tag + " scales")
        assert_bits_equal(host_codes(q[e].contiguous()), q_ref, tag + " codes")
        assert_bits_equal(host_f32(st[e].contiguous()), np.ascontiguousarray(s_ref.T), tag + " transposed scales")
        assert_bits_equal(host_codes(qt[e].contiguous()), np.ascontiguousarray(q_ref.T), tag + " transposed codes")
    if pad:   # nothing outside the windows written
        assert torch.all(bufs[0][:, n:, :] == 0x5A) and torch.all(bufs[0][:, :, k:] == 0x5A)
        assert torch.all(bufs[2][:, k:, :] == 0x5A) and torch.all(bufs[2][:, :, n:] == 0x5A)
        assert torch.all(bufs[1][:, n // 128:, :] == 7.0) and torch.all(bufs[1][:, :, k // 128:] == 7.0)
        assert torch.all(bufs[3][:, k // 128:, :] == 7.0) and torch.all(bufs[3][:, :, n // 128:] == 7.0)


def test_weight_grouped_small_experts_edge_blocks():
    rng = np.random.default_rng(14)
    w = np.stack([wl.weight(1, "tiny_fprop", 40 + e, 256, 384) for e in range(5)])
    w[1, 0:128, 0:128] = 0                                                        # all-zero block
    w[2, 128:256, 128:256] = rng.integers(1, 0x80, (128, 128)).astype(np.uint16)  # subnormals
    w[3, 17, 300] = 0x7F7F                                                        # bf16 max
    w[4] = wl.f32_to_bf16_bits(wl.bf16_bits_to_f32(w[4]) * np.float32(1e-30))    # tiny scales
    _check_grouped_weights(w, "small experts")


def test_weight_grouped_padded_strides():
    w = np.stack([wl.weight(2, "tiny_fprop", 50 + e, 384, 256) for e in range(3)])
    _check_grouped_weights(w, "padded", pad=True)


def test_weight_grouped_moe_experts_all():
    """The 32 MoE expert weights [32][4096][7168] in one launch, with their
    transposed copies (the grouped Dgrad operand); every expert checked."""
    _check_grouped_weights(wl.grouped_fprop()["w"], "MoE")


# ------------------------------------ activation and weight in one launch

def _check_act_weight(x_bits, w_bits, what, transposed=True):
    """fp8_quantize_act_weight equals the oracle's 1x128 and 128x128
    quantizations (and the transposed copy) bit for bit."""
    out = fq.fp8_quantize_act_weight(dev_bf16(x_bits), dev_bf16(w_bits), transposed=transposed)
    torch.cuda.synchronize()
    q_ref, s_ref = oracle.quant_act_1x128(x_bits)
    assert_bits_equal(host_f32(out[1]), s_ref, what + " act scales")
    assert_bits_equal(host_codes(out[0]), q_ref, what + " act codes")
    wq_ref, ws_ref = oracle.quant_weight_128x128(w_bits)
    assert_bits_equal(host_f32(out[3]), ws_ref, what + " weight scales")
    assert_bits_equal(host_codes(out[2]), wq_ref, what + " weight codes")
    if transposed:
        assert_bits_equal(host_f32(out[5]), np.ascontiguousarray(ws_ref.T), what + " transposed scales")
        assert_bits_equal(host_codes(out[4]), np.ascontiguousarray(wq_ref.T), what + " transposed codes")


@pytest.mark.parametrize("rows", [1, 17, 129, 1000])
def test_act_weight_ragged_rows(rows):
    x = wl.activation(1, "tiny_fprop", 60, rows, 384, 100.0)
    w = wl.weight(1, "tiny_fprop", 61, 256, 384)
    _check_act_weight(x, w, "rows=%d" % rows, transposed=rows != 17)


def test_act_weight_edge_tiles_and_blocks():
    rng = np.random.default_rng(62)
    e = _edge_rows(rng)
    x = np.concatenate([e, wl.activation(1, "tiny_fprop", 63, e.shape[0], 128, None)], axis=1)
    w = wl.weight(1, "tiny_fprop", 64, 384, 256)
    w[0:128, 0:128] = 0
    w[128:256, 128:256] = rng.integers(1, 0x80, (128, 128)).astype(np.uint16)
    w[256, 7] = 0x7F7F
    _check_act_weight(x, w, "edge")


@pytest.mark.parametrize("name,transposed", [("tiny_fprop", True), ("dense_fprop", False), ("dense_fprop", True),
                                              ("dgrad", True)])
def test_act_weight_equals_separate_launches_full_size(name, transposed):
    """At the Linear layer's full size the one launch writes exactly what the
    two separate launches write (each of which the tests above pin to the
    oracle at full size). Both block orders: weight blocks first without
    the transposed copy, activation tiles first with it."""
    g = {"tiny_fprop": wl.tiny_fprop, "dense_fprop": wl.dense_fprop, "dgrad": wl.dgrad}[name]()
    x, w = dev_bf16(g["dy" if name == "dgrad" else "x"]), dev_bf16(g["w"])
    got = fq.fp8_quantize_act_weight(x, w, transposed=transposed)
    q, s = fq.fp8_quantize_act(x)
    ref = fq.fp8_quantize_weight(w, transposed=transposed)
    torch.cuda.synchronize()
    for a, b, tag in zip(got, (q, s) + tuple(ref), ("q", "scale", "wq", "wscale", "wq_t", "wscale_t")):
        assert torch.equal(a.view(torch.uint8) if a.dtype == torch.float8_e4m3fn else a.view(torch.int32),
                           b.view(torch.uint8) if b.dtype == torch.float8_e4m3fn else b.view(torch.int32)), tag


def test_act_weight_one_side_empty():
    x = wl.activation(1, "tiny_fprop", 65, 40, 256, 100.0)
    w = wl.weight(1, "tiny_fprop", 66, 128, 256)
    empty_x = torch.empty((0, 256), dtype=torch.bfloat16, device="cuda")
    empty_w = torch.empty((0, 256), dtype=torch.bfloat16, device="cuda")
    _, _, wq, ws = fq.fp8_quantize_act_weight(empty_x, dev_bf16(w))
    q, s, _, _ = fq.fp8_quantize_act_weight(dev_bf16(x), empty_w)
    torch.cuda.synchronize()
    wq_ref, ws_ref = oracle.quant_weight_128x128(w)
    assert_bits_equal(host_codes(wq), wq_ref, "weight alone codes")
    assert_bits_equal(host_f32(ws), ws_ref, "weight alone scales")
    q_ref, s_ref = oracle.quant_act_1x128(x)
    assert_bits_equal(host_codes(q), q_ref, "act alone codes")
    assert_bits_equal(host_f32(s), s_ref, "act alone scales")


def test_act_weight_padded_leading_dimensions():
    x = wl.activation(1, "tiny_fprop", 67, 70, 384, 100.0)
    w = wl.weight(1, "tiny_fprop", 68, 256, 384)
    xd = torch.zeros((70, 512), dtype=torch.bfloat16, device="cuda")
    xd[:, :384] = dev_bf16(x)
    wd = torch.zeros((256, 400), dtype=torch.bfloat16, device="cuda")
    wd[:, :384] = dev_bf16(w)
    q = torch.full((70, 400), 0x5A, dtype=torch.uint8, device="cuda")[:, :384]
    s = torch.full((3, 80), 7.0, device="cuda")[:, :70]
    wq = torch.full((256, 416), 0x5A, dtype=torch.uint8, device="cuda")[:, :384]
    ws = torch.full((2, 5), 7.0, device="cuda")[:, :3]
    fq.fp8_quantize_act_weight(xd[:, :384], wd[:, :384], q=q, scale=s, wq=wq, wscale=ws)
    torch.cuda.synchronize()
    q_ref, s_ref = oracle.quant_act_1x128(x)
    wq_ref, ws_ref = oracle.quant_weight_128x128(w)
    assert_bits_equal(host_codes(q.contiguous()), q_ref, "padded act codes")
    assert_bits_equal(host_f32(s.contiguous()), s_ref, "padded act scales")
    assert_bits_equal(host_codes(wq.contiguous()), wq_ref, "padded weight codes")
    assert_bits_equal(host_f32(ws.contiguous()), ws_ref, "padded weight scales")
    assert torch.all(q.as_strided((70, 16), (400, 1), q.storage_offset() + 384) == 0x5A)
    assert torch.all(wq.as_strided((256, 32), (416, 1), wq.storage_offset() + 384) == 0x5A)


# ------------------------------------- both Wgrad operands (128x1) in one launch

def test_act_128x1_pair_equals_separate_launches_full_size():
    """The Wgrad operands dY [8192][2048] and X [8192][7168] in one launch:
    byte-identical to the two separate 128x1 launches (each pinned to the
    oracle at full size above)."""
    g = wl.wgrad()
    dy, x = dev_bf16(g["dy"]), dev_bf16(g["x"])
    got = fq.fp8_quantize_act_128x1_pair(dy, x)
    ref = fq.fp8_quantize_act(dy, "128x1") + fq.fp8_quantize_act(x, "128x1")
    torch.cuda.synchronize()
    for a, b, tag in zip(got, ref, ("q0", "scale0", "q1", "scale1")):
        assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), tag


@pytest.mark.parametrize("cols0,cols1", [(8, 264), (200, 128), (128, 0), (0, 72)])
def test_act_128x1_pair_ragged_and_empty_sides(cols0, cols1):
    tokens = 256
    x0 = wl.activation(1, "wgrad", 70, tokens, max(cols0, 8), None)[:, :cols0]
    x1 = wl.activation(1, "wgrad", 71, tokens, max(cols1, 8), 50.0)[:, :cols1]
    d0 = torch.empty((tokens, cols0), dtype=torch.bfloat16, device="cuda") if cols0 == 0 else dev_bf16(x0)
    d1 = torch.empty((tokens, cols1), dtype=torch.bfloat16, device="cuda") if cols1 == 0 else dev_bf16(x1)
    q0, s0, q1, s1 = fq.fp8_quantize_act_128x1_pair(d0, d1)
    torch.cuda.synchronize()
    for cols, x, q, s, tag in ((cols0, x0, q0, s0, "x0"), (cols1, x1, q1, s1, "x1")):
        if cols == 0:
            continue
        q_ref, s_ref = oracle.quant_act_128x1(np.ascontiguousarray(x))
        assert_bits_equal(host_f32(s), s_ref, tag + " scales")
        assert_bits_equal(host_codes(q), q_ref, tag + " codes")


def test_act_128x1_pair_edge_tiles():
    rng = np.random.default_rng(72)
    e = _edge_rows(rng)                                           # [10][128] special tiles
    # the 10 special tiles as token columns, plus 6 plain ones: [128][16]
    x0 = np.concatenate([e.T, wl.activation(1, "wgrad", 73, 128, 128, None)[:, :6]], axis=1)
    x0 = np.concatenate([x0, x0[::-1]], axis=0)                   # [256][16]
    x1 = wl.activation(1, "wgrad", 74, 256, 136, 50.0)
    q0, s0, q1, s1 = fq.fp8_quantize_act_128x1_pair(dev_bf16(x0), dev_bf16(x1))
    torch.cuda.synchronize()
    for x, q, s, tag in ((x0, q0, s0, "edge"), (x1, q1, s1, "plain")):
        q_ref, s_ref = oracle.quant_act_128x1(np.ascontiguousarray(x))
        assert_bits_equal(host_f32(s), s_ref, tag + " scales")
        assert_bits_equal(host_codes(q), q_ref, tag + " codes")
