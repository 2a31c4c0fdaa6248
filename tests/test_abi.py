"""CPU checks of the C ABI boundary (no GPU, no kernel launch).

* the shared library loads and exports every function ``include/fp8q.h``
  declares;
* host-side validation returns the documented status code for NULL
  pointers, bad shapes, misalignment and bad enums, before anything touches
  the GPU (so these run without one);
* the Python binding exposes the same names and refuses CPU tensors.
"""
from __future__ import annotations

import ctypes
import os
import re

import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fp8q.h")

import fine_grained_fp8_quantize_amd as fq  # noqa: E402

OK, ERR_NULL, ERR_SHAPE, ERR_ALIGN, ERR_ENUM, ERR_HIP = 0, 1, 2, 3, 4, 5


def _declared_functions() -> list[str]:
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", text, flags=re.M)


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(fq.library_path()):
        from fine_grained_fp8_quantize_amd import build
        build.build(force=False)
    return fq._load()


def test_header_declares_the_four_entry_points():
    names = _declared_functions()
    for n in ("fp8_quantize_act", "fp8_quantize_weight", "fp8_gemm", "fp8_grouped_gemm",
              "fp8q_status_string", "fp8q_last_hip_error"):
        assert n in names


def test_library_exports_every_declared_symbol(lib):
    raw = ctypes.CDLL(fq.library_path())
    for name in _declared_functions():
        assert hasattr(raw, name), name


def test_header_status_codes_match_binding():
    text = open(HEADER).read()
    codes = dict(re.findall(r"#define\s+(FP8Q_\w+)\s+(\d+)", text))
    assert int(codes["FP8Q_OK"]) == OK
    assert int(codes["FP8Q_ERR_NULL"]) == ERR_NULL
    assert int(codes["FP8Q_ERR_SHAPE"]) == ERR_SHAPE
    assert int(codes["FP8Q_ERR_ALIGN"]) == ERR_ALIGN
    assert int(codes["FP8Q_ERR_ENUM"]) == ERR_ENUM
    assert int(codes["FP8Q_ERR_HIP"]) == ERR_HIP
    assert int(codes["FP8Q_TILE_1x128"]) == fq.TILE_1x128
    assert int(codes["FP8Q_TILE_128x1"]) == fq.TILE_128x1
    assert int(codes["FP8Q_BSCALE_BLOCK128"]) == fq.BSCALE_BLOCK128
    assert int(codes["FP8Q_BSCALE_ROW128"]) == fq.BSCALE_ROW128
    assert int(codes["FP8Q_OUT_BF16"]) == fq.OUT_BF16
    assert int(codes["FP8Q_OUT_F32"]) == fq.OUT_F32
    sizes = dict(re.findall(r"#define\s+(FP8Q_\w+)\s+(\d+)LL", text))
    assert int(sizes["FP8Q_GROUPED_WORKSPACE_BYTES"]) == fq.GROUPED_WORKSPACE_BYTES


def test_status_strings(lib):
    for s in range(6):
        assert fq.fp8q_status_string(s)
    assert fq.fp8q_status_string(99) == "unknown status"
    assert fq.fp8q_last_hip_error() == 0


# Fake, well-aligned device addresses: validation never dereferences them.
# The default arguments of each helper below describe a VALID call; every
# test call changes at least one argument so that validation rejects it (or
# an empty size returns OK) before anything is launched.
A16 = 0x10000
A16b = 0x20000
A16c = 0x30000
A4 = 0x40000


def _act(lib, x=A16, rows=256, cols=512, ld_x=512, tiling=0, q=A16b, ld_q=512, s=A4, ld_s=256):
    return lib.fp8_quantize_act(x, rows, cols, ld_x, tiling, q, ld_q, s, ld_s, None)


def test_quantize_act_validation(lib):
    assert _act(lib, tiling=2) == ERR_ENUM
    assert _act(lib, rows=-1) == ERR_SHAPE
    assert _act(lib, rows=0) == OK                  # empty: nothing to do, no launch
    assert _act(lib, cols=0) == OK
    assert _act(lib, x=0) == ERR_NULL
    assert _act(lib, q=0) == ERR_NULL
    assert _act(lib, s=0) == ERR_NULL
    assert _act(lib, cols=500, ld_x=512, ld_q=512) == ERR_SHAPE      # not a multiple of 128
    assert _act(lib, ld_x=256) == ERR_SHAPE                           # ld below width
    assert _act(lib, ld_s=255) == ERR_SHAPE                           # scale ld below rows
    assert _act(lib, x=A16 + 8) == ERR_ALIGN
    assert _act(lib, q=A16b + 4) == ERR_ALIGN
    assert _act(lib, s=A4 + 2) == ERR_ALIGN
    # 128x1: rows must be a multiple of 128, q is [cols][rows]
    assert _act(lib, tiling=1, rows=200, ld_q=512, ld_s=512) == ERR_SHAPE
    assert _act(lib, tiling=1, rows=256, cols=100, ld_x=512, ld_q=256, ld_s=512) == ERR_SHAPE
    assert _act(lib, tiling=1, rows=256, ld_q=128, ld_s=512) == ERR_SHAPE   # ld_q < rows


def test_quantize_act_ld_alignment_rule(lib):
    # ld_x must be a multiple of 8 elements (16 bytes); ld_q a multiple of 16.
    assert _act(lib, ld_x=516) == ERR_ALIGN
    assert _act(lib, ld_q=520) == ERR_ALIGN


def _sc(lib, x=A16, tokens=100, cols=512, ld_x=512, topk=8, dst=A4, m_total=256, q=A16b, ld_q=512,
        s=A4, ld_s=256):
    return lib.fp8_quantize_act_scatter(x, tokens, cols, ld_x, topk, dst, m_total, q, ld_q, s, ld_s, None)


def test_quantize_act_scatter_validation(lib):
    assert _sc(lib, tokens=0) == OK
    assert _sc(lib, m_total=0) == OK
    assert _sc(lib, tokens=-1) == ERR_SHAPE
    assert _sc(lib, topk=0) == ERR_SHAPE                  # 1..8 routes per token
    assert _sc(lib, topk=9) == ERR_SHAPE
    assert _sc(lib, dst=0) == ERR_NULL
    assert _sc(lib, x=0) == ERR_NULL
    assert _sc(lib, cols=500, ld_x=512, ld_q=512) == ERR_SHAPE
    assert _sc(lib, ld_s=255) == ERR_SHAPE                # scale ld below m_total
    assert _sc(lib, ld_q=256) == ERR_SHAPE
    assert _sc(lib, dst=A4 + 2) == ERR_ALIGN
    assert _sc(lib, q=A16b + 8) == ERR_ALIGN


def _w(lib, w=A16, n=256, k=384, ld_w=384, q=A16b, ld_q=384, s=A4, ld_s=3, qt=0, ld_qt=0, st=0, ld_st=0):
    return lib.fp8_quantize_weight(w, n, k, ld_w, q, ld_q, s, ld_s, qt, ld_qt, st, ld_st, None)


def test_quantize_weight_validation(lib):
    assert _w(lib, n=0) == OK
    assert _w(lib, n=-128) == ERR_SHAPE
    assert _w(lib, w=0) == ERR_NULL
    assert _w(lib, qt=A16c, st=0) == ERR_NULL          # transposed codes without scales
    assert _w(lib, n=200) == ERR_SHAPE
    assert _w(lib, k=200, ld_w=384, ld_q=384) == ERR_SHAPE
    assert _w(lib, ld_s=2) == ERR_SHAPE
    assert _w(lib, qt=A16c, ld_qt=128, st=A4, ld_st=2) == ERR_SHAPE   # ld_qt < n
    assert _w(lib, qt=A16c, ld_qt=256, st=A4, ld_st=1) == ERR_SHAPE   # ld_st < n/128
    assert _w(lib, w=A16 + 2) == ERR_ALIGN
    assert _w(lib, qt=A16c + 8, ld_qt=256, st=A4, ld_st=2) == ERR_ALIGN


def _g(lib, m=300, n=200, k=256, a=A16, lda=256, a_s=A4, ld_as=300, b=A16b, ldb=256, b_s=A4,
       ld_bs=2, kind=0, c=A16c, ldc=200, out=0):
    return lib.fp8_gemm(m, n, k, a, lda, a_s, ld_as, b, ldb, b_s, ld_bs, kind, c, ldc, out, None)


def test_gemm_validation(lib):
    assert _g(lib, kind=2) == ERR_ENUM
    assert _g(lib, out=3) == ERR_ENUM
    assert _g(lib, m=-1) == ERR_SHAPE
    assert _g(lib, m=0) == OK
    assert _g(lib, n=0) == OK
    assert _g(lib, a=0) == ERR_NULL
    assert _g(lib, c=0) == ERR_NULL
    assert _g(lib, a_s=0) == ERR_NULL
    assert _g(lib, k=200, lda=256, ldb=256) == ERR_SHAPE      # K not a multiple of 128
    assert _g(lib, lda=128) == ERR_SHAPE
    assert _g(lib, ldc=100) == ERR_SHAPE
    assert _g(lib, ld_as=299) == ERR_SHAPE
    assert _g(lib, ld_bs=1) == ERR_SHAPE                      # block scales need k/128 per row
    assert _g(lib, kind=1, ld_bs=199) == ERR_SHAPE            # row scales need n per slab
    assert _g(lib, a=A16 + 8) == ERR_ALIGN
    assert _g(lib, lda=264) == ERR_ALIGN                      # 264 % 16 != 0
    assert _g(lib, c=A16c + 4) == ERR_ALIGN
    assert _g(lib, ldc=204) == ERR_ALIGN


def test_gemm_operand_pitch_limits(lib):
    """Tiles and scales are addressed through 31-bit buffer ranges from the
    tile origin, so row pitches above 2^23 - 128 bytes and scale arrays of
    2^29 floats or more are refused on the host; at the limit the call is
    valid."""
    big = (1 << 23) - 128
    span = 1 << 29
    assert _g(lib, lda=big + 16) == ERR_SHAPE
    assert _g(lib, ldb=big + 16) == ERR_SHAPE
    assert _g(lib, ld_bs=span // 2) == ERR_SHAPE               # ceil(200/128) = 2 block rows
    assert _g(lib, ld_bs=(1 << 62)) == ERR_SHAPE               # no overflow in the span check
    assert _g(lib, ld_as=span // 2) == ERR_SHAPE               # 2 slabs of A scales
    assert _g(lib, kind=1, ld_bs=span // 2) == ERR_SHAPE       # 2 slabs of row scales
    assert _g(lib, kind=1, lda=big + 16, ld_bs=200) == ERR_SHAPE
    assert _gg(lib, lda=big + 16) == ERR_SHAPE
    assert _gg(lib, ldb=big + 16) == ERR_SHAPE
    assert _gg(lib, ld_bs=span // 2) == ERR_SHAPE              # 2 block rows per expert
    assert _gw(lib, lda=big + 16) == ERR_SHAPE
    assert _gw(lib, ld_bs=span // 4) == ERR_SHAPE              # 4 token slabs of row scales
    assert _mxg(lib, ldb=big + 16) == ERR_SHAPE
    assert _mxg(lib, ld_bs=span // 2) == ERR_SHAPE
    assert _tg(lib, lda=big + 16) == ERR_SHAPE
    if not torch.cuda.is_available():   # valid at the limit: fails only at the launch
        assert _g(lib, lda=big) == ERR_HIP
        assert _g(lib, ldb=big) == ERR_HIP
        assert _g(lib, ld_as=span // 2 - 1) == ERR_HIP


def _gg(lib, groups=4, off=A16, rows=0, m=512, n=256, k=256, a=A16b, lda=256, a_s=A4, ld_as=512,
        b=A16c, ldb=256, sb=256 * 256, b_s=A4, ld_bs=2, sbs=4, c=A16, ldc=256, out=0, ws=0, wsb=0):
    return lib.fp8_grouped_gemm(groups, off, rows, m, n, k, a, lda, a_s, ld_as, b, ldb, sb,
                                b_s, ld_bs, sbs, c, ldc, out, ws, wsb, None)


def test_grouped_gemm_validation(lib):
    assert _gg(lib, groups=0) == OK
    assert _gg(lib, m=0) == OK
    assert _gg(lib, groups=-1) == ERR_SHAPE
    assert _gg(lib, out=5) == ERR_ENUM
    assert _gg(lib, off=0) == ERR_NULL
    assert _gg(lib, m=500, ld_as=512) == ERR_SHAPE         # m_total not a multiple of 128
    assert _gg(lib, n=200, ldc=256) == ERR_SHAPE           # n not a multiple of 128
    assert _gg(lib, sb=-256) == ERR_SHAPE
    assert _gg(lib, sbs=-1) == ERR_SHAPE
    assert _gg(lib, sb=256 * 256 + 8) == ERR_ALIGN
    assert _gg(lib, ws=A16, wsb=-1) == ERR_SHAPE            # negative workspace size
    assert _gg(lib, ws=A16 + 128, wsb=1 << 20) == ERR_ALIGN  # workspace not 256-byte aligned


def _ggn(lib, groups=4, off=A16, rows=0, m=512, n=256, k=256, a=A16b, lda=256, a_s=A4, ld_as=512,
         b=A16c, ldb=256, sb=256 * 256, b_s=A4, ld_bs=2, sbs=4, c=A16, ldc=256, out=0):
    return lib.fp8_grouped_gemm_noalloc(groups, off, rows, m, n, k, a, lda, a_s, ld_as, b, ldb, sb,
                                        b_s, ld_bs, sbs, c, ldc, out, None)


def test_grouped_gemm_noalloc_validation(lib):
    """The allocation-free entry point checks its arguments as
    fp8_grouped_gemm does, before it looks for its scratch."""
    assert _ggn(lib, groups=0) == OK
    assert _ggn(lib, m=0) == OK
    assert _ggn(lib, groups=-1) == ERR_SHAPE
    assert _ggn(lib, out=5) == ERR_ENUM
    assert _ggn(lib, off=0) == ERR_NULL
    assert _ggn(lib, m=500, ld_as=512) == ERR_SHAPE
    assert _ggn(lib, n=200, ldc=256) == ERR_SHAPE
    assert _ggn(lib, sb=256 * 256 + 8) == ERR_ALIGN
    assert _ggn(lib, lda=(1 << 23)) == ERR_SHAPE


@pytest.mark.skipif(torch.cuda.is_available(), reason="would launch on the fake pointers")
def test_grouped_gemm_accepts_interleaved_expert_weights(lib):
    """The weights are only read, so experts' rows may interleave: the
    transposed copy of all experts quantized as one matrix has stride_b = k
    and ldb = groups * k. Without a GPU the call gets past validation and
    fails only at the launch (FP8Q_ERR_HIP), never with a shape error."""
    assert _gg(lib, sb=256, ldb=4 * 256, sbs=2, ld_bs=8) == ERR_HIP


def _gw(lib, groups=4, off=A16, kt=512, m=256, n=384, a=A16b, lda=512, a_s=A4, ld_as=256,
        b=A16c, ldb=512, b_s=A4, ld_bs=384, c=A16, ldc=384, sc=256 * 384, out=1):
    return lib.fp8_grouped_gemm_wgrad(groups, off, kt, m, n, a, lda, a_s, ld_as, b, ldb, b_s, ld_bs,
                                      c, ldc, sc, out, None)


def test_grouped_gemm_wgrad_validation(lib):
    assert _gw(lib, groups=0) == OK
    assert _gw(lib, m=0) == OK
    assert _gw(lib, groups=-1) == ERR_SHAPE
    assert _gw(lib, out=7) == ERR_ENUM
    assert _gw(lib, off=0) == ERR_NULL
    assert _gw(lib, b_s=0) == ERR_NULL
    assert _gw(lib, kt=500, lda=512, ldb=512) == ERR_SHAPE     # tokens not a multiple of 128
    assert _gw(lib, lda=256) == ERR_SHAPE                      # lda below k_total
    assert _gw(lib, ld_bs=383) == ERR_SHAPE                    # row scales need n per slab
    assert _gw(lib, sc=256 * 384 - 8) == ERR_SHAPE             # expert outputs overlap
    assert _gw(lib, sc=256 * 384 + 4) == ERR_ALIGN
    assert _gw(lib, c=A16 + 4) == ERR_ALIGN


def _mxq(lib, x=A16, rows=256, cols=512, ld_x=512, q=A16b, ld_q=512, s=A4, ld_s=256):
    return lib.fp8_quantize_mx(x, rows, cols, ld_x, q, ld_q, s, ld_s, None)


def _mxg(lib, m=300, n=200, k=256, a=A16, lda=256, a_s=A4, ld_as=300, b=A16b, ldb=256, b_s=A4,
         ld_bs=200, c=A16c, ldc=200, out=0):
    return lib.fp8_gemm_mx(m, n, k, a, lda, a_s, ld_as, b, ldb, b_s, ld_bs, c, ldc, out, None)


def test_mx_validation(lib):
    assert _mxq(lib, rows=0) == OK
    assert _mxq(lib, rows=-1) == ERR_SHAPE
    assert _mxq(lib, x=0) == ERR_NULL
    assert _mxq(lib, cols=480, ld_x=512, ld_q=512) == ERR_SHAPE   # whole 128-column slabs only
    assert _mxq(lib, ld_s=255) == ERR_SHAPE
    assert _mxq(lib, q=A16b + 8) == ERR_ALIGN
    assert _mxg(lib, m=0) == OK
    assert _mxg(lib, out=2) == ERR_ENUM
    assert _mxg(lib, b_s=0) == ERR_NULL
    assert _mxg(lib, k=200, lda=256, ldb=256) == ERR_SHAPE
    assert _mxg(lib, ld_bs=199) == ERR_SHAPE                    # one scale word per B row
    assert _mxg(lib, lda=264) == ERR_ALIGN


def _rt(lib, q=A16, tokens=256, cols=384, ld_q=384, s=A4, ld_s=256, qt=A16b, ld_qt=256, st=A4 + 0x1000,
        ld_st=384):
    return lib.fp8_retile_act_128x1(q, tokens, cols, ld_q, s, ld_s, qt, ld_qt, st, ld_st, None)


def test_retile_validation(lib):
    assert _rt(lib, tokens=0) == OK
    assert _rt(lib, cols=-128) == ERR_SHAPE
    assert _rt(lib, qt=0) == ERR_NULL
    assert _rt(lib, st=0) == ERR_NULL
    assert _rt(lib, tokens=200, ld_s=256, ld_qt=256) == ERR_SHAPE   # whole 128-token tiles
    assert _rt(lib, cols=320, ld_q=320, ld_st=320) == ERR_SHAPE     # whole 128-channel tiles
    assert _rt(lib, ld_q=256) == ERR_SHAPE
    assert _rt(lib, ld_s=128) == ERR_SHAPE
    assert _rt(lib, ld_qt=128) == ERR_SHAPE
    assert _rt(lib, ld_st=256) == ERR_SHAPE
    assert _rt(lib, s=A4 + 4) == ERR_ALIGN                         # 16-byte scale reads
    assert _rt(lib, ld_s=258) == ERR_ALIGN
    assert _rt(lib, ld_q=392) == ERR_ALIGN
    assert _rt(lib, qt=A16b + 8) == ERR_ALIGN


def _tg(lib, m=300, n=200, k=256, a=A16, lda=256, a_s=A4, b=A16b, ldb=256, b_s=A4, c=A16c, ldc=200, out=1):
    return lib.fp8_gemm_tensor(m, n, k, a, lda, a_s, b, ldb, b_s, c, ldc, out, None)


def test_gemm_tensor_validation(lib):
    assert _tg(lib, m=0) == OK
    assert _tg(lib, k=-128) == ERR_SHAPE
    assert _tg(lib, out=3) == ERR_ENUM
    assert _tg(lib, a_s=0) == ERR_NULL
    assert _tg(lib, b=0) == ERR_NULL
    assert _tg(lib, k=200, lda=256, ldb=256) == ERR_SHAPE
    assert _tg(lib, lda=128) == ERR_SHAPE
    assert _tg(lib, ldc=100) == ERR_SHAPE
    assert _tg(lib, ldb=264) == ERR_ALIGN
    assert _tg(lib, c=A16c + 4) == ERR_ALIGN


def _aw(lib, x=A16, rows=256, cols=512, ld_x=512, q=A16b, ld_q=512, s=A4, ld_s=256, w=A16c, n=256, k=384,
        ld_w=384, wq=A16 + 0x100000, ld_wq=384, ws=A4 + 0x1000, ld_ws=3, wqt=0, ld_wqt=0, wst=0, ld_wst=0):
    return lib.fp8_quantize_act_weight(x, rows, cols, ld_x, q, ld_q, s, ld_s, w, n, k, ld_w, wq, ld_wq, ws, ld_ws,
                                       wqt, ld_wqt, wst, ld_wst, None)


def test_quantize_act_weight_validation(lib):
    assert _aw(lib, rows=0, n=0) == OK                           # both empty: nothing launched
    assert _aw(lib, rows=-1) == ERR_SHAPE
    assert _aw(lib, x=0) == ERR_NULL
    assert _aw(lib, wq=0) == ERR_NULL
    assert _aw(lib, wqt=A16c + 0x200000, ld_wqt=256) == ERR_NULL  # q_t without scale_t
    assert _aw(lib, cols=500, ld_x=512, ld_q=512) == ERR_SHAPE
    assert _aw(lib, n=200) == ERR_SHAPE
    assert _aw(lib, ld_s=255) == ERR_SHAPE
    assert _aw(lib, ld_ws=2) == ERR_SHAPE
    assert _aw(lib, q=A16b + 8) == ERR_ALIGN
    assert _aw(lib, ld_wq=392) == ERR_ALIGN
    # an empty side is not checked (its pointers are not read)
    assert _aw(lib, rows=0, n=0, x=0, w=0) == OK
    # outputs of the two halves must not overlap (checked before any launch)
    assert _aw(lib, wq=A16b + 0x100) == ERR_SHAPE                   # codes over codes
    assert _aw(lib, ws=A4 + 8) == ERR_SHAPE                         # scales over scales
    assert _aw(lib, ws=A16b + 0x1000) == ERR_SHAPE                  # weight scales over act codes
    assert _aw(lib, wqt=A4 + 0x800, ld_wqt=256, wst=A4 + 0x2000, ld_wst=2) == ERR_SHAPE  # Wt codes over act scales
    assert _aw(lib, wqt=A16c + 0x200000, ld_wqt=256, wst=A16b, ld_wst=2) == ERR_SHAPE    # Wt scales over act codes


def _p128(lib, tokens=256, x0=A16, c0=256, ld_x0=256, q0=A16b, ld_q0=256, s0=A4, ld_s0=256, x1=A16c, c1=136,
          ld_x1=136, q1=A16 + 0x100000, ld_q1=256, s1=A4 + 0x1000, ld_s1=136):
    return lib.fp8_quantize_act_128x1_pair(tokens, x0, c0, ld_x0, q0, ld_q0, s0, ld_s0, x1, c1, ld_x1, q1, ld_q1,
                                           s1, ld_s1, None)


def test_quantize_act_128x1_pair_validation(lib):
    assert _p128(lib, tokens=0) == OK                              # nothing to do
    assert _p128(lib, c0=0, c1=0) == OK
    assert _p128(lib, tokens=-128) == ERR_SHAPE
    assert _p128(lib, tokens=200) == ERR_SHAPE                     # tokens % 128
    assert _p128(lib, c1=132, ld_x1=136, ld_s1=136) == ERR_SHAPE   # cols % 8
    assert _p128(lib, ld_q0=128) == ERR_SHAPE                      # ld_q < tokens
    assert _p128(lib, ld_s1=128) == ERR_SHAPE                      # ld_s < cols
    assert _p128(lib, x1=0) == ERR_NULL
    assert _p128(lib, q0=A16b + 8) == ERR_ALIGN
    assert _p128(lib, ld_x1=140) == ERR_ALIGN                      # ld_x % 8
    # empty operands are not read (both empty: nothing is launched)
    assert _p128(lib, c0=0, c1=0, x0=0, q0=0, s0=0, x1=0, q1=0, s1=0) == OK
    # outputs of the two halves must not overlap
    assert _p128(lib, q1=A16b + 0x400) == ERR_SHAPE
    assert _p128(lib, s1=A4 + 0x100) == ERR_SHAPE
    assert _p128(lib, s1=A16b + 0x100) == ERR_SHAPE


def _qr(lib, tokens=256, x0=A16, c0=256, ld_x0=256, q0=A16b, ld_q0=256, s0=A4, ld_s0=256, xq=A16c, c1=256,
        ld_xq=256, xs=A4 + 0x2000, ld_xs=256, q1=A16 + 0x100000, ld_q1=256, s1=A4 + 0x1000, ld_s1=256):
    return lib.fp8_quantize_act_128x1_retile(tokens, x0, c0, ld_x0, q0, ld_q0, s0, ld_s0, xq, c1, ld_xq, xs, ld_xs,
                                             q1, ld_q1, s1, ld_s1, None)


def test_quantize_act_128x1_retile_validation(lib):
    assert _qr(lib, tokens=0) == OK
    assert _qr(lib, c0=0, c1=0, x0=0, q0=0, s0=0, xq=0, xs=0, q1=0, s1=0) == OK   # nothing read or launched
    assert _qr(lib, tokens=-128) == ERR_SHAPE
    assert _qr(lib, tokens=200) == ERR_SHAPE
    assert _qr(lib, c1=136, ld_xq=256, ld_s1=256) == ERR_SHAPE     # the cache is re-tiled in whole 128 columns
    assert _qr(lib, ld_xs=128) == ERR_SHAPE                        # ld_xs < tokens
    assert _qr(lib, xq=0) == ERR_NULL
    assert _qr(lib, xs=A4 + 0x2004) == ERR_ALIGN                   # cache scales 16-byte aligned
    assert _qr(lib, ld_xs=258) == ERR_ALIGN
    assert _qr(lib, q1=A16b + 0x400) == ERR_SHAPE                  # outputs of the two halves overlap
    assert _qr(lib, s1=A4 + 0x100) == ERR_SHAPE


def _mxp(lib, x0=A16, r0=64, c0=256, ld_x0=256, q0=A16b, ld_q0=256, s0=A4, ld_s0=64, x1=A16c, r1=40, c1=128,
         ld_x1=128, q1=A16 + 0x100000, ld_q1=128, s1=A4 + 0x1000, ld_s1=40):
    return lib.fp8_quantize_mx_pair(x0, r0, c0, ld_x0, q0, ld_q0, s0, ld_s0, x1, r1, c1, ld_x1, q1, ld_q1, s1, ld_s1,
                                    None)


def test_quantize_mx_pair_validation(lib):
    assert _mxp(lib, r0=0, r1=0) == OK
    assert _mxp(lib, c0=0, c1=0, x0=0, q0=0, s0=0, x1=0, q1=0, s1=0) == OK   # nothing read or launched
    assert _mxp(lib, r1=-1) == ERR_SHAPE
    assert _mxp(lib, c0=200, ld_x0=256, ld_q0=256) == ERR_SHAPE
    assert _mxp(lib, ld_s1=39) == ERR_SHAPE
    assert _mxp(lib, q1=0) == ERR_NULL
    assert _mxp(lib, x0=A16 + 8) == ERR_ALIGN
    assert _mxp(lib, ld_q1=136) == ERR_ALIGN
    assert _mxp(lib, q1=A16b + 0x100) == ERR_SHAPE                  # outputs of the two halves overlap
    assert _mxp(lib, s1=A4 + 0x10) == ERR_SHAPE


def _wg(lib, groups=3, w=A16, n=256, k=384, ld_w=384, sw=256 * 384, q=A16b, ld_q=384, sq=256 * 384,
        s=A4, ld_s=3, ss=6, qt=A16c, ld_qt=256, sqt=384 * 256, st=A4 + 0x1000, ld_st=2, sst=6):
    return lib.fp8_quantize_weight_grouped(groups, w, n, k, ld_w, sw, q, ld_q, sq, s, ld_s, ss,
                                           qt, ld_qt, sqt, st, ld_st, sst, None)


def test_quantize_weight_grouped_validation(lib):
    assert _wg(lib, groups=0) == OK
    assert _wg(lib, n=0) == OK
    assert _wg(lib, groups=-1) == ERR_SHAPE
    assert _wg(lib, w=0) == ERR_NULL
    assert _wg(lib, st=0) == ERR_NULL                            # q_t without scale_t
    assert _wg(lib, n=200) == ERR_SHAPE
    assert _wg(lib, sq=256 * 384 - 16) == ERR_SHAPE              # output groups overlap
    assert _wg(lib, ss=5) == ERR_SHAPE
    assert _wg(lib, sqt=384 * 256 - 16) == ERR_SHAPE
    assert _wg(lib, sst=5) == ERR_SHAPE
    assert _wg(lib, sw=-8) == ERR_SHAPE
    assert _wg(lib, sw=256 * 384 + 4) == ERR_ALIGN               # 16-byte bf16 rows
    assert _wg(lib, sq=256 * 384 + 8) == ERR_ALIGN
    assert _wg(lib, sqt=384 * 256 + 8) == ERR_ALIGN


def test_binding_names_match_c_entry_points():
    for name in ("fp8_quantize_act", "fp8_quantize_act_scatter", "fp8_quantize_weight",
                 "fp8_quantize_weight_grouped", "fp8_quantize_act_weight", "fp8_quantize_act_128x1_pair",
                 "fp8_quantize_act_128x1_retile", "fp8_gemm", "fp8_grouped_gemm", "fp8_grouped_gemm_noalloc",
                 "fp8_grouped_gemm_wgrad", "fp8_quantize_mx", "fp8_quantize_mx_pair", "fp8_gemm_mx",
                 "fp8_retile_act_128x1", "fp8_gemm_tensor"):
        assert callable(getattr(fq, name))


def test_binding_refuses_cpu_tensors():
    x = torch.zeros((128, 128), dtype=torch.bfloat16)
    with pytest.raises(fq.Fp8qError):
        fq.fp8_quantize_act(x)
    w = torch.zeros((128, 128), dtype=torch.bfloat16)
    with pytest.raises(fq.Fp8qError):
        fq.fp8_quantize_weight(w)


def test_binding_checks_shapes_dtypes_and_strides():
    """The binding's own checks (the C ABI sees only pointers and leading
    dimensions, so a tensor smaller than the launch assumes must be refused
    in Python): dtype, exact shape, unit stride in the last dimension."""
    t = torch.zeros((4, 6), dtype=torch.float32)
    fq._check_tensor(t, (4, 6), fq._F32, "t")
    with pytest.raises(fq.Fp8qError, match="dtype"):
        fq._check_tensor(t.to(torch.bfloat16), (4, 6), fq._F32, "t")
    with pytest.raises(fq.Fp8qError, match="shape"):
        fq._check_tensor(t, (4, 7), fq._F32, "t")
    with pytest.raises(fq.Fp8qError, match="shape"):
        fq._check_tensor(t, (3, 6), fq._F32, "t")
    with pytest.raises(fq.Fp8qError, match="unit stride"):
        fq._check_tensor(t.t(), (6, 4), fq._F32, "t")
    # a view with a padded leading dimension is fine
    fq._check_tensor(torch.zeros((4, 8))[:, :6], (4, 6), fq._F32, "t")
    # GEMM outputs: wrong dtype (a bf16 buffer for fp32 output would be
    # written past its end), wrong shape, transposed view
    out = torch.zeros((5, 7), dtype=torch.bfloat16)
    assert fq._gemm_out(out, (5, 7), torch.bfloat16, "cpu", None) is out
    with pytest.raises(fq.Fp8qError, match="dtype"):
        fq._gemm_out(out, (5, 7), torch.float32, "cpu", None)
    with pytest.raises(fq.Fp8qError, match="shape"):
        fq._gemm_out(out, (5, 8), torch.bfloat16, "cpu", None)
    with pytest.raises(fq.Fp8qError, match="unit stride"):
        fq._gemm_out(torch.zeros((7, 5), dtype=torch.bfloat16).t(), (5, 7), torch.bfloat16, "cpu", None)
    # codes accept E4M3 or uint8 only
    fq._check_tensor(torch.zeros((2, 16), dtype=torch.uint8), (2, 16), fq._CODES, "q")
    with pytest.raises(fq.Fp8qError, match="dtype"):
        fq._check_tensor(torch.zeros((2, 16), dtype=torch.int8), (2, 16), fq._CODES, "q")
