"""The Python binding refuses arguments the C ABI cannot check, before any
launch: it alone knows the tensors' sizes, so a GEMM output of the wrong
dtype or shape, a scale tensor of the wrong shape or a weight of the wrong K
would otherwise be read or written out of bounds. Every refused call leaves
its (sentinel-filled) output untouched. Outputs allocated for an explicit
stream come back correct on that stream."""
from __future__ import annotations

import pytest
import torch

import fine_grained_fp8_quantize_amd as fq

pytestmark = pytest.mark.gpu


def _codes(r, c, v=0x38):
    return torch.full((r, c), v, dtype=torch.uint8, device="cuda")


def _f32(*shape, v=1.0):
    return torch.full(shape, v, dtype=torch.float32, device="cuda")


def _refused(fn, out, what):
    before = out.clone()
    with pytest.raises(fq.Fp8qError, match=what):
        fn()
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.uint8), before.view(torch.uint8)), "output written by a refused call"


def test_gemm_refuses_bad_out_and_scales():
    m, n, k = 256, 384, 256
    a, b = _codes(m, k), _codes(n, k)
    sa, sb = _f32(k // 128, m), _f32((n + 127) // 128, k // 128)
    good = torch.full((m, n), 7.0, dtype=torch.bfloat16, device="cuda")
    # fp32 output into a bf16 buffer: the kernel would write twice its size
    _refused(lambda: fq.fp8_gemm(a, sa, b, sb, "block", torch.float32, out=good), good, "dtype")
    small = torch.full((m - 1, n), 7.0, dtype=torch.bfloat16, device="cuda")
    _refused(lambda: fq.fp8_gemm(a, sa, b, sb, "block", torch.bfloat16, out=small), small, "shape")
    _refused(lambda: fq.fp8_gemm(a, _f32(k // 128, m - 1), b, sb, "block", torch.bfloat16, out=good), good,
             "a_scale")
    _refused(lambda: fq.fp8_gemm(a, sa, b, _f32(k // 128, n), "block", torch.bfloat16, out=good), good,
             "b_scale")
    _refused(lambda: fq.fp8_gemm(a, sa, b, sb.to(torch.float16), "block", torch.bfloat16, out=good), good,
             "b_scale")
    # the valid call still works on the same buffers
    fq.fp8_gemm(a, sa, b, sb, "block", torch.bfloat16, out=good)
    torch.cuda.synchronize()
    assert torch.all(good == 256.0)    # 256 products of 1.0 * 1.0 (code 0x38 = 1.0)


def test_grouped_gemms_refuse_bad_out_and_weights():
    E, n, k = 3, 256, 256
    off = torch.tensor([0, 128, 256, 384], dtype=torch.int32, device="cuda")
    rows = torch.tensor([5, 128, 0], dtype=torch.int32, device="cuda")
    a, sa = _codes(384, k), _f32(k // 128, 384)
    b = torch.full((E, n, k), 0x38, dtype=torch.uint8, device="cuda")
    sb = _f32(E, n // 128, k // 128)
    out = torch.full((384, n), 7.0, dtype=torch.bfloat16, device="cuda")
    _refused(lambda: fq.fp8_grouped_gemm(off, rows, a, sa, b, sb, torch.float32, out=out), out, "dtype")
    _refused(lambda: fq.fp8_grouped_gemm(off, rows, a, sa, b[:, :, :128], sb, torch.bfloat16, out=out), out,
             "disagree on K")
    _refused(lambda: fq.fp8_grouped_gemm(off, rows, a, sa, b, sb[:, :1], torch.bfloat16, out=out), out, "b_scale")
    _refused(lambda: fq.fp8_grouped_gemm(off[:3], rows, a, sa, b, sb, torch.bfloat16, out=out), out,
             "group_offsets")
    # Wgrad: its default output is fp32; a bf16 buffer must be refused
    at, bt = _codes(n, 384), _codes(k, 384)
    sat, sbt = _f32(3, n), _f32(3, k)
    wout = torch.full((E, n, k), 7.0, dtype=torch.bfloat16, device="cuda")
    _refused(lambda: fq.fp8_grouped_gemm_wgrad(off, at, sat, bt, sbt, out=wout), wout, "dtype")
    _refused(lambda: fq.fp8_grouped_gemm_wgrad(off, at, sat, bt, sbt, torch.bfloat16, out=wout[:, :, :128]),
             wout, "shape")
    _refused(lambda: fq.fp8_grouped_gemm_wgrad(off, at, _f32(2, n), bt, sbt, torch.bfloat16, out=wout), wout,
             "a_scale")


def test_quantizers_refuse_bad_outputs():
    x = torch.ones((256, 384), dtype=torch.bfloat16, device="cuda")
    q = torch.full((256, 256), 0x5A, dtype=torch.uint8, device="cuda")     # too few columns
    _refused(lambda: fq.fp8_quantize_act(x, q=q), q, "shape")
    s = torch.full((2, 256), 7.0, device="cuda")                           # too few slabs
    _refused(lambda: fq.fp8_quantize_act(x, scale=s), s, "shape")
    qt = torch.full((384, 255), 0x5A, dtype=torch.uint8, device="cuda")    # 128x1: q is [cols][rows]
    _refused(lambda: fq.fp8_quantize_act(x, "128x1", q=qt), qt, "shape")
    w = torch.ones((256, 384), dtype=torch.bfloat16, device="cuda")
    ws = torch.full((2, 3), 7.0, dtype=torch.float64, device="cuda")
    _refused(lambda: fq.fp8_quantize_weight(w, scale=ws), ws, "dtype")


def test_outputs_for_a_side_stream():
    """With stream= the outputs are taken on that stream and the kernels run
    there; the result equals the current-stream result bit for bit."""
    m, n, k = 512, 384, 512
    g = torch.Generator(device="cuda").manual_seed(3)
    x = torch.randn((m, k), device="cuda", generator=g).to(torch.bfloat16)
    w = (0.02 * torch.randn((n, k), device="cuda", generator=g)).to(torch.bfloat16)
    q, s, wq, ws = fq.fp8_quantize_act_weight(x, w)
    ref = fq.fp8_gemm(q, s, wq, ws, "block", torch.bfloat16)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    q2, s2, wq2, ws2 = fq.fp8_quantize_act_weight(x, w, stream=side)
    y = fq.fp8_gemm(q2, s2, wq2, ws2, "block", torch.bfloat16, stream=side)
    side.synchronize()
    assert torch.equal(y.view(torch.int16), ref.view(torch.int16))
    assert torch.equal(q2.view(torch.uint8), q.view(torch.uint8))


def test_debug_flag_checks_segment_arrays(monkeypatch):
    """FP8Q_DEBUG=1: the grouped GEMMs copy their segment arrays to the host
    and refuse a contract violation (FP8Q_ERR_SHAPE) before launching."""
    monkeypatch.setenv("FP8Q_DEBUG", "1")
    E, n, k = 3, 256, 256
    a, sa = _codes(384, k), _f32(k // 128, 384)
    b = torch.full((E, n, k), 0x38, dtype=torch.uint8, device="cuda")
    sb = _f32(E, n // 128, k // 128)
    out = torch.full((384, n), 7.0, dtype=torch.bfloat16, device="cuda")

    def off(v):
        return torch.tensor(v, dtype=torch.int32, device="cuda")
    rows_ok = off([5, 128, 0])
    for bad in ([0, 256, 128, 384], [0, 100, 256, 384], [0, 128, 256, 256], [128, 128, 256, 384]):
        _refused(lambda: fq.fp8_grouped_gemm(off(bad), rows_ok, a, sa, b, sb, torch.bfloat16, out=out), out,
                 "bad shape")
    _refused(lambda: fq.fp8_grouped_gemm(off([0, 128, 256, 384]), off([5, 129, 0]), a, sa, b, sb, torch.bfloat16,
                                         out=out), out, "bad shape")
    fq.fp8_grouped_gemm(off([0, 128, 256, 384]), rows_ok, a, sa, b, sb, torch.bfloat16, out=out)
    torch.cuda.synchronize()
    assert torch.all(out[:5] == 256.0) and torch.all(out[5:128] == 0) and torch.all(out[128:256] == 256.0)
    at, bt = _codes(n, 384), _codes(k, 384)
    sat, sbt = _f32(3, n), _f32(3, k)
    wout = torch.full((E, n, k), 7.0, dtype=torch.float32, device="cuda")
    _refused(lambda: fq.fp8_grouped_gemm_wgrad(off([0, 256, 128, 384]), at, sat, bt, sbt, out=wout), wout,
             "bad shape")
    fq.fp8_grouped_gemm_wgrad(off([0, 0, 256, 384]), at, sat, bt, sbt, out=wout)
    torch.cuda.synchronize()
    assert torch.all(wout[0] == 0) and torch.all(wout[1] == 256.0) and torch.all(wout[2] == 128.0)
