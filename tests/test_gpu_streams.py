"""The library on the caller's streams: calls hold no state, so work enqueued
on two streams at once gives the same bytes as the same work done one call
after another; a quantize + GEMM step, and the grouped GEMM with its K-split
fix-up (caller workspace or the library's scratch), captured into a HIP graph
replay to the eager result (the kernels use no memset and no atomics).
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import fine_grained_fp8_quantize_amd as fq
import workloads as wl
from gpu_util import dev_bf16

pytestmark = pytest.mark.gpu


def _step(x, w, bufs):
    """One Fprop step into preallocated buffers: X and W in one launch, then the GEMM."""
    q, s, wq, ws, y = bufs
    fq.fp8_quantize_act_weight(x, w, q=q, scale=s, wq=wq, wscale=ws)
    fq.fp8_gemm(q, s, wq, ws, "block", torch.bfloat16, out=y)


def _bufs(m, n, k):
    return (torch.empty((m, k), dtype=torch.uint8, device="cuda"),
            torch.empty((k // 128, m), dtype=torch.float32, device="cuda"),
            torch.empty((n, k), dtype=torch.uint8, device="cuda"),
            torch.empty((n // 128, k // 128), dtype=torch.float32, device="cuda"),
            torch.empty((m, n), dtype=torch.bfloat16, device="cuda"))


def _same(a, b):
    """Bit-equal (any dtype, compared as bytes)."""
    return torch.equal(a.view(torch.uint8), b.view(torch.uint8))


def test_two_streams_at_once_match_serial():
    m, n, k = 1024, 512, 2048
    xs = [dev_bf16(wl.activation(6, "tiny_fprop", 110 + i, m, k, 50.0)) for i in range(2)]
    ws = [dev_bf16(wl.weight(6, "tiny_fprop", 120 + i, n, k)) for i in range(2)]
    serial = [_bufs(m, n, k) for _ in range(2)]
    for i in range(2):
        _step(xs[i], ws[i], serial[i])
    torch.cuda.synchronize()
    conc = [_bufs(m, n, k) for _ in range(2)]
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]   # default priority
    start = torch.cuda.Event()
    start.record()
    for rep in range(3):          # several rounds, interleaved across the streams
        for i in range(2):
            streams[i].wait_event(start)
            with torch.cuda.stream(streams[i]):
                _step(xs[i], ws[i], conc[i])
    torch.cuda.synchronize()
    for i in range(2):
        for a, b, what in zip(conc[i], serial[i], ("q", "scale", "wq", "wscale", "y")):
            assert _same(a, b), "stream %d: %s differs from the serial run" % (i, what)


def test_graph_replay_matches_eager():
    m, n, k = 512, 256, 1024
    inputs = [dev_bf16(wl.activation(7, "tiny_fprop", 130 + i, m, k, 50.0)) for i in range(3)]
    w = dev_bf16(wl.weight(7, "tiny_fprop", 140, n, k))
    x = torch.empty_like(inputs[0])
    x.copy_(inputs[0])
    bufs = _bufs(m, n, k)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm up on the capture stream
        _step(x, w, bufs)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        _step(x, w, bufs)
    torch.cuda.synchronize()
    ref = _bufs(m, n, k)
    for rep in range(6):
        src = inputs[rep % 3]
        x.copy_(src)                 # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        _step(src, w, ref)           # the eager result for the same input
        torch.cuda.synchronize()
        for a, b, what in zip(bufs, ref, ("q", "scale", "wq", "wscale", "y")):
            assert _same(a, b), "replay %d: %s differs from eager" % (rep, what)
    assert not np.isnan(bufs[4].float().cpu().numpy()).any()


def test_grouped_gemm_graph_replay_matches_eager():
    """The grouped GEMM with its K-split last round (the GEMM kernel, then the
    fix-up kernel over the workspace) captured into a HIP graph, once with a
    caller workspace and once through the allocation-free entry point (whose
    scratch address is looked up by a call made before the capture); every
    replay, with new activations copied in eagerly between replays, equals
    an eager call bit for bit."""
    rows = np.array([300, 5, 0, 128, 257, 40])
    n, k = 384, 18 * 128                        # 14 tiles: 4 K pieces each
    off = wl.pad_offsets(rows)
    m_total = int(off[-1])
    E = len(rows)
    xs = [dev_bf16(wl.activation(9, "grouped_fprop", 150 + i, m_total, k, 50.0)) for i in range(3)]
    w = dev_bf16(wl.weight(9, "grouped_fprop", 160, E * n, k))
    wq, wsc = fq.fp8_quantize_weight(w)
    wq, wsc = wq.view(E, n, k), wsc.view(E, n // 128, k // 128)
    off_d = torch.from_numpy(off.astype(np.int32)).cuda()
    rows_d = torch.from_numpy(rows.astype(np.int32)).cuda()
    a = torch.empty((m_total, k), dtype=torch.uint8, device="cuda")
    sa = torch.empty((k // 128, m_total), dtype=torch.float32, device="cuda")
    ws = torch.empty(fq.GROUPED_WORKSPACE_BYTES, dtype=torch.uint8, device="cuda")
    y_ws = torch.empty((m_total, n), dtype=torch.bfloat16, device="cuda")
    y_na = torch.empty((m_total, n), dtype=torch.bfloat16, device="cuda")
    ref = torch.empty((m_total, n), dtype=torch.bfloat16, device="cuda")
    ref_ws = torch.empty(fq.GROUPED_WORKSPACE_BYTES, dtype=torch.uint8, device="cuda")

    def quant(x):
        fq.fp8_quantize_act(x, q=a, scale=sa)

    def gemms():
        fq.fp8_grouped_gemm(off_d, rows_d, a, sa, wq, wsc, torch.bfloat16, out=y_ws, workspace=ws)
        fq.fp8_grouped_gemm_noalloc(off_d, rows_d, a, sa, wq, wsc, torch.bfloat16, out=y_na)

    quant(xs[0])
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):   # warm up (and look up the scratch) on the capture stream
        gemms()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        gemms()
    torch.cuda.synchronize()
    for rep in range(6):
        quant(xs[rep % 3])           # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        fq.fp8_grouped_gemm(off_d, rows_d, a, sa, wq, wsc, torch.bfloat16, out=ref, workspace=ref_ws)
        torch.cuda.synchronize()
        assert _same(y_ws, ref), "replay %d: workspace entry point differs from eager" % rep
        assert _same(y_na, ref), "replay %d: allocation-free entry point differs from eager" % rep
    assert torch.isfinite(ref.float()).all()
