"""fine_grained_fp8_quantize_amd -- fine-grained FP8 quantization and block-scaled
FP8 GEMM for AMD Instinct MI355X (gfx950).

A thin binding over the C ABI of ``libfp8q.so`` (declared in
``include/fp8q.h``). The functions carry the same names as the C entry
points; they only marshal torch tensors into pointers, sizes and the current
HIP stream, and allocate outputs with torch when the caller does not pass
them. Every step of the computation runs in the library's gfx950 kernels;
there is no fallback: if the library is not built, or a tensor is not on the
GPU, the call raises.

Layouts (row-major, K contiguous for GEMM operands):

* ``fp8_quantize_act(x)`` -- bf16 ``x[rows][cols]`` -> E4M3 codes
  ``q[rows][cols]`` and FP32 scales ``scale[cols/128][rows]`` (1x128 tiles);
  with ``tiling="128x1"`` the codes come out transposed, ``q[cols][rows]``,
  with scales ``scale[rows/128][cols]``.
* ``fp8_quantize_weight(w)`` -- bf16 ``w[n][k]`` -> ``q[n][k]``,
  ``scale[n/128][k/128]`` (128x128 blocks), optionally also the transpose.
* ``fp8_gemm(a, a_scale, b, b_scale)`` -- ``C[m][n] = dequant(A) dequant(B)^T``.
* ``fp8_grouped_gemm(offsets, rows, a, a_scale, b, b_scale)`` -- per-expert
  Fprop (or Dgrad, with transposed weights) over an expert-sorted, 128-padded
  row layout.
* ``fp8_grouped_gemm_noalloc(...)`` -- the same on the library's per-GPU
  scratch instead of a workspace, for callers that cannot allocate.
* ``fp8_quantize_weight_grouped(w)`` -- ``w[E][n][k]`` quantized in one
  launch, optionally with per-expert transposed copies.
* ``fp8_quantize_act_weight(x, w)`` -- a Linear layer's activation (1x128)
  and weight (128x128, optionally transposed too) in one launch.
* ``fp8_quantize_act_128x1_pair(dy, x)`` -- the two Wgrad operands in 128x1
  token tiles in one launch.
* ``fp8_quantize_act_128x1_retile(dy, xq, xs)`` -- the same when X comes from
  the FP8 activation cache (dY quantized, X re-tiled) in one launch.
* ``fp8_quantize_act_scatter(x, dst_rows, m_total)`` -- quantize each token
  once and scatter its codes and scales to its expert-sorted rows.
* ``fp8_grouped_gemm_wgrad(offsets, a, a_scale, b, b_scale)`` -- per-expert
  Wgrad over each expert's token segment.
* ``fp8_retile_act_128x1(q, scale)`` -- a cached 1x128 activation re-tiled
  into 128x1 token tiles.
* ``fp8_quantize_mx`` / ``fp8_quantize_mx_pair`` / ``fp8_gemm_mx`` -- the
  microscaling variant (1x32 blocks, E8M0 scales, scaled MFMA); the pair
  quantizes both GEMM operands in one launch.
* ``fp8_gemm_tensor`` -- one scale per operand, the whole K sum in the MFMA
  accumulators.

E4M3 tensors are returned as ``torch.float8_e4m3fn`` (OCP E4M3FN bytes);
``uint8`` tensors are accepted wherever codes are inputs.
"""
from __future__ import annotations

import ctypes
import os

import torch

__all__ = [
    "fp8_quantize_act",
    "fp8_quantize_act_scatter",
    "fp8_quantize_weight",
    "fp8_quantize_weight_grouped",
    "fp8_quantize_act_weight",
    "fp8_quantize_act_128x1_pair",
    "fp8_quantize_act_128x1_retile",
    "fp8_quantize_mx_pair",
    "fp8_gemm",
    "fp8_grouped_gemm",
    "fp8_grouped_gemm_noalloc",
    "fp8_grouped_gemm_wgrad",
    "fp8_quantize_mx",
    "fp8_gemm_mx",
    "fp8_retile_act_128x1",
    "fp8_gemm_tensor",
    "fp8q_status_string",
    "fp8q_last_hip_error",
    "Fp8qError",
    "library_path",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
# FP8Q_LIBRARY names another build of the same C ABI (the sanitizer build of
# the host-side layer, for the CPU test suites); by default the in-tree one.
_LIB_PATH = os.environ.get("FP8Q_LIBRARY") or os.path.join(_HERE, "libfp8q.so")

TILE_1x128 = 0
TILE_128x1 = 1
# device bytes that let fp8_grouped_gemm split every partial last round
# (FP8Q_GROUPED_WORKSPACE_BYTES)
GROUPED_WORKSPACE_BYTES = 256 * 32 + 256 * 256 * 256 * 4
BSCALE_BLOCK128 = 0
BSCALE_ROW128 = 1
OUT_BF16 = 0
OUT_F32 = 1

_lib = None


class Fp8qError(RuntimeError):
    """A libfp8q entry point returned a non-zero status."""


def library_path() -> str:
    return _LIB_PATH


def _load() -> ctypes.CDLL:
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise Fp8qError(
            "libfp8q.so is not built (expected at %s); build it with "
            "`python -m fine_grained_fp8_quantize_amd.build`" % _LIB_PATH)
    L = ctypes.CDLL(_LIB_PATH)
    p, i64, i32, cint = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_int
    L.fp8_quantize_act.argtypes = [p, i64, i64, i64, cint, p, i64, p, i64, p]
    L.fp8_quantize_act_scatter.argtypes = [p, i64, i64, i64, i32, p, i64, p, i64, p, i64, p]
    L.fp8_quantize_weight.argtypes = [p, i64, i64, i64, p, i64, p, i64, p, i64, p, i64, p]
    L.fp8_quantize_act_weight.argtypes = [p, i64, i64, i64, p, i64, p, i64, p, i64, i64, i64, p, i64, p, i64,
                                          p, i64, p, i64, p]
    L.fp8_quantize_act_128x1_pair.argtypes = [i64, p, i64, i64, p, i64, p, i64, p, i64, i64, p, i64, p, i64, p]
    L.fp8_quantize_act_128x1_retile.argtypes = [i64, p, i64, i64, p, i64, p, i64, p, i64, i64, p, i64, p, i64, p,
                                                i64, p]
    L.fp8_quantize_mx_pair.argtypes = [p, i64, i64, i64, p, i64, p, i64, p, i64, i64, i64, p, i64, p, i64, p]
    L.fp8_quantize_weight_grouped.argtypes = [i32, p, i64, i64, i64, i64, p, i64, i64, p, i64, i64,
                                              p, i64, i64, p, i64, i64, p]
    L.fp8_quantize_mx.argtypes = [p, i64, i64, i64, p, i64, p, i64, p]
    L.fp8_gemm_mx.argtypes = [i64, i64, i64, p, i64, p, i64, p, i64, p, i64, p, i64, cint, p]
    L.fp8_gemm.argtypes = [i64, i64, i64, p, i64, p, i64, p, i64, p, i64, cint, p, i64, cint, p]
    L.fp8_grouped_gemm_wgrad.argtypes = [i32, p, i64, i64, i64, p, i64, p, i64, p, i64, p, i64,
                                         p, i64, i64, cint, p]
    L.fp8_grouped_gemm.argtypes = [i32, p, p, i64, i64, i64, p, i64, p, i64, p, i64, i64, p, i64,
                                   i64, p, i64, cint, p, i64, p]
    L.fp8_grouped_gemm_noalloc.argtypes = [i32, p, p, i64, i64, i64, p, i64, p, i64, p, i64, i64, p, i64,
                                           i64, p, i64, cint, p]
    L.fp8_retile_act_128x1.argtypes = [p, i64, i64, i64, p, i64, p, i64, p, i64, p]
    L.fp8_gemm_tensor.argtypes = [i64, i64, i64, p, i64, p, p, i64, p, p, i64, cint, p]
    for name in ("fp8_quantize_act", "fp8_quantize_act_scatter", "fp8_quantize_weight",
                 "fp8_quantize_weight_grouped", "fp8_quantize_act_weight", "fp8_quantize_act_128x1_pair",
                 "fp8_quantize_act_128x1_retile", "fp8_gemm", "fp8_grouped_gemm", "fp8_grouped_gemm_noalloc",
                 "fp8_grouped_gemm_wgrad", "fp8_quantize_mx", "fp8_quantize_mx_pair", "fp8_gemm_mx",
                 "fp8_retile_act_128x1", "fp8_gemm_tensor"):
        getattr(L, name).restype = cint
    L.fp8q_status_string.argtypes = [cint]
    L.fp8q_status_string.restype = ctypes.c_char_p
    L.fp8q_last_hip_error.argtypes = []
    L.fp8q_last_hip_error.restype = cint
    _lib = L
    return L


def fp8q_status_string(status: int) -> str:
    return _load().fp8q_status_string(status).decode()


def fp8q_last_hip_error() -> int:
    return int(_load().fp8q_last_hip_error())


def _check(status: int, what: str) -> None:
    if status != 0:
        msg = "%s failed: %s (status %d)" % (what, fp8q_status_string(status), status)
        if status == 5:
            msg += ", hipError %d" % fp8q_last_hip_error()
        raise Fp8qError(msg)


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _ptr(t: torch.Tensor | None) -> ctypes.c_void_p:
    return ctypes.c_void_p(0 if t is None else t.data_ptr())


def _need_gpu(*ts: torch.Tensor) -> None:
    for t in ts:
        if t is not None and not t.is_cuda:
            raise Fp8qError("fp8q tensors must live on the GPU (got a %s tensor)" % t.device)


def _rowmajor(t: torch.Tensor, name: str) -> None:
    # an empty matrix has no layout to check (numpy hands out zero strides)
    if t.dim() != 2 or (t.numel() > 0 and t.stride(1) != 1):
        raise Fp8qError("%s must be a 2-D tensor with unit column stride" % name)


def _codes(t: torch.Tensor, name: str) -> torch.Tensor:
    if t.dtype == torch.float8_e4m3fn:
        return t
    if t.dtype == torch.uint8:
        return t
    raise Fp8qError("%s must hold E4M3 codes (float8_e4m3fn or uint8), got %s" % (name, t.dtype))


def _empty(shape, dtype, device, stream):
    """A new output tensor. With an explicit ``stream`` the memory is taken on
    that stream, the one the kernel writes it on, so that the caching
    allocator does not hand the block to other work while the kernel runs."""
    if stream is None:
        return torch.empty(shape, dtype=dtype, device=device)
    with torch.cuda.stream(stream):
        return torch.empty(shape, dtype=dtype, device=device)


def _check_tensor(t: torch.Tensor, shape, dtypes, name: str) -> None:
    """Exact shape, an accepted dtype and a unit stride in the last dimension:
    the C ABI sees only a pointer and leading dimensions, so a tensor smaller
    than the launch assumes would be written or read out of bounds."""
    if t.dtype not in dtypes:
        raise Fp8qError("%s has dtype %s, expected %s" % (name, t.dtype, " or ".join(str(d) for d in dtypes)))
    if tuple(t.shape) != tuple(int(v) for v in shape):
        raise Fp8qError("%s has shape %s, expected %s" % (name, tuple(t.shape), tuple(int(v) for v in shape)))
    if t.numel() > 0 and t.stride(-1) != 1:
        raise Fp8qError("%s must have a unit stride in its last dimension" % name)
    if t.numel() > 0 and any(t.stride(i) < 0 for i in range(t.dim())):
        raise Fp8qError("%s has a negative stride" % name)


_CODES = (torch.float8_e4m3fn, torch.uint8)
_F32 = (torch.float32,)


# ------------------------------------------------------------- quantization

def fp8_quantize_act(x: torch.Tensor, tiling: str = "1x128", q: torch.Tensor | None = None,
                     scale: torch.Tensor | None = None, stream=None):
    """Quantize bf16 activations to E4M3 with one FP32 scale per tile.

    ``tiling="1x128"``: returns ``q[rows][cols]``, ``scale[cols/128][rows]``.
    ``tiling="128x1"``: returns ``q[cols][rows]`` (transposed, token-contiguous)
    and ``scale[rows/128][cols]``.
    """
    _need_gpu(x, q, scale)
    _rowmajor(x, "x")
    if x.dtype != torch.bfloat16:
        raise Fp8qError("x must be bfloat16")
    rows, cols = x.shape
    t = {"1x128": TILE_1x128, "128x1": TILE_128x1}.get(tiling)
    if t is None:
        raise Fp8qError("tiling must be '1x128' or '128x1'")
    dev = x.device
    q_shape = (rows, cols) if t == TILE_1x128 else (cols, rows)
    s_shape = (cols // 128, rows) if t == TILE_1x128 else (rows // 128, cols)
    if q is None:
        q = _empty(q_shape, torch.float8_e4m3fn, dev, stream)
    if scale is None:
        scale = _empty(s_shape, torch.float32, dev, stream)
    _check_tensor(q, q_shape, _CODES, "q")
    _check_tensor(scale, s_shape, _F32, "scale")
    st = _load().fp8_quantize_act(_ptr(x), rows, cols, x.stride(0), t, _ptr(q), q.stride(0),
                                  _ptr(scale), scale.stride(0), _stream(stream))
    _check(st, "fp8_quantize_act")
    return q, scale


def fp8_quantize_act_scatter(x: torch.Tensor, dst_rows: torch.Tensor, m_total: int,
                             q: torch.Tensor | None = None, scale: torch.Tensor | None = None,
                             stream=None):
    """Quantize bf16 token rows once (1x128 tiles) and scatter codes and
    scales to their expert-sorted destination rows.

    ``dst_rows`` is an int32 device tensor ``[tokens][topk]`` (topk 1..8) of
    destination rows in ``q``, -1 for routes outside this layout. Returns
    ``q[m_total][cols]`` and ``scale[cols/128][m_total]``; rows no route names
    (segment padding) are left as they were.
    """
    _need_gpu(x, dst_rows, q, scale)
    _rowmajor(x, "x")
    if not dst_rows.is_contiguous():
        raise Fp8qError("dst_rows must be contiguous [tokens][topk]")
    if x.dtype != torch.bfloat16:
        raise Fp8qError("x must be bfloat16")
    if dst_rows.dtype != torch.int32 or dst_rows.dim() != 2 or dst_rows.shape[0] != x.shape[0]:
        raise Fp8qError("dst_rows must be int32 [tokens][topk]")
    tokens, cols = x.shape
    topk = dst_rows.shape[1]
    dev = x.device
    if q is None:
        q = _empty((m_total, cols), torch.float8_e4m3fn, dev, stream)
    if scale is None:
        scale = _empty((cols // 128, m_total), torch.float32, dev, stream)
    _check_tensor(q, (m_total, cols), _CODES, "q")
    _check_tensor(scale, (cols // 128, m_total), _F32, "scale")
    st = _load().fp8_quantize_act_scatter(_ptr(x), tokens, cols, x.stride(0), topk, _ptr(dst_rows),
                                          m_total, _ptr(q), q.stride(0), _ptr(scale),
                                          scale.stride(0), _stream(stream))
    _check(st, "fp8_quantize_act_scatter")
    return q, scale


def fp8_quantize_weight(w: torch.Tensor, transposed: bool = False, q: torch.Tensor | None = None,
                        scale: torch.Tensor | None = None, q_t: torch.Tensor | None = None,
                        scale_t: torch.Tensor | None = None, stream=None):
    """Quantize a bf16 weight ``w[n][k]`` in 128x128 blocks.

    Returns ``(q, scale)``, or ``(q, scale, q_t, scale_t)`` when ``transposed``
    (``q_t[k][n]``, ``scale_t[k/128][n/128]``: the exact transpose, for Dgrad).
    """
    _need_gpu(w, q, scale, q_t, scale_t)
    _rowmajor(w, "w")
    if w.dtype != torch.bfloat16:
        raise Fp8qError("w must be bfloat16")
    n, k = w.shape
    dev = w.device
    if q is None:
        q = _empty((n, k), torch.float8_e4m3fn, dev, stream)
    if scale is None:
        scale = _empty((n // 128, k // 128), torch.float32, dev, stream)
    _check_tensor(q, (n, k), _CODES, "q")
    _check_tensor(scale, (n // 128, k // 128), _F32, "scale")
    if transposed:
        if q_t is None:
            q_t = _empty((k, n), torch.float8_e4m3fn, dev, stream)
        if scale_t is None:
            scale_t = _empty((k // 128, n // 128), torch.float32, dev, stream)
        _check_tensor(q_t, (k, n), _CODES, "q_t")
        _check_tensor(scale_t, (k // 128, n // 128), _F32, "scale_t")
    st = _load().fp8_quantize_weight(
        _ptr(w), n, k, w.stride(0), _ptr(q), q.stride(0), _ptr(scale), scale.stride(0),
        _ptr(q_t if transposed else None), q_t.stride(0) if transposed else 0,
        _ptr(scale_t if transposed else None), scale_t.stride(0) if transposed else 0,
        _stream(stream))
    _check(st, "fp8_quantize_weight")
    return (q, scale, q_t, scale_t) if transposed else (q, scale)


def fp8_quantize_act_weight(x: torch.Tensor, w: torch.Tensor, transposed: bool = False,
                            q: torch.Tensor | None = None, scale: torch.Tensor | None = None,
                            wq: torch.Tensor | None = None, wscale: torch.Tensor | None = None,
                            wq_t: torch.Tensor | None = None, wscale_t: torch.Tensor | None = None, stream=None):
    """A Linear layer's operands in one launch: ``x`` in 1x128 tiles (as
    :func:`fp8_quantize_act`) and ``w`` in 128x128 blocks (as
    :func:`fp8_quantize_weight`, with the transposed copy when ``transposed``).

    Returns ``(q, scale, wq, wscale)`` or, transposed, ``(q, scale, wq,
    wscale, wq_t, wscale_t)``."""
    _need_gpu(x, w, q, scale, wq, wscale, wq_t, wscale_t)
    _rowmajor(x, "x")
    _rowmajor(w, "w")
    if x.dtype != torch.bfloat16 or w.dtype != torch.bfloat16:
        raise Fp8qError("x and w must be bfloat16")
    rows, cols = x.shape
    n, k = w.shape
    dev = x.device
    if q is None:
        q = _empty((rows, cols), torch.float8_e4m3fn, dev, stream)
    if scale is None:
        scale = _empty((cols // 128, rows), torch.float32, dev, stream)
    if wq is None:
        wq = _empty((n, k), torch.float8_e4m3fn, dev, stream)
    if wscale is None:
        wscale = _empty((n // 128, k // 128), torch.float32, dev, stream)
    _check_tensor(q, (rows, cols), _CODES, "q")
    _check_tensor(scale, (cols // 128, rows), _F32, "scale")
    _check_tensor(wq, (n, k), _CODES, "wq")
    _check_tensor(wscale, (n // 128, k // 128), _F32, "wscale")
    if transposed:
        if wq_t is None:
            wq_t = _empty((k, n), torch.float8_e4m3fn, dev, stream)
        if wscale_t is None:
            wscale_t = _empty((k // 128, n // 128), torch.float32, dev, stream)
        _check_tensor(wq_t, (k, n), _CODES, "wq_t")
        _check_tensor(wscale_t, (k // 128, n // 128), _F32, "wscale_t")
    st = _load().fp8_quantize_act_weight(
        _ptr(x), rows, cols, x.stride(0), _ptr(q), q.stride(0), _ptr(scale), scale.stride(0),
        _ptr(w), n, k, w.stride(0), _ptr(wq), wq.stride(0), _ptr(wscale), wscale.stride(0),
        _ptr(wq_t if transposed else None), wq_t.stride(0) if transposed else 0,
        _ptr(wscale_t if transposed else None), wscale_t.stride(0) if transposed else 0, _stream(stream))
    _check(st, "fp8_quantize_act_weight")
    return (q, scale, wq, wscale, wq_t, wscale_t) if transposed else (q, scale, wq, wscale)


def _outputs_128x1(tokens, c0, c1, dev, stream, q0, scale0, q1, scale1):
    """Outputs of the two 128x1 operands: allocated when absent, checked otherwise."""
    if q0 is None:
        q0 = _empty((c0, tokens), torch.float8_e4m3fn, dev, stream)
    if scale0 is None:
        scale0 = _empty((tokens // 128, c0), torch.float32, dev, stream)
    if q1 is None:
        q1 = _empty((c1, tokens), torch.float8_e4m3fn, dev, stream)
    if scale1 is None:
        scale1 = _empty((tokens // 128, c1), torch.float32, dev, stream)
    _check_tensor(q0, (c0, tokens), _CODES, "q0")
    _check_tensor(scale0, (tokens // 128, c0), _F32, "scale0")
    _check_tensor(q1, (c1, tokens), _CODES, "q1")
    _check_tensor(scale1, (tokens // 128, c1), _F32, "scale1")
    return q0, scale0, q1, scale1


def fp8_quantize_act_128x1_pair(x0: torch.Tensor, x1: torch.Tensor, q0: torch.Tensor | None = None,
                                scale0: torch.Tensor | None = None, q1: torch.Tensor | None = None,
                                scale1: torch.Tensor | None = None, stream=None):
    """The two Wgrad operands (``x0 = dY``, ``x1 = X``, one token count) in
    128x1 token tiles in one launch, as :func:`fp8_quantize_act` with
    ``tiling="128x1"`` on each. Returns ``(q0, scale0, q1, scale1)``."""
    _need_gpu(x0, x1, q0, scale0, q1, scale1)
    _rowmajor(x0, "x0")
    _rowmajor(x1, "x1")
    if x0.dtype != torch.bfloat16 or x1.dtype != torch.bfloat16:
        raise Fp8qError("x0 and x1 must be bfloat16")
    tokens, c0 = x0.shape
    if x1.shape[0] != tokens:
        raise Fp8qError("x0 and x1 must have the same token count")
    c1 = x1.shape[1]
    q0, scale0, q1, scale1 = _outputs_128x1(tokens, c0, c1, x0.device, stream, q0, scale0, q1, scale1)
    st = _load().fp8_quantize_act_128x1_pair(
        tokens, _ptr(x0), c0, x0.stride(0), _ptr(q0), q0.stride(0), _ptr(scale0), scale0.stride(0),
        _ptr(x1), c1, x1.stride(0), _ptr(q1), q1.stride(0), _ptr(scale1), scale1.stride(0), _stream(stream))
    _check(st, "fp8_quantize_act_128x1_pair")
    return q0, scale0, q1, scale1


def fp8_quantize_act_128x1_retile(x0: torch.Tensor, xq: torch.Tensor, xs: torch.Tensor,
                                  q0: torch.Tensor | None = None, scale0: torch.Tensor | None = None,
                                  q1: torch.Tensor | None = None, scale1: torch.Tensor | None = None, stream=None):
    """The two Wgrad operands in one launch when X comes from the FP8 cache:
    ``x0`` (dY, bf16) in 128x1 token tiles as :func:`fp8_quantize_act`, and the
    cached 1x128 codes ``xq[tokens][cols]`` with scales ``xs[cols/128][tokens]``
    re-tiled as :func:`fp8_retile_act_128x1`. Returns ``(q0, scale0, q1, scale1)``."""
    _need_gpu(x0, xq, xs, q0, scale0, q1, scale1)
    _rowmajor(x0, "x0")
    _rowmajor(xq, "xq")
    if x0.dtype != torch.bfloat16:
        raise Fp8qError("x0 must be bfloat16")
    _codes(xq, "xq")
    tokens, c0 = x0.shape
    if xq.shape[0] != tokens:
        raise Fp8qError("x0 and xq must have the same token count")
    c1 = xq.shape[1]
    _check_tensor(xs, (c1 // 128, tokens), _F32, "xs")
    q0, scale0, q1, scale1 = _outputs_128x1(tokens, c0, c1, x0.device, stream, q0, scale0, q1, scale1)
    st = _load().fp8_quantize_act_128x1_retile(
        tokens, _ptr(x0), c0, x0.stride(0), _ptr(q0), q0.stride(0), _ptr(scale0), scale0.stride(0),
        _ptr(xq), c1, xq.stride(0), _ptr(xs), xs.stride(0), _ptr(q1), q1.stride(0), _ptr(scale1),
        scale1.stride(0), _stream(stream))
    _check(st, "fp8_quantize_act_128x1_retile")
    return q0, scale0, q1, scale1


def fp8_quantize_weight_grouped(w: torch.Tensor, transposed: bool = False, q: torch.Tensor | None = None,
                                scale: torch.Tensor | None = None, q_t: torch.Tensor | None = None,
                                scale_t: torch.Tensor | None = None, stream=None):
    """Quantize ``E`` bf16 weights ``w[E][n][k]`` (say the experts of an MoE
    layer) in 128x128 blocks with one launch.

    Returns ``(q[E][n][k], scale[E][n/128][k/128])``, or with ``transposed``
    also ``q_t[E][k][n]`` and ``scale_t[E][k/128][n/128]`` (each expert's exact
    transpose, contiguous per expert, for Dgrad).
    """
    _need_gpu(w, q, scale, q_t, scale_t)
    if w.dtype != torch.bfloat16:
        raise Fp8qError("w must be bfloat16")
    if w.dim() != 3 or w.stride(2) != 1:
        raise Fp8qError("w must be [E][n][k] with k contiguous")
    groups, n, k = w.shape
    dev = w.device
    if q is None:
        q = _empty((groups, n, k), torch.float8_e4m3fn, dev, stream)
    if scale is None:
        scale = _empty((groups, n // 128, k // 128), torch.float32, dev, stream)
    _check_tensor(q, (groups, n, k), _CODES, "q")
    _check_tensor(scale, (groups, n // 128, k // 128), _F32, "scale")
    if transposed:
        if q_t is None:
            q_t = _empty((groups, k, n), torch.float8_e4m3fn, dev, stream)
        if scale_t is None:
            scale_t = _empty((groups, k // 128, n // 128), torch.float32, dev, stream)
        _check_tensor(q_t, (groups, k, n), _CODES, "q_t")
        _check_tensor(scale_t, (groups, k // 128, n // 128), _F32, "scale_t")
    st = _load().fp8_quantize_weight_grouped(
        groups, _ptr(w), n, k, w.stride(1), w.stride(0),
        _ptr(q), q.stride(1), q.stride(0), _ptr(scale), scale.stride(1), scale.stride(0),
        _ptr(q_t if transposed else None), q_t.stride(1) if transposed else 0,
        q_t.stride(0) if transposed else 0,
        _ptr(scale_t if transposed else None), scale_t.stride(1) if transposed else 0,
        scale_t.stride(0) if transposed else 0, _stream(stream))
    _check(st, "fp8_quantize_weight_grouped")
    return (q, scale, q_t, scale_t) if transposed else (q, scale)


# --------------------------------------------------------------------- GEMM

def _out_code(out_dtype) -> int:
    if out_dtype == torch.bfloat16:
        return OUT_BF16
    if out_dtype == torch.float32:
        return OUT_F32
    raise Fp8qError("out_dtype must be torch.bfloat16 or torch.float32")


def _gemm_out(out, shape, out_dtype, dev, stream):
    """The GEMM output: allocated when absent; otherwise its dtype must be
    ``out_dtype`` (the kernels write elements of that size) and its shape
    exactly ``shape``, with unit column stride."""
    if out is None:
        out = _empty(shape, out_dtype, dev, stream)
    _check_tensor(out, shape, (out_dtype,), "out")
    return out


def fp8_gemm(a: torch.Tensor, a_scale: torch.Tensor, b: torch.Tensor, b_scale: torch.Tensor,
             b_scale_kind: str = "block", out_dtype=torch.bfloat16, out: torch.Tensor | None = None,
             stream=None) -> torch.Tensor:
    """``C[m][n] = sum_k deq(A)[m][k] deq(B)[n][k]`` with per-128-slab promotion.

    ``a[m][k]`` codes with ``a_scale[k/128][m]``; ``b[n][k]`` codes with
    ``b_scale[ceil(n/128)][k/128]`` (``"block"``) or ``b_scale[k/128][n]`` (``"row"``).
    """
    _need_gpu(a, a_scale, b, b_scale, out)
    _rowmajor(a, "a")
    _rowmajor(b, "b")
    _codes(a, "a")
    _codes(b, "b")
    m, k = a.shape
    n, kb = b.shape
    if kb != k:
        raise Fp8qError("a and b disagree on K (%d vs %d)" % (k, kb))
    kind = {"block": BSCALE_BLOCK128, "row": BSCALE_ROW128}.get(b_scale_kind)
    if kind is None:
        raise Fp8qError("b_scale_kind must be 'block' or 'row'")
    oc = _out_code(out_dtype)
    _check_tensor(a_scale, (k // 128, m), _F32, "a_scale")
    _check_tensor(b_scale, ((n + 127) // 128, k // 128) if kind == BSCALE_BLOCK128 else (k // 128, n),
                  _F32, "b_scale")
    out = _gemm_out(out, (m, n), out_dtype, a.device, stream)
    st = _load().fp8_gemm(m, n, k, _ptr(a), a.stride(0), _ptr(a_scale), a_scale.stride(0),
                          _ptr(b), b.stride(0), _ptr(b_scale), b_scale.stride(0), kind,
                          _ptr(out), out.stride(0), oc, _stream(stream))
    _check(st, "fp8_gemm")
    return out


def _grouped_gemm_args(group_offsets, group_rows, a, a_scale, b, b_scale, out_dtype, out, stream):
    """Checked arguments of the grouped Fprop GEMM entry points, up to out_dtype."""
    _need_gpu(group_offsets, group_rows, a, a_scale, b, b_scale, out)
    _rowmajor(a, "a")
    _codes(a, "a")
    _codes(b, "b")
    if group_offsets.dtype != torch.int32 or (group_rows is not None and group_rows.dtype != torch.int32):
        raise Fp8qError("group_offsets / group_rows must be int32")
    if b.dim() != 3 or b.stride(2) != 1:
        raise Fp8qError("b must be [E][n][k] with k contiguous")
    groups = b.shape[0]
    if group_offsets.dim() != 1 or group_offsets.numel() != groups + 1 or not group_offsets.is_contiguous():
        raise Fp8qError("group_offsets needs E+1 contiguous entries")
    if group_rows is not None and (group_rows.numel() != groups or not group_rows.is_contiguous()):
        raise Fp8qError("group_rows needs E contiguous entries")
    m_total, k = a.shape
    n = b.shape[1]
    if b.shape[2] != k:
        raise Fp8qError("a and b disagree on K (%d vs %d)" % (k, b.shape[2]))
    oc = _out_code(out_dtype)
    _check_tensor(a_scale, (k // 128, m_total), _F32, "a_scale")
    _check_tensor(b_scale, (groups, n // 128, k // 128), _F32, "b_scale")
    out = _gemm_out(out, (m_total, n), out_dtype, a.device, stream)
    args = (groups, _ptr(group_offsets), _ptr(group_rows), m_total, n, k,
            _ptr(a), a.stride(0), _ptr(a_scale), a_scale.stride(0),
            _ptr(b), b.stride(1), b.stride(0), _ptr(b_scale), b_scale.stride(1), b_scale.stride(0),
            _ptr(out), out.stride(0), oc)
    return args, out


def fp8_grouped_gemm(group_offsets: torch.Tensor, group_rows: torch.Tensor | None,
                     a: torch.Tensor, a_scale: torch.Tensor, b: torch.Tensor, b_scale: torch.Tensor,
                     out_dtype=torch.bfloat16, out: torch.Tensor | None = None,
                     stream=None, workspace: torch.Tensor | None = None) -> torch.Tensor:
    """MoE expert Fprop: rows ``[off[e], off[e+1])`` of ``a`` times ``W_e = b[e]``.

    ``group_offsets``: int32 GPU tensor ``[E+1]`` (multiples of 128);
    ``group_rows``: int32 GPU tensor ``[E]`` of real rows, or None; padding rows
    of the output are zero. ``b[E][n][k]`` codes, ``b_scale[E][n/128][k/128]``.
    ``workspace``: a contiguous uint8 GPU tensor for the K-split of a partial
    last round of tiles (``GROUPED_WORKSPACE_BYTES`` allow every split; an
    empty one turns the split off); None takes one from torch's allocator on
    the output's stream.
    """
    args, out = _grouped_gemm_args(group_offsets, group_rows, a, a_scale, b, b_scale, out_dtype, out, stream)
    if workspace is None:
        workspace = _empty((GROUPED_WORKSPACE_BYTES,), torch.uint8, a.device, stream)
    _need_gpu(workspace)
    if workspace.dtype != torch.uint8 or not workspace.is_contiguous():
        raise Fp8qError("workspace must be a contiguous uint8 tensor")
    st = _load().fp8_grouped_gemm(*args, _ptr(workspace) if workspace.numel() else None, workspace.numel(),
                                  _stream(stream))
    _check(st, "fp8_grouped_gemm")
    return out


def fp8_grouped_gemm_noalloc(group_offsets: torch.Tensor, group_rows: torch.Tensor | None,
                             a: torch.Tensor, a_scale: torch.Tensor, b: torch.Tensor, b_scale: torch.Tensor,
                             out_dtype=torch.bfloat16, out: torch.Tensor | None = None,
                             stream=None) -> torch.Tensor:
    """``fp8_grouped_gemm`` on the library's own per-GPU scratch: the C call
    allocates nothing (pass ``out`` to keep this wrapper from allocating it).
    Calls that overlap in time on one GPU share the scratch and race."""
    args, out = _grouped_gemm_args(group_offsets, group_rows, a, a_scale, b, b_scale, out_dtype, out, stream)
    st = _load().fp8_grouped_gemm_noalloc(*args, _stream(stream))
    _check(st, "fp8_grouped_gemm_noalloc")
    return out


def fp8_grouped_gemm_wgrad(group_offsets: torch.Tensor, a: torch.Tensor, a_scale: torch.Tensor,
                           b: torch.Tensor, b_scale: torch.Tensor, out_dtype=torch.float32,
                           out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """MoE expert Wgrad: ``out[e] = sum over e's tokens t of A[:, t] B[:, t]^T``.

    ``a``: dY^T codes ``[m][k_total]`` and ``a_scale[k_total/128][m]`` (from
    ``fp8_quantize_act(dY, "128x1")`` on the expert-sorted layout); ``b``: X^T
    codes ``[n][k_total]``, ``b_scale[k_total/128][n]``; ``group_offsets``:
    int32 GPU tensor ``[E+1]`` of token offsets (multiples of 128). Returns
    ``out[E][m][n]``.
    """
    _need_gpu(group_offsets, a, a_scale, b, b_scale, out)
    _rowmajor(a, "a")
    _rowmajor(b, "b")
    _codes(a, "a")
    _codes(b, "b")
    if group_offsets.dtype != torch.int32 or group_offsets.dim() != 1 or not group_offsets.is_contiguous():
        raise Fp8qError("group_offsets must be a contiguous 1-D int32 tensor")
    groups = group_offsets.numel() - 1
    m, k_total = a.shape
    n = b.shape[0]
    if b.shape[1] != k_total:
        raise Fp8qError("a and b must cover the same tokens")
    oc = _out_code(out_dtype)
    _check_tensor(a_scale, (k_total // 128, m), _F32, "a_scale")
    _check_tensor(b_scale, (k_total // 128, n), _F32, "b_scale")
    out = _gemm_out(out, (groups, m, n), out_dtype, a.device, stream)
    st = _load().fp8_grouped_gemm_wgrad(
        groups, _ptr(group_offsets), k_total, m, n,
        _ptr(a), a.stride(0), _ptr(a_scale), a_scale.stride(0),
        _ptr(b), b.stride(0), _ptr(b_scale), b_scale.stride(0),
        _ptr(out), out.stride(1), out.stride(0), oc, _stream(stream))
    _check(st, "fp8_grouped_gemm_wgrad")
    return out


# ------------------------------------------------------------- microscaling

_WORDS = (torch.int32, torch.uint32) if hasattr(torch, "uint32") else (torch.int32,)


def fp8_quantize_mx(x: torch.Tensor, q: torch.Tensor | None = None, scale: torch.Tensor | None = None,
                    stream=None):
    """Microscaling quantization (32-element blocks along each row, E8M0
    power-of-two scales, E4M3 codes). Returns ``q[rows][cols]`` and the scale
    words ``scale[cols/128][rows]`` (int32 tensor of 4 E8M0 bytes each)."""
    _need_gpu(x, q, scale)
    _rowmajor(x, "x")
    if x.dtype != torch.bfloat16:
        raise Fp8qError("x must be bfloat16")
    rows, cols = x.shape
    if q is None:
        q = _empty((rows, cols), torch.float8_e4m3fn, x.device, stream)
    if scale is None:
        scale = _empty((cols // 128, rows), torch.int32, x.device, stream)
    _check_tensor(q, (rows, cols), _CODES, "q")
    _check_tensor(scale, (cols // 128, rows), _WORDS, "scale")
    st = _load().fp8_quantize_mx(_ptr(x), rows, cols, x.stride(0), _ptr(q), q.stride(0), _ptr(scale),
                                 scale.stride(0), _stream(stream))
    _check(st, "fp8_quantize_mx")
    return q, scale


def fp8_quantize_mx_pair(x0: torch.Tensor, x1: torch.Tensor, q0: torch.Tensor | None = None,
                         scale0: torch.Tensor | None = None, q1: torch.Tensor | None = None,
                         scale1: torch.Tensor | None = None, stream=None):
    """Both operands of the microscaling GEMM in one launch, as
    :func:`fp8_quantize_mx` on each. Returns ``(q0, scale0, q1, scale1)``."""
    _need_gpu(x0, x1, q0, scale0, q1, scale1)
    _rowmajor(x0, "x0")
    _rowmajor(x1, "x1")
    if x0.dtype != torch.bfloat16 or x1.dtype != torch.bfloat16:
        raise Fp8qError("x0 and x1 must be bfloat16")
    (r0, c0), (r1, c1) = x0.shape, x1.shape
    dev = x0.device
    if q0 is None:
        q0 = _empty((r0, c0), torch.float8_e4m3fn, dev, stream)
    if scale0 is None:
        scale0 = _empty((c0 // 128, r0), torch.int32, dev, stream)
    if q1 is None:
        q1 = _empty((r1, c1), torch.float8_e4m3fn, dev, stream)
    if scale1 is None:
        scale1 = _empty((c1 // 128, r1), torch.int32, dev, stream)
    _check_tensor(q0, (r0, c0), _CODES, "q0")
    _check_tensor(scale0, (c0 // 128, r0), _WORDS, "scale0")
    _check_tensor(q1, (r1, c1), _CODES, "q1")
    _check_tensor(scale1, (c1 // 128, r1), _WORDS, "scale1")
    st = _load().fp8_quantize_mx_pair(
        _ptr(x0), r0, c0, x0.stride(0), _ptr(q0), q0.stride(0), _ptr(scale0), scale0.stride(0),
        _ptr(x1), r1, c1, x1.stride(0), _ptr(q1), q1.stride(0), _ptr(scale1), scale1.stride(0), _stream(stream))
    _check(st, "fp8_quantize_mx_pair")
    return q0, scale0, q1, scale1


def fp8_gemm_mx(a: torch.Tensor, a_scale: torch.Tensor, b: torch.Tensor, b_scale: torch.Tensor,
                out_dtype=torch.bfloat16, out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """``C = dequant_mx(A) @ dequant_mx(B)^T`` with both operands from
    :func:`fp8_quantize_mx` along K."""
    _need_gpu(a, a_scale, b, b_scale, out)
    _rowmajor(a, "a")
    _rowmajor(b, "b")
    _codes(a, "a")
    _codes(b, "b")
    m, k = a.shape
    n, kb = b.shape
    if kb != k:
        raise Fp8qError("a and b disagree on K (%d vs %d)" % (k, kb))
    oc = _out_code(out_dtype)
    _check_tensor(a_scale, (k // 128, m), _WORDS, "a_scale")
    _check_tensor(b_scale, (k // 128, n), _WORDS, "b_scale")
    out = _gemm_out(out, (m, n), out_dtype, a.device, stream)
    st = _load().fp8_gemm_mx(m, n, k, _ptr(a), a.stride(0), _ptr(a_scale), a_scale.stride(0),
                             _ptr(b), b.stride(0), _ptr(b_scale), b_scale.stride(0),
                             _ptr(out), out.stride(0), oc, _stream(stream))
    _check(st, "fp8_gemm_mx")
    return out


def fp8_retile_act_128x1(q: torch.Tensor, scale: torch.Tensor, q_t: torch.Tensor | None = None,
                         scale_t: torch.Tensor | None = None, stream=None):
    """Cached 1x128 FP8 activation (codes ``q[tokens][cols]``, scales
    ``scale[cols/128][tokens]``) -> 128x1 token tiles for Wgrad: codes
    ``q_t[cols][tokens]`` and scales ``scale_t[tokens/128][cols]``."""
    _need_gpu(q, scale, q_t, scale_t)
    _rowmajor(q, "q")
    _codes(q, "q")
    tokens, cols = q.shape
    _check_tensor(scale, (cols // 128, tokens), _F32, "scale")
    if q_t is None:
        q_t = _empty((cols, tokens), torch.float8_e4m3fn, q.device, stream)
    if scale_t is None:
        scale_t = _empty((tokens // 128, cols), torch.float32, q.device, stream)
    _check_tensor(q_t, (cols, tokens), _CODES, "q_t")
    _check_tensor(scale_t, (tokens // 128, cols), _F32, "scale_t")
    st = _load().fp8_retile_act_128x1(_ptr(q), tokens, cols, q.stride(0), _ptr(scale), scale.stride(0),
                                      _ptr(q_t), q_t.stride(0), _ptr(scale_t), scale_t.stride(0),
                                      _stream(stream))
    _check(st, "fp8_retile_act_128x1")
    return q_t, scale_t


def fp8_gemm_tensor(a: torch.Tensor, a_scale: torch.Tensor, b: torch.Tensor, b_scale: torch.Tensor,
                    out_dtype=torch.bfloat16, out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """``C = sA * sB * sum_k dec(A)[m][k] dec(B)[n][k]`` with one scale per
    operand (one-element float32 tensors) and the whole K sum accumulated in
    the MFMA accumulators (no per-slab promotion)."""
    _need_gpu(a, a_scale, b, b_scale, out)
    _rowmajor(a, "a")
    _rowmajor(b, "b")
    _codes(a, "a")
    _codes(b, "b")
    m, k = a.shape
    n, kb = b.shape
    if kb != k:
        raise Fp8qError("a and b disagree on K (%d vs %d)" % (k, kb))
    if a_scale.dtype != torch.float32 or b_scale.dtype != torch.float32:
        raise Fp8qError("scales must be float32")
    if a_scale.numel() != 1 or b_scale.numel() != 1:
        raise Fp8qError("per-tensor scales hold one element each")
    oc = _out_code(out_dtype)
    out = _gemm_out(out, (m, n), out_dtype, a.device, stream)
    st = _load().fp8_gemm_tensor(m, n, k, _ptr(a), a.stride(0), _ptr(a_scale), _ptr(b), b.stride(0),
                                 _ptr(b_scale), _ptr(out), out.stride(0), oc, _stream(stream))
    _check(st, "fp8_gemm_tensor")
    return out
