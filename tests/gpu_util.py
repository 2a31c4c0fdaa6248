"""Helpers for the GPU parity tests: host <-> device marshalling and the pass
criteria. Inputs come from ``workloads`` (seeded), expected values from
``oracle`` only."""
from __future__ import annotations

import numpy as np
import torch

NORM_TOL = 2e-3       # normwise ||C - ref||_F / ||ref||_F
ELEM_TOL = 1e-2       # |C - ref| <= ELEM_TOL * (|ref| + rms(ref)) element-wise


def dev_bf16(bits: np.ndarray) -> torch.Tensor:
    """bf16 bit array (uint16) -> bf16 GPU tensor with the same bits."""
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.view(torch.bfloat16).cuda()


def dev_codes(q: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(q)).cuda()


def dev_f32(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()


def host_codes(t: torch.Tensor) -> np.ndarray:
    return t.view(torch.uint8).cpu().numpy()


def host_f32(t: torch.Tensor) -> np.ndarray:
    return t.float().cpu().numpy()


def host_out(t: torch.Tensor) -> np.ndarray:
    """GEMM output (bf16 or fp32) as float64."""
    return t.float().cpu().numpy().astype(np.float64)


def assert_bits_equal(got: np.ndarray, ref: np.ndarray, what: str) -> None:
    got = np.asarray(got)
    ref = np.asarray(ref)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    if got.dtype == np.float32:
        got, ref = got.view(np.uint32), ref.view(np.uint32)
    bad = np.nonzero(got != ref)
    if len(bad[0]):
        idx = tuple(b[:5] for b in bad)
        raise AssertionError("%s: %d mismatches, first at %s: got %s ref %s" % (
            what, len(bad[0]), [tuple(int(x) for x in i) for i in zip(*idx)],
            got[idx], ref[idx]))


def gemm_errors(got: np.ndarray, ref: np.ndarray) -> dict:
    """The pass metrics against the unrounded float64 oracle, plus (a
    diagnostic only) the normwise error against the oracle rounded to bf16
    nearest-even: for bf16 output that isolates the GEMM's own error."""
    import oracle
    diff = got - ref
    rms = float(np.sqrt(np.mean(ref * ref))) if ref.size else 0.0
    norm_ref = float(np.linalg.norm(ref))
    normwise = float(np.linalg.norm(diff)) / norm_ref if norm_ref > 0 else float(np.linalg.norm(diff))
    bound = ELEM_TOL * (np.abs(ref) + rms)
    worst = float(np.max(np.abs(diff) / np.where(bound > 0, bound, 1.0))) if ref.size else 0.0
    diff16 = got - oracle.bf16_round(ref)
    normwise16 = float(np.linalg.norm(diff16)) / norm_ref if norm_ref > 0 else float(np.linalg.norm(diff16))
    return {"normwise": normwise, "worst_elem_ratio": worst, "rms_ref": rms,
            "normwise_vs_bf16_rounded_ref": normwise16}


def assert_gemm_close(got: np.ndarray, ref: np.ndarray, what: str) -> dict:
    """The pass criteria against the unrounded float64 oracle."""
    e = gemm_errors(got, ref)
    assert np.all(np.isfinite(got)), what + ": non-finite output"
    assert e["normwise"] <= NORM_TOL, "%s: normwise %.3e > %.1e" % (what, e["normwise"], NORM_TOL)
    assert e["worst_elem_ratio"] <= 1.0, "%s: element error %.3f x bound" % (what, e["worst_elem_ratio"])
    return e


def nan_out(shape, dtype) -> torch.Tensor:
    """A GEMM output buffer filled with NaN: an element the kernel leaves
    unwritten stays NaN and fails the finiteness check."""
    return torch.full(shape, float("nan"), dtype=dtype, device="cuda")


def assert_grouped_close(got: np.ndarray, ref: np.ndarray, offsets, rows, what: str) -> dict:
    """Grouped output [m_total][n]: every real row of every expert against the
    oracle, with rms(ref) taken over all real rows together (the compared
    output); every padding row exactly zero; nothing non-finite anywhere."""
    assert np.all(np.isfinite(got)), what + ": non-finite output (an unwritten tile?)"
    real = np.concatenate([np.arange(int(offsets[e]), int(offsets[e]) + int(rows[e]))
                           for e in range(len(rows))] + [np.zeros(0, np.int64)]).astype(np.int64)
    pad = np.setdiff1d(np.arange(got.shape[0]), real)
    assert np.all(got[pad] == 0), what + ": padding rows not zero"
    if real.size == 0:
        return {}
    return assert_gemm_close(got[real], ref[real], what)


_CACHE: dict = {}


def cached(key, fn):
    """Memoize an expensive oracle result (say the 32 expert weights'
    quantization) across the tests of one process."""
    if key not in _CACHE:
        _CACHE[key] = fn()
    return _CACHE[key]
