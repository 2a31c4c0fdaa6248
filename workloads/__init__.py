"""Seeded synthetic inputs for the fine-grained FP8 GEMM path.

This module is shared by the tests, the benchmark and the smoke check. It only
draws random numbers and rounds them to bf16 inputs; it holds none of the
method's arithmetic (no scales, no FP8 encoding, no GEMM), so neither the CPU
oracle nor the GPU library depends on the other through it.

Recipe (the pages describe DeepSeek-V3 training traffic, which is not
available; these shapes and distributions stand in for it):

* every tensor is drawn in float32 from its own stream,
  ``np.random.default_rng(SeedSequence([seed, config_id, tensor_id]))``, then
  rounded to bf16 with round-to-nearest-even;
* ``N(0, sigma)`` means standard deviation ``sigma``;
* "0.1% outliers xF": each entry independently (Bernoulli(0.001)) has its
  value multiplied by F;
* Dgrad's dY is ``1e-3 * z * m_row`` with ``z ~ N(0,1)`` and one
  ``m_row ~ lognormal(0, 1)`` per row;
* grouped MoE routing: Zipf(1.1) popularity over the 32 local experts,
  ``rows = multinomial(8192, p[permutation])`` from ``default_rng(seed)``, each
  expert's segment padded up to a multiple of 128 with zero rows.

All arrays are returned as numpy ``uint16`` bf16 bit patterns (row-major).
"""
from __future__ import annotations

import numpy as np

CONFIG_IDS = {
    "tiny_fprop": 0,
    "dense_fprop": 1,
    "dgrad": 2,
    "wgrad": 3,
    "grouped_fprop": 4,
}


def _rng(seed: int, config: str, tensor_id: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([seed, CONFIG_IDS[config], tensor_id]))


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round finite float32 values to bf16 (nearest, ties to even); return the bits."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    rounded = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return rounded.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to float32 (exact)."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _normal(rng: np.random.Generator, shape, std: float) -> np.ndarray:
    out = rng.standard_normal(shape, dtype=np.float32)
    if std != 1.0:
        out *= np.float32(std)
    return out


def _with_outliers(rng: np.random.Generator, a: np.ndarray, factor: float, frac: float = 1e-3) -> np.ndarray:
    mask = rng.random(a.shape, dtype=np.float32) < np.float32(frac)
    a[mask] *= np.float32(factor)
    return a


def activation(seed: int, config: str, tensor_id: int, rows: int, cols: int,
               outlier_factor: float | None) -> np.ndarray:
    """``N(0,1)`` activations with optional 0.1% outliers, as bf16 bits."""
    rng = _rng(seed, config, tensor_id)
    a = _normal(rng, (rows, cols), 1.0)
    if outlier_factor is not None:
        a = _with_outliers(rng, a, outlier_factor)
    return f32_to_bf16_bits(a)


def weight(seed: int, config: str, tensor_id: int, *shape: int, std: float = 0.02) -> np.ndarray:
    """``N(0, std)`` weights as bf16 bits."""
    return f32_to_bf16_bits(_normal(_rng(seed, config, tensor_id), shape, std))


def grad_rowscaled(seed: int, config: str, tensor_id: int, rows: int, cols: int,
                   std: float = 1e-3) -> np.ndarray:
    """Output gradient ``std * z * m_row`` with per-row lognormal(0,1) magnitude."""
    rng = _rng(seed, config, tensor_id)
    z = _normal(rng, (rows, cols), 1.0)
    m = rng.lognormal(0.0, 1.0, size=(rows, 1)).astype(np.float32)
    return f32_to_bf16_bits(z * (np.float32(std) * m))


def moe_rows(seed: int = 0, tokens: int = 8192, top_k: int = 8, experts_total: int = 256,
             experts_local: int = 32, zipf_a: float = 1.1) -> np.ndarray:
    """Rows routed to each local expert (int64[experts_local], sums to the local share).

    The local share is tokens * top_k * experts_local / experts_total (8192 for
    8192 tokens, top-8, 32 of 256 experts); popularity is Zipf(zipf_a) over
    the local experts in a random order.
    """
    rng = np.random.default_rng(seed)
    ranks = np.arange(1, experts_local + 1, dtype=np.float64)
    p = ranks ** (-zipf_a)
    p /= p.sum()
    perm = rng.permutation(experts_local)
    share = tokens * top_k * experts_local // experts_total
    return rng.multinomial(share, p[perm]).astype(np.int64)


def pad_offsets(rows: np.ndarray, align: int = 128) -> np.ndarray:
    """Segment starts of the expert-sorted layout, each segment padded to ``align``."""
    padded = (np.asarray(rows, dtype=np.int64) + align - 1) // align * align
    return np.concatenate([[0], np.cumsum(padded)]).astype(np.int64)


def tiny_fprop(seed: int = 0) -> dict:
    """X 128x512 N(0,1) with 0.1% x100 outliers; W 256x512 N(0,0.02)."""
    return {
        "x": activation(seed, "tiny_fprop", 0, 128, 512, 100.0),
        "w": weight(seed, "tiny_fprop", 1, 256, 512),
    }


def dense_fprop(seed: int = 0, m: int = 4096, n: int = 4096, k: int = 7168) -> dict:
    """X MxK N(0,1) with 0.1% x50 outliers; W NxK N(0,0.02) (gate+up of a 2048-wide expert FFN)."""
    return {
        "x": activation(seed, "dense_fprop", 0, m, k, 50.0),
        "w": weight(seed, "dense_fprop", 1, n, k),
    }


def dgrad(seed: int = 0, m: int = 4096, n_out: int = 2048, k_in: int = 7168) -> dict:
    """dY [m][n_out] = 1e-3 * z * lognormal row magnitude; W [n_out][k_in] N(0,0.02)."""
    return {
        "dy": grad_rowscaled(seed, "dgrad", 0, m, n_out),
        "w": weight(seed, "dgrad", 1, n_out, k_in),
    }


def wgrad(seed: int = 0, tokens: int = 8192, n_out: int = 2048, k_in: int = 7168) -> dict:
    """dY [tokens][n_out] N(0,1e-3); X [tokens][k_in] N(0,1) with 0.1% x50 outliers."""
    rng = _rng(seed, "wgrad", 0)
    dy = f32_to_bf16_bits(_normal(rng, (tokens, n_out), 1e-3))
    return {
        "dy": dy,
        "x": activation(seed, "wgrad", 1, tokens, k_in, 50.0),
    }


def grouped_fprop(seed: int = 0, n: int = 4096, k: int = 7168, experts: int = 32,
                  rows: np.ndarray | None = None, with_weights: bool = True) -> dict:
    """Expert-sorted, 128-padded X [m_total][k] (padding rows are zero) and W [experts][n][k]."""
    if rows is None:
        rows = moe_rows(seed, experts_local=experts)
    rows = np.asarray(rows, dtype=np.int64)
    offsets = pad_offsets(rows)
    m_total = int(offsets[-1])
    x_real = activation(seed, "grouped_fprop", 0, int(rows.sum()), k, 50.0)
    x = np.zeros((m_total, k), dtype=np.uint16)
    src = 0
    for e in range(len(rows)):
        r = int(rows[e])
        x[offsets[e]:offsets[e] + r] = x_real[src:src + r]
        src += r
    out = {"x": x, "rows": rows, "offsets": offsets}
    if with_weights:
        out["w"] = weight(seed, "grouped_fprop", 1, len(rows), n, k)
    return out


def moe_dispatch(seed: int = 0, k: int = 7168, tokens: int = 8192, top_k: int = 8,
                 rows: np.ndarray | None = None) -> dict:
    """Token activations and their routes into the expert-sorted layout.

    Expert e's rows (moe_rows) are r_e distinct tokens drawn uniformly without
    replacement, kept in token order inside the expert's 128-padded segment.
    dst_rows[t] lists token t's destination rows in increasing expert order,
    -1 past its last route; a draw that gives some token more than top_k
    routes is redrawn (next stream of the same seed).
    """
    if rows is None:
        rows = moe_rows(seed, tokens=tokens, top_k=top_k)
    rows = np.asarray(rows, dtype=np.int64)
    offsets = pad_offsets(rows)
    for attempt in range(64):
        rng = _rng(seed, "grouped_fprop", 3 + attempt)
        dst = np.full((tokens, top_k), -1, dtype=np.int32)
        fill = np.zeros(tokens, dtype=np.int64)
        ok = True
        for e in range(len(rows)):
            toks = np.sort(rng.choice(tokens, size=int(rows[e]), replace=False))
            if np.any(fill[toks] >= top_k):
                ok = False
                break
            dst[toks, fill[toks]] = offsets[e] + np.arange(len(toks), dtype=np.int64)
            fill[toks] += 1
        if ok:
            break
    else:  # pragma: no cover - needs an absurd routing skew
        raise RuntimeError("no routing with at most top_k routes per token")
    x = activation(seed, "grouped_fprop", 2, tokens, k, 50.0)
    return {"x": x, "dst_rows": dst, "rows": rows, "offsets": offsets}
