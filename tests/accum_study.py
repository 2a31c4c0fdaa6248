"""Accumulation study: what a whole K = 4096 FP8 GEMM loses when its sum stays
inside the MFMA accumulators, against promoting every 128-element slab into
FP32 registers (page "Eliminate Deepseek Ai News For Good", passage on
limited accumulation precision: on H800 tensor cores, a K = 4096 GEMM of
random matrices reached a maximum relative error near 2%).

Inputs: two random matrices, A [M][K] and B [N][K], seeded bf16 from
``workloads`` (normal, or the magnitudes of normal values for the
all-positive case, where every partial sum grows), quantized to E4M3 by the
oracle in 1x128 tiles. The study multiplies the codes with unit scales, so
every arm approximates the same exact sum E = sum_k dec(a) dec(b), which
``oracle.gemm_tensor`` gives exactly in float64.

Arms, all with FP32 output:
  mfma_chain         fp8_gemm_tensor: the MFMA accumulates over all of K;
  mfma_scaled_chain  fp8_gemm_mx with every E8M0 byte 127 (2^0): the scaled
                     MFMA, accumulating over all of K;
  slab_promotion     fp8_gemm with all scales 1: each slab's MFMA result is
                     added into FP32 by a VALU FMA;
  rn32_exact         fl32(E), the best any FP32 output can do;
  fp32_sequential    (CPU, sampled rows) the products added one by one, in K
                     order, into an FP32 accumulator rounded to nearest after
                     every addition: what an exact-product FP32 accumulator
                     would give.

Metrics per arm:
  normwise    ||C - E||_F / ||E||_F;
  max_rel     max |C - E| / |E| over entries with E != 0 (the pages' metric,
              read literally; entries near zero dominate it);
  max_rel_cond  the same over entries with |E| >= rms(E);
  max_err_over_max  max |C - E| / max |E|;
  ulp_max     max |C - rn32(E)| in units of the FP32 ulp of rn32(E).

Run as a script on a GPU for the table; ``tests/test_gpu_accum.py`` calls
:func:`run` with its bounds.
"""
from __future__ import annotations

import json
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(HERE))
sys.path.insert(0, HERE)


def make_codes(m: int, n: int, k: int, positive: bool, seed: int = 0):
    """E4M3 codes of two seeded random matrices (oracle 1x128 quantization)."""
    import oracle
    import workloads as wl
    a = wl.activation(seed, "wgrad", 101, m, k, 0.0)
    b = wl.activation(seed, "wgrad", 102, n, k, 0.0)
    if positive:
        a, b = a & np.uint16(0x7FFF), b & np.uint16(0x7FFF)
    return oracle.quant_act_1x128(a)[0], oracle.quant_act_1x128(b)[0]


def metrics(c: np.ndarray, exact: np.ndarray) -> dict:
    err = c.astype(np.float64) - exact
    nz = exact != 0
    rms = float(np.sqrt(np.mean(exact * exact)))
    cond = np.abs(exact) >= rms
    r32 = exact.astype(np.float32)
    ulp = np.spacing(np.abs(r32)).astype(np.float64)
    return {
        "normwise": float(np.linalg.norm(err) / np.linalg.norm(exact)),
        "max_rel": float(np.max(np.abs(err[nz]) / np.abs(exact[nz]))),
        "max_rel_cond": float(np.max(np.abs(err[cond]) / np.abs(exact[cond]))),
        "max_err_over_max": float(np.max(np.abs(err)) / np.max(np.abs(exact))),
        "ulp_max": float(np.max(np.abs(c.astype(np.float64) - r32.astype(np.float64)) / ulp)),
    }


def run(m: int = 2048, n: int = 2048, k: int = 4096, positive: bool = False, time_iters: int = 0) -> dict:
    """Run the three GPU arms on one pair of random code matrices and return
    the metrics (and, with time_iters, each arm's mean kernel time in ms)."""
    import torch

    import fine_grained_fp8_quantize_amd as fq
    import oracle

    qa, qb = make_codes(m, n, k, positive)
    exact = oracle.gemm_tensor(qa, 1.0, qb, 1.0)
    dev = "cuda"
    A = torch.from_numpy(qa).to(dev)
    B = torch.from_numpy(qb).to(dev)
    one = torch.ones(1, dtype=torch.float32, device=dev)
    ones_a = torch.ones((k // 128, m), dtype=torch.float32, device=dev)
    ones_b = torch.ones((n // 128, k // 128), dtype=torch.float32, device=dev)
    e8_a = torch.full((k // 128, m), 0x7F7F7F7F, dtype=torch.int32, device=dev)
    e8_b = torch.full((k // 128, n), 0x7F7F7F7F, dtype=torch.int32, device=dev)
    out = torch.empty((m, n), dtype=torch.float32, device=dev)
    arms = {
        "mfma_chain": lambda: fq.fp8_gemm_tensor(A, one, B, one, torch.float32, out=out),
        "mfma_scaled_chain": lambda: fq.fp8_gemm_mx(A, e8_a, B, e8_b, torch.float32, out=out),
        "slab_promotion": lambda: fq.fp8_gemm(A, ones_a, B, ones_b, "block", torch.float32, out=out),
    }
    res = {"shape": [m, n, k], "inputs": "positive" if positive else "normal",
           "rms_exact": float(np.sqrt(np.mean(exact * exact))), "arms": {}}
    for name, fn in arms.items():
        out.fill_(float("nan"))
        fn()
        torch.cuda.synchronize()
        ent = metrics(out.cpu().numpy(), exact)
        if time_iters:
            ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            for _ in range(3):
                fn()
            ev0.record()
            for _ in range(time_iters):
                fn()
            ev1.record()
            torch.cuda.synchronize()
            ms = ev0.elapsed_time(ev1) / time_iters
            ent["ms"] = round(ms, 4)
            ent["tflops"] = round(2.0 * m * n * k / (ms * 1e-3) / 1e12, 1)
        res["arms"][name] = ent
    res["arms"]["rn32_exact"] = metrics(exact.astype(np.float32), exact)
    rows = np.arange(0, m, max(1, m // 64))
    res["arms"]["fp32_sequential"] = metrics(fp32_sequential(qa[rows], qb), exact[rows])
    res["arms"]["fp32_sequential"]["rows_sampled"] = int(len(rows))
    return res


def fp32_sequential(qa: np.ndarray, qb: np.ndarray) -> np.ndarray:
    """C[i][j] = (((p_0 + p_1) + p_2) + ...) in binary32, round to nearest
    after each addition; every product of two E4M3 values is exact in
    binary32 (at most 8 significant bits)."""
    import oracle
    d = oracle.e4m3_decode_table().astype(np.float32)
    a, b = d[qa], d[qb]
    acc = np.zeros((a.shape[0], b.shape[0]), np.float32)
    for kk in range(a.shape[1]):
        acc += np.outer(a[:, kk], b[:, kk])          # exact products, one rounding per add
    return acc


def _e4m3_code(v: float) -> int:
    """Code of an exactly representable E4M3 value (search of the decode table)."""
    import oracle
    d = oracle.e4m3_decode_table()
    hits = [c for c in range(256) if d[c] == v and not (v == 0 and c == 0x80)]
    assert hits, v
    return hits[0]


def alignment_probe() -> list:
    """How one K = 128 MFMA adds small products next to a large one.

    Row s of A against B holds, in one 128-element slab, a large product
    448 * 448 (K position 0) and 127 small products 2^-s (1 * 2^-s), or a
    cancelling pair +448*448, -448*448 (positions 0 and 64) and 126 small
    products. The exact sums are 200704 + 127 * 2^-s and 126 * 2^-s. The
    result shows below which magnitude, relative to the largest product in
    the instruction, small products stop counting. Returns one dict per s.
    """
    import torch

    import fine_grained_fp8_quantize_amd as fq
    svals = list(range(0, 19))
    k = 128
    rows = []
    for cancel in (False, True):
        for sv in svals:
            a = np.full(k, _e4m3_code(1.0), np.uint8)
            b = np.full(k, _e4m3_code(2.0 ** -min(sv, 9)), np.uint8)
            if sv > 9:
                a[:] = _e4m3_code(2.0 ** -(sv - 9))
            a[0], b[0] = _e4m3_code(448.0), _e4m3_code(448.0)
            if cancel:
                a[64], b[64] = _e4m3_code(-448.0), _e4m3_code(448.0)
            rows.append((cancel, sv, a, b))
    A = torch.from_numpy(np.stack([r[2] for r in rows])).cuda()
    nr = len(rows)
    out = torch.empty((nr, (nr + 7) // 8 * 8), dtype=torch.float32, device="cuda")  # ldc % 8 == 0
    one = torch.ones(1, dtype=torch.float32, device="cuda")
    fq.fp8_gemm_tensor(A, one, torch.from_numpy(np.stack([r[3] for r in rows])).cuda(), one,
                       torch.float32, out=out[:, :nr])
    torch.cuda.synchronize()
    diag = out[:, :nr].cpu().numpy().diagonal().astype(np.float64)
    res = []
    for (cancel, sv, _, _), got in zip(rows, diag):
        small = (126 if cancel else 127) * 2.0 ** -sv
        big = 0.0 if cancel else 200704.0
        res.append({"cancel": cancel, "s": sv, "small_exact": small, "small_seen": got - big,
                    "fraction_seen": (got - big) / small})
    return res


def _table(results: list) -> str:
    cols = ["normwise", "max_rel", "max_rel_cond", "max_err_over_max", "ulp_max"]
    lines = ["| inputs | arm | " + " | ".join(cols) + " | ms | TFLOP/s |",
             "|---" * (len(cols) + 4) + "|"]
    for r in results:
        for arm, e in r["arms"].items():
            lines.append("| %s | %s | " % (r["inputs"], arm) + " | ".join("%.3g" % e[c] for c in cols)
                         + " | %s | %s |" % (e.get("ms", "—"), e.get("tflops", "—")))
    return "\n".join(lines)


if __name__ == "__main__":
    import argparse
    ap = argparse.ArgumentParser()
    ap.add_argument("--m", type=int, default=4096)
    ap.add_argument("--n", type=int, default=4096)
    ap.add_argument("--k", type=int, default=4096)
    ap.add_argument("--time-iters", type=int, default=20)
    args = ap.parse_args()
    results = []
    for positive in (False, True):
        results.append(run(args.m, args.n, args.k, positive, args.time_iters))
        print(json.dumps(results[-1]), flush=True)
    print(_table(results), flush=True)
    probe = alignment_probe()
    print(json.dumps(probe), flush=True)
    print("| products | s | small products exact | seen by the MFMA | fraction |\n|---|---|---|---|---|")
    for p in probe:
        print("| %s | %d | %.6g | %.6g | %.4f |" % ("+big, -big, 126 x 2^-s" if p["cancel"] else
                                                  "big, 127 x 2^-s", p["s"], p["small_exact"],
                                                  p["small_seen"], p["fraction_seen"]), flush=True)
