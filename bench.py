"""Benchmark of the fine-grained FP8 hot path on one MI355X.

One step is one pass of the path over one batch of seeded synthetic input
already resident in HBM: quantize the activations (1x128 tiles), quantize the
weights (128x128 blocks), and run the block-scaled FP8 GEMM with bf16 output.
The default workload is the dense Fprop layer X[4096][7168] x W[4096][7168]^T.

Prints ONE JSON line with the whole-step throughput in TFLOP/s (2*M*N*K per
step), the GEMM kernel's roofline (its own launches timed with HIP events on
the launch stream inside the timed region) and the CPU oracle timed on the
host as a reported baseline.

    python bench.py [--steps K] [--warmup W] [--config dense_fprop|dgrad|wgrad|grouped_fprop]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

FP8_DENSE_PEAK_TFLOPS = 5000.0  # MI355X dense FP8 MFMA (no sparsity)
HBM_PEAK_GBS = 8000.0

METRIC = "FP8 block-scaled GEMM TFLOP/s and % of MI355X FP8 MFMA peak (1 GPU)"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", default="dense_fprop",
                    choices=["dense_fprop", "dgrad", "wgrad", "grouped_fprop", "tiny_fprop"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--traffic-json", default=os.path.join(ROOT, "profiles", "traffic.json"),
                    help="HBM bytes per GEMM launch from rocprofv3 counters (see DESIGN.md)")
    return ap.parse_args()


class Workload:
    """Inputs on the GPU plus preallocated outputs; step() enqueues one pass."""

    def __init__(self, name: str):
        import numpy as np
        import torch

        import fine_grained_fp8_quantize_amd as fq
        import workloads as wl

        self.fq, self.torch, self.name = fq, torch, name

        def dev(bits):
            return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()

        self.host = None
        if name in ("dense_fprop", "tiny_fprop"):
            d = wl.dense_fprop() if name == "dense_fprop" else wl.tiny_fprop()
            self.host = d
            self.x, self.w = dev(d["x"]), dev(d["w"])
            m, k = self.x.shape
            n = self.w.shape[0]
            self.m, self.n, self.k = m, n, k
            self.flops = 2.0 * m * n * k
            self.xq = torch.empty((m, k), dtype=torch.uint8, device="cuda")
            self.xs = torch.empty((k // 128, m), dtype=torch.float32, device="cuda")
            self.wq = torch.empty((n, k), dtype=torch.uint8, device="cuda")
            self.ws = torch.empty((n // 128, k // 128), dtype=torch.float32, device="cuda")
            self.y = torch.empty((m, n), dtype=torch.bfloat16, device="cuda")
            self.desc = {"workload": name, "m": m, "n": n, "k": k, "x": "bf16 1x128 tiles",
                         "w": "bf16 128x128 blocks", "out": "bf16"}
        elif name == "dgrad":
            d = wl.dgrad()
            self.dy, self.w = dev(d["dy"]), dev(d["w"])
            m, n_out = self.dy.shape
            k_in = self.w.shape[1]
            self.m, self.n, self.k = m, k_in, n_out
            self.flops = 2.0 * m * k_in * n_out
            self.dq = torch.empty((m, n_out), dtype=torch.uint8, device="cuda")
            self.ds = torch.empty((n_out // 128, m), dtype=torch.float32, device="cuda")
            self.wq = torch.empty((n_out, k_in), dtype=torch.uint8, device="cuda")
            self.ws = torch.empty((n_out // 128, k_in // 128), dtype=torch.float32, device="cuda")
            self.wqt = torch.empty((k_in, n_out), dtype=torch.uint8, device="cuda")
            self.wst = torch.empty((k_in // 128, n_out // 128), dtype=torch.float32, device="cuda")
            self.y = torch.empty((m, k_in), dtype=torch.bfloat16, device="cuda")
            self.desc = {"workload": name, "m": m, "n": k_in, "k": n_out, "out": "bf16"}
        elif name == "wgrad":
            d = wl.wgrad()
            self.dy, self.x = dev(d["dy"]), dev(d["x"])
            t, n_out = self.dy.shape
            k_in = self.x.shape[1]
            self.m, self.n, self.k = n_out, k_in, t
            self.flops = 2.0 * n_out * k_in * t
            self.aq = torch.empty((n_out, t), dtype=torch.uint8, device="cuda")
            self.as_ = torch.empty((t // 128, n_out), dtype=torch.float32, device="cuda")
            self.bq = torch.empty((k_in, t), dtype=torch.uint8, device="cuda")
            self.bs = torch.empty((t // 128, k_in), dtype=torch.float32, device="cuda")
            self.y = torch.empty((n_out, k_in), dtype=torch.float32, device="cuda")
            self.desc = {"workload": name, "m": n_out, "n": k_in, "k": t, "out": "fp32"}
        else:  # grouped_fprop
            g = wl.grouped_fprop()
            rows = g["rows"]
            self.x = dev(g["x"])
            E, n, k = g["w"].shape
            self.w = dev(g["w"].reshape(E * n, k))
            m_total = self.x.shape[0]
            self.m, self.n, self.k = int(rows.sum()), n, k
            self.flops = 2.0 * float(rows.sum()) * n * k   # real rows only
            self.off = torch.from_numpy(g["offsets"].astype("int32")).cuda()
            self.rows = torch.from_numpy(rows.astype("int32")).cuda()
            self.xq = torch.empty((m_total, k), dtype=torch.uint8, device="cuda")
            self.xs = torch.empty((k // 128, m_total), dtype=torch.float32, device="cuda")
            self.wq = torch.empty((E * n, k), dtype=torch.uint8, device="cuda")
            self.ws = torch.empty((E * n // 128, k // 128), dtype=torch.float32, device="cuda")
            self.E = E
            self.y = torch.empty((m_total, n), dtype=torch.bfloat16, device="cuda")
            self.desc = {"workload": name, "experts": E, "rows_real": int(rows.sum()),
                         "rows_padded": m_total, "n": n, "k": k, "out": "bf16"}
        torch.cuda.synchronize()

    def step(self, ev=None):
        fq, torch = self.fq, self.torch
        if self.name in ("dense_fprop", "tiny_fprop"):
            fq.fp8_quantize_act(self.x, "1x128", q=self.xq, scale=self.xs)
            fq.fp8_quantize_weight(self.w, q=self.wq, scale=self.ws)
            if ev is not None:
                ev[0].record()
            fq.fp8_gemm(self.xq, self.xs, self.wq, self.ws, "block", torch.bfloat16, out=self.y)
            if ev is not None:
                ev[1].record()
        elif self.name == "dgrad":
            fq.fp8_quantize_act(self.dy, "1x128", q=self.dq, scale=self.ds)
            fq.fp8_quantize_weight(self.w, transposed=True, q=self.wq, scale=self.ws, q_t=self.wqt,
                                   scale_t=self.wst)
            if ev is not None:
                ev[0].record()
            fq.fp8_gemm(self.dq, self.ds, self.wqt, self.wst, "block", torch.bfloat16, out=self.y)
            if ev is not None:
                ev[1].record()
        elif self.name == "wgrad":
            fq.fp8_quantize_act(self.dy, "128x1", q=self.aq, scale=self.as_)
            fq.fp8_quantize_act(self.x, "128x1", q=self.bq, scale=self.bs)
            if ev is not None:
                ev[0].record()
            fq.fp8_gemm(self.aq, self.as_, self.bq, self.bs, "row", torch.float32, out=self.y)
            if ev is not None:
                ev[1].record()
        else:
            fq.fp8_quantize_act(self.x, "1x128", q=self.xq, scale=self.xs)
            fq.fp8_quantize_weight(self.w, q=self.wq, scale=self.ws)
            if ev is not None:
                ev[0].record()
            n, k = self.n, self.k
            fq.fp8_grouped_gemm(self.off, self.rows, self.xq, self.xs,
                                self.wq.view(self.E, n, k), self.ws.view(self.E, n // 128, k // 128),
                                torch.bfloat16, out=self.y)
            if ev is not None:
                ev[1].record()


def cpu_baseline(wl_obj: Workload) -> dict:
    """The oracle, as it stands, on the same Dense Fprop inputs (the whole step)."""
    import numpy as np

    import oracle
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # pragma: no cover - informational only
        blas_threads = 1
    omp = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    d = wl_obj.host
    t0 = time.perf_counter()
    a_q, a_s = oracle.quant_act_1x128(d["x"])
    b_q, b_s = oracle.quant_weight_128x128(d["w"])
    c = oracle.gemm(a_q, a_s, b_q, b_s, "block")
    dt = time.perf_counter() - t0
    del c
    m, k = d["x"].shape
    n = d["w"].shape[0]
    return {
        "value": 2.0 * m * n * k / dt / 1e12,
        "unit": "TFLOP/s",
        "cores": max(omp, blas_threads),
        "kind": "oracle",
        "seconds": round(dt, 3),
        "sample": "one full step of the workload (X %dx%d 1x128 quantize, W %dx%d 128x128 "
                  "quantize, float64 dequantize + GEMM), scalar C quantizers with OpenMP and "
                  "numpy float64 matmul" % (m, k, n, k),
    }


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)
    import torch

    wl_obj = Workload(args.config)
    stream = torch.cuda.current_stream()
    for _ in range(args.warmup):
        wl_obj.step()
    torch.cuda.synchronize()

    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    start.record(stream)
    for i in range(args.steps):
        wl_obj.step(evs[i])
    stop.record(stream)
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall
    ms = start.elapsed_time(stop) / args.steps
    gemm_ms = sum(a.elapsed_time(b) for a, b in evs) / args.steps

    value = wl_obj.flops / (ms * 1e-3) / 1e12
    gemm_tflops = wl_obj.flops / (gemm_ms * 1e-3) / 1e12
    traffic = None
    try:
        with open(args.traffic_json) as f:
            traffic = json.load(f).get(args.config)
    except (OSError, ValueError):
        traffic = None

    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8-e4m3 x fp8-e4m3 -> fp32 accumulate, bf16 out" if args.config != "wgrad"
                 else "fp8-e4m3 x fp8-e4m3 -> fp32 accumulate, fp32 out",
        "data": "synthetic (seeded; see workloads/)",
        "config": wl_obj.desc,
        "pct_of_fp8_peak": round(100.0 * value / FP8_DENSE_PEAK_TFLOPS, 2),
        "gemm_ms": round(gemm_ms, 4),
        "gemm_tflops": round(gemm_tflops, 2),
        "roofline": {
            "bound": "mfma",
            "achieved": round(gemm_tflops, 2),
            "peak": FP8_DENSE_PEAK_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(gemm_tflops / FP8_DENSE_PEAK_TFLOPS, 4),
            "traffic": traffic,
            "kernel": "gemm_kernel" if args.config != "grouped_fprop" else "gemm_kernel (grouped)",
        },
        "wall_s": round(t_wall, 3),
    }
    if not args.no_cpu_baseline and wl_obj.host is not None:
        out["cpu_baseline"] = cpu_baseline(wl_obj)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
