"""Benchmark of the fine-grained FP8 hot path on one MI355X.

One step is one pass of the path over one batch of seeded synthetic input
already resident in HBM: quantize the operands (activations in 1x128 tiles,
weights in 128x128 blocks, or both Wgrad operands in 128x1 tiles) and run the
block-scaled FP8 GEMM, in that order on one stream (``--streams 2`` puts the
two independent quantizations on two streams; that measures slower). The
default workload is the largest single-GPU configuration, the grouped MoE
Fprop: 8192 tokens [8192][7168] quantized before dispatch into 32 local
experts (Zipf(1.1) routing, 8192 routed rows, 10112 after 128-padding), the
32 expert weights [32][4096][7168] quantized in 128x128 blocks, and the
grouped GEMM with bf16 output.

Prints ONE JSON line: the whole-step throughput in TFLOP/s (2*M*N*K per step),
the GEMM kernel's roofline (its launches timed with HIP events on the launch
stream inside the timed region, where only the GEMM is bracketed: each event
pair costs the step GPU time), every kernel's own time and rate (from a second
pass with every launch bracketed), and the CPU oracle timed on the host as a
reported baseline. The roofline carries the GEMM's fraction of both peaks,
dense FP8 MFMA and HBM; ``bound`` names the one its arithmetic intensity
puts it under.

    python bench.py [--steps K] [--warmup W] [--streams 1|2]
                    [--config dense_fprop|dgrad|wgrad|grouped_fprop|grouped_dgrad|
                              grouped_wgrad|mx_fprop|wgrad_cached|
                              grouped_wgrad_cached|tiny_fprop]

Counter runs (HBM traffic of each kernel, from rocprofv3 FETCH_SIZE and
WRITE_SIZE; a plain copy of known size calibrates each counter):

    rocprofv3 --pmc FETCH_SIZE -d OUT -o fetch --output-format csv -- \
        python bench.py --steps 3 --warmup 1 --prewarm-s 0 --no-cpu-baseline --copy-probe-mib 256
    (same with WRITE_SIZE and -o write)
    python bench.py --pmc-summary OUT/fetch_counter_collection.csv OUT/write_counter_collection.csv
"""
from __future__ import annotations

import argparse
import csv
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

FP8_DENSE_PEAK_TFLOPS = 5000.0  # MI355X dense FP8 MFMA (no sparsity)
HBM_PEAK_GBS = 8000.0           # MI355X HBM3E

METRIC = "FP8 block-scaled GEMM TFLOP/s and % of MI355X FP8 MFMA peak (1 GPU)"
CONFIGS = ["dense_fprop", "dgrad", "wgrad", "grouped_fprop", "grouped_dgrad", "grouped_wgrad",
           "mx_fprop", "wgrad_cached", "grouped_wgrad_cached", "tiny_fprop"]
TRAFFIC_JSON = os.path.join(ROOT, "profiles", "traffic.json")

# Kernel name fragments (as rocprofv3 prints them) for each launch label.
KERNEL_NAMES = {
    "quant_act_1x128": "quant_act_1x128_kernel<false>",
    "quant_act_scatter": "quant_act_1x128_kernel<true>",
    "quant_act_128x1": "quant_act_128x1_kernel",
    "quant_weight": "quant_weight_kernel",
    "quant_act_weight": "quant_act_weight_kernel",
    "quant_act_128x1_pair": "quant_act_128x1_pair_kernel",
    "quant_retile_128x1": "quant_retile_128x1_kernel",
    "quant_mx": "quant_mx_1x32_kernel",
    "quant_mx_pair": "quant_mx_1x32_pair_kernel",
    "retile_128x1": "retile_128x1_kernel",
    "gemm": ("gemm_kernel", "grouped_fixup_kernel"),  # a grouped GEMM may add its fix-up kernel
}


def _code_only(text: str) -> str:
    """Source text without comments, blank lines and indentation (what the
    kernels are made of)."""
    import re
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    text = re.sub(r"//[^\n]*", "", text)
    return "\n".join(line.strip() for line in text.splitlines() if line.strip())


def kernel_source_digest(csrc: str | None = None) -> str:
    """Digest of the kernel sources (the .hip files, with their launchers, and
    the headers they include), comments and blank lines left out; stored
    counter figures are valid only for the kernels they were taken on. The
    C ABI's host-side argument checks (.cpp) are not part of it."""
    h = hashlib.sha256()
    csrc = csrc or os.path.join(ROOT, "fine_grained_fp8_quantize_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        if name.endswith((".hip", ".h")):
            with open(os.path.join(csrc, name), encoding="utf-8") as f:
                h.update(name.encode() + b"\0" + _code_only(f.read()).encode())
    return h.hexdigest()[:16]


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--prewarm-s", type=float, default=0.5,
                    help="seconds of untimed steps before the warmup steps (clock ramp)")
    ap.add_argument("--config", default="grouped_fprop", choices=CONFIGS)
    ap.add_argument("--rotate", type=int, default=3,
                    help="bf16 input sets cycled over the steps, so that the inputs of one "
                         "step are not left in the 256 MiB MALL by the step before")
    ap.add_argument("--streams", type=int, default=1, choices=(1, 2),
                    help="2: the two independent operand quantizations run on two streams "
                         "(measured slower: both are HBM-bound, and the cross-stream wait "
                         "before the GEMM costs more than the overlap saves)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="run one device copy of this size first (counter calibration)")
    ap.add_argument("--traffic-json", default=TRAFFIC_JSON)
    ap.add_argument("--counter-table", metavar="CSV",
                    help="print a markdown table of a rocprofv3 counter CSV of this script, "
                         "per kernel of the step")
    ap.add_argument("--pmc-summary", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="turn two rocprofv3 counter CSVs of this script into --traffic-json")
    return ap.parse_args()


class Launch:
    """One kernel launch of the step with its algorithmic cost."""

    def __init__(self, label, fn, nbytes, flops=0.0, dispatches=1):
        self.label, self.fn, self.bytes, self.flops = label, fn, float(nbytes), float(flops)
        self.dispatches = dispatches  # kernel dispatches the launch makes


class Workload:
    """Inputs on the GPU plus preallocated outputs; step() enqueues one pass."""

    def __init__(self, name: str, rotate: int = 1, streams: int = 1):
        import numpy as np
        import torch

        import fine_grained_fp8_quantize_amd as fq
        import workloads as wl

        self.torch, self.name = torch, name
        u8, f32, bf16 = torch.uint8, torch.float32, torch.bfloat16

        def dev(bits):
            return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(bf16).cuda()

        def empty(shape, dt):
            return torch.empty(shape, dtype=dt, device="cuda")

        # the grouped GEMM's workspace (the K-split of a partial last round)
        gws = empty((fq.GROUPED_WORKSPACE_BYTES,), u8)

        def sets(bits):
            # `rotate` device copies of one bf16 input; step i reads copy i % rotate
            t = dev(bits)
            return [t] + [t.clone() for _ in range(rotate - 1)]

        def act_bytes(r, c):       # bf16 in, codes + one fp32 scale per 128 values out
            return 2 * r * c + r * c + 4 * r * c // 128

        def gemm_bytes(m_a, n, k, b_scale_count, out_elem, m_out):
            return m_a * k + n * k + 4 * m_a * (k // 128) + 4 * b_scale_count + out_elem * m_out * n

        def packed(real_bits, off, rows):
            # expert-sorted rows, 128-padded segments, zero padding rows
            out = np.zeros((int(off[-1]), real_bits.shape[1]), np.uint16)
            src = 0
            for e in range(len(rows)):
                out[off[e]:off[e] + rows[e]] = real_bits[src:src + rows[e]]
                src += int(rows[e])
            return out

        self.host = None
        self.bound = "mfma"
        if name in ("dense_fprop", "tiny_fprop"):
            d = wl.dense_fprop() if name == "dense_fprop" else wl.tiny_fprop()
            self.host = d
            X, W = sets(d["x"]), sets(d["w"])
            m, k = X[0].shape
            n = W[0].shape[0]
            xq, xs = empty((m, k), u8), empty((k // 128, m), f32)
            wq, ws = empty((n, k), u8), empty((n // 128, k // 128), f32)
            y = empty((m, n), bf16)
            self.flops = 2.0 * m * n * k
            self.launches = [
                # x in 1x128 tiles and w in 128x128 blocks, one launch
                Launch("quant_act_weight", lambda r: fq.fp8_quantize_act_weight(
                    X[r], W[r], q=xq, scale=xs, wq=wq, wscale=ws),
                       act_bytes(m, k) + 3 * n * k + 4 * (n // 128) * (k // 128)),
                Launch("gemm", lambda r: fq.fp8_gemm(xq, xs, wq, ws, "block", bf16, out=y),
                       gemm_bytes(m, n, k, (n // 128) * (k // 128), 2, m), self.flops),
            ]
            self.desc = {"workload": name, "m": m, "n": n, "k": k, "x": "bf16, 1x128 tiles",
                         "w": "bf16, 128x128 blocks", "out": "bf16"}
        elif name == "mx_fprop":
            # the Dense Fprop shapes with microscaling: both operands in 1x32
            # blocks along K with E8M0 scales, scaled-MFMA GEMM
            d = wl.dense_fprop()
            X, W = sets(d["x"]), sets(d["w"])
            m, k = X[0].shape
            n = W[0].shape[0]
            xq, xs = empty((m, k), u8), empty((k // 128, m), torch.int32)
            wq, ws = empty((n, k), u8), empty((k // 128, n), torch.int32)
            y = empty((m, n), bf16)
            self.flops = 2.0 * m * n * k

            def mx_bytes(r, c):   # bf16 in, codes + one byte per 32 values out
                return 2 * r * c + r * c + r * c // 32
            self.launches = [
                # X and W in 1x32 blocks, one launch
                Launch("quant_mx_pair", lambda r: fq.fp8_quantize_mx_pair(
                    X[r], W[r], q0=xq, scale0=xs, q1=wq, scale1=ws), mx_bytes(m, k) + mx_bytes(n, k)),
                Launch("gemm", lambda r: fq.fp8_gemm_mx(xq, xs, wq, ws, bf16, out=y),
                       m * k + n * k + (m + n) * k // 32 + 2 * m * n, self.flops),
            ]
            self.desc = {"workload": name, "m": m, "n": n, "k": k,
                         "x, w": "bf16, 1x32 blocks along K, E8M0 scales (OCP MX)", "out": "bf16"}
        elif name == "dgrad":
            d = wl.dgrad()
            DY, W = sets(d["dy"]), sets(d["w"])
            m, n_out = DY[0].shape
            k_in = W[0].shape[1]
            dq, ds = empty((m, n_out), u8), empty((n_out // 128, m), f32)
            wq, ws = empty((n_out, k_in), u8), empty((n_out // 128, k_in // 128), f32)
            wqt, wst = empty((k_in, n_out), u8), empty((k_in // 128, n_out // 128), f32)
            y = empty((m, k_in), bf16)
            self.flops = 2.0 * m * k_in * n_out
            nb = (n_out // 128) * (k_in // 128)
            self.launches = [
                # dy in 1x128 tiles and w in 128x128 blocks with the
                # transposed copy the GEMM reads, one launch
                Launch("quant_act_weight", lambda r: fq.fp8_quantize_act_weight(
                    DY[r], W[r], transposed=True, q=dq, scale=ds, wq=wq, wscale=ws, wq_t=wqt, wscale_t=wst),
                       act_bytes(m, n_out) + 4 * n_out * k_in + 8 * nb),
                Launch("gemm", lambda r: fq.fp8_gemm(dq, ds, wqt, wst, "block", bf16, out=y),
                       gemm_bytes(m, k_in, n_out, nb, 2, m), self.flops),
            ]
            self.desc = {"workload": name, "m": m, "n": k_in, "k": n_out,
                         "dy": "bf16, 1x128 tiles", "w": "bf16, 128x128 blocks, transposed copy",
                         "out": "bf16"}
        elif name == "wgrad":
            d = wl.wgrad()
            DY, X = sets(d["dy"]), sets(d["x"])
            t, n_out = DY[0].shape
            k_in = X[0].shape[1]
            aq, as_ = empty((n_out, t), u8), empty((t // 128, n_out), f32)
            bq, bs = empty((k_in, t), u8), empty((t // 128, k_in), f32)
            y = empty((n_out, k_in), f32)
            self.flops = 2.0 * n_out * k_in * t
            self.launches = [
                # dY and X in 128x1 token tiles, one launch
                Launch("quant_act_128x1_pair", lambda r: fq.fp8_quantize_act_128x1_pair(
                    DY[r], X[r], q0=aq, scale0=as_, q1=bq, scale1=bs),
                       act_bytes(t, n_out) + act_bytes(t, k_in)),
                Launch("gemm", lambda r: fq.fp8_gemm(aq, as_, bq, bs, "row", f32, out=y),
                       gemm_bytes(n_out, k_in, t, k_in * (t // 128), 4, n_out), self.flops),
            ]
            self.desc = {"workload": name, "m": n_out, "n": k_in, "k": t,
                         "dy, x": "bf16, 128x1 tiles (along tokens)", "out": "fp32"}
        elif name == "wgrad_cached":
            # Wgrad with X taken from its forward-pass FP8 cache (1x128 codes
            # and scales, written by the forward quantizer before the step):
            # dY quantized 128x1, the cache re-tiled to 128x1, then the GEMM
            d = wl.wgrad()
            DY = sets(d["dy"])
            t, n_out = DY[0].shape
            k_in = d["x"].shape[1]
            x_dev = dev(d["x"])
            XQ, XS = [], []
            for _ in range(rotate):
                xq_, xs_ = fq.fp8_quantize_act(x_dev, "1x128")
                XQ.append(xq_)
                XS.append(xs_)
            del x_dev
            aq, as_ = empty((n_out, t), u8), empty((t // 128, n_out), f32)
            bq, bs = empty((k_in, t), u8), empty((t // 128, k_in), f32)
            y = empty((n_out, k_in), f32)
            self.flops = 2.0 * n_out * k_in * t
            self.launches = [
                # dY quantized 128x1 and the cache re-tiled (codes + 1x128
                # scales in, codes + 128x1 scales out), one launch
                Launch("quant_retile_128x1", lambda r: fq.fp8_quantize_act_128x1_retile(
                    DY[r], XQ[r], XS[r], q0=aq, scale0=as_, q1=bq, scale1=bs),
                       act_bytes(t, n_out) + 2 * t * k_in + 8 * t * k_in // 128),
                Launch("gemm", lambda r: fq.fp8_gemm(aq, as_, bq, bs, "row", f32, out=y),
                       gemm_bytes(n_out, k_in, t, k_in * (t // 128), 4, n_out), self.flops),
            ]
            self.desc = {"workload": name, "m": n_out, "n": k_in, "k": t,
                         "dy": "bf16, 128x1 tiles (along tokens)",
                         "x": "FP8 cache (1x128 codes + scales) re-tiled to 128x1", "out": "fp32"}
        elif name == "grouped_dgrad":
            # MoE up-projection Dgrad: dX_e = dY_e W_e with each expert's transposed copy
            rows = wl.moe_rows(0)
            off = wl.pad_offsets(rows)
            E, n_out, k_in = len(rows), 4096, 7168
            real = int(rows.sum())
            m_total = int(off[-1])
            DY = sets(packed(wl.grad_rowscaled(0, "grouped_fprop", 4, real, n_out), off, rows))
            w = dev(wl.weight(0, "grouped_fprop", 1, E, n_out, k_in))
            offd = torch.from_numpy(off.astype("int32")).cuda()
            rws = torch.from_numpy(rows.astype("int32")).cuda()
            dq, ds = empty((m_total, n_out), u8), empty((n_out // 128, m_total), f32)
            # all experts' weights in one grouped-quantizer launch, with each
            # expert's transposed copy contiguous (the Dgrad B operand)
            wq, ws = empty((E, n_out, k_in), u8), empty((E, n_out // 128, k_in // 128), f32)
            wqt, wst = empty((E, k_in, n_out), u8), empty((E, k_in // 128, n_out // 128), f32)
            y = empty((m_total, k_in), bf16)
            self.flops = 2.0 * real * k_in * n_out
            nb = E * (n_out // 128) * (k_in // 128)
            self.launches = [
                Launch("quant_act_1x128", lambda r: fq.fp8_quantize_act(DY[r], "1x128", q=dq, scale=ds),
                       act_bytes(m_total, n_out)),
                Launch("quant_weight", lambda r: fq.fp8_quantize_weight_grouped(
                    w, transposed=True, q=wq, scale=ws, q_t=wqt, scale_t=wst),
                       4 * E * n_out * k_in + 8 * nb),
                Launch("gemm", lambda r: fq.fp8_grouped_gemm(offd, rws, dq, ds, wqt, wst, bf16, out=y,
                                                             workspace=gws),
                       gemm_bytes(real, E * k_in, n_out, nb, 2, 0) + 2 * m_total * k_in, self.flops),
            ]
            self.desc = {"workload": name, "experts": E, "rows_real": real, "rows_padded": m_total,
                         "n": k_in, "k": n_out, "dy": "bf16, 1x128 tiles",
                         "w": "bf16, 128x128 blocks, all experts in one launch with per-expert transposed copies",
                         "out": "bf16"}
        elif name == "grouped_wgrad_cached":
            # MoE Wgrad with X taken from the FP8 cache the dispatch quantizer
            # wrote in the forward pass (expert-sorted 1x128 codes + scales,
            # padding rows zero): dY quantized 128x1, the cache re-tiled to
            # 128x1 (128-aligned segments: no tile straddles experts), GEMM
            d = wl.moe_dispatch()
            rows, off = d["rows"], d["offsets"]
            E, n_out, k_in = len(rows), 4096, 7168
            real = int(rows.sum())
            m_total = int(off[-1])
            DY = sets(packed(wl.grad_rowscaled(0, "grouped_fprop", 4, real, n_out), off, rows))
            x_dev = dev(d["x"])
            dst = torch.from_numpy(d["dst_rows"]).cuda()
            XQ, XS = [], []
            for _ in range(rotate):
                xq_ = torch.zeros((m_total, k_in), dtype=u8, device="cuda")
                xs_ = torch.zeros((k_in // 128, m_total), dtype=f32, device="cuda")
                fq.fp8_quantize_act_scatter(x_dev, dst, m_total, q=xq_, scale=xs_)
                XQ.append(xq_)
                XS.append(xs_)
            del x_dev
            offd = torch.from_numpy(off.astype("int32")).cuda()
            aq, as_ = empty((n_out, m_total), u8), empty((m_total // 128, n_out), f32)
            bq, bs = empty((k_in, m_total), u8), empty((m_total // 128, k_in), f32)
            y = empty((E, n_out, k_in), f32)
            self.flops = 2.0 * real * n_out * k_in   # real tokens only
            self.bound = "hbm"                        # 3.8 GB of fp32 gradients written
            self.launches = [
                # dY quantized 128x1 and the dispatch cache re-tiled, one launch
                Launch("quant_retile_128x1", lambda r: fq.fp8_quantize_act_128x1_retile(
                    DY[r], XQ[r], XS[r], q0=aq, scale0=as_, q1=bq, scale1=bs),
                       act_bytes(m_total, n_out) + 2 * m_total * k_in + 8 * m_total * k_in // 128),
                Launch("gemm", lambda r: fq.fp8_grouped_gemm_wgrad(offd, aq, as_, bq, bs, f32, out=y),
                       (n_out + k_in) * m_total * (1 + 4 / 128) + 4 * E * n_out * k_in, self.flops),
            ]
            self.desc = {"workload": name, "experts": E, "tokens_real": real, "tokens_padded": m_total,
                         "m": n_out, "n": k_in, "dy": "bf16, 128x1 tiles (along tokens)",
                         "x": "FP8 dispatch cache (expert-sorted 1x128 codes + scales) re-tiled to 128x1",
                         "out": "fp32 [experts][m][n]"}
        elif name == "grouped_wgrad":
            # MoE up-projection Wgrad: dW_e = dY_e^T X_e over each expert's tokens
            rows = wl.moe_rows(0)
            off = wl.pad_offsets(rows)
            E, n_out, k_in = len(rows), 4096, 7168
            real = int(rows.sum())
            m_total = int(off[-1])
            DY = sets(packed(wl.grad_rowscaled(0, "grouped_fprop", 4, real, n_out), off, rows))
            X = sets(packed(wl.activation(0, "grouped_fprop", 5, real, k_in, 50.0), off, rows))
            offd = torch.from_numpy(off.astype("int32")).cuda()
            aq, as_ = empty((n_out, m_total), u8), empty((m_total // 128, n_out), f32)
            bq, bs = empty((k_in, m_total), u8), empty((m_total // 128, k_in), f32)
            y = empty((E, n_out, k_in), f32)
            self.flops = 2.0 * real * n_out * k_in   # real tokens only
            self.bound = "hbm"                        # 3.8 GB of fp32 gradients written
            self.launches = [
                # dY and X (expert-sorted) in 128x1 token tiles, one launch
                Launch("quant_act_128x1_pair", lambda r: fq.fp8_quantize_act_128x1_pair(
                    DY[r], X[r], q0=aq, scale0=as_, q1=bq, scale1=bs),
                       act_bytes(m_total, n_out) + act_bytes(m_total, k_in)),
                Launch("gemm", lambda r: fq.fp8_grouped_gemm_wgrad(offd, aq, as_, bq, bs, f32, out=y),
                       (n_out + k_in) * m_total * (1 + 4 / 128) + 4 * E * n_out * k_in, self.flops),
            ]
            self.desc = {"workload": name, "experts": E, "tokens_real": real, "tokens_padded": m_total,
                         "m": n_out, "n": k_in, "dy, x": "bf16, 128x1 tiles (along tokens)",
                         "out": "fp32 [experts][m][n]"}
        else:  # grouped_fprop: quantize the tokens before dispatch, then the expert GEMM
            d = wl.moe_dispatch()
            rows = d["rows"]
            X = sets(d["x"])
            E, n, k = len(rows), 4096, X[0].shape[1]
            # the expert weights of the grouped MoE config (1.9 GB: far beyond the MALL)
            w_bits = wl.weight(0, "grouped_fprop", 1, E, n, k)
            w = dev(w_bits.reshape(E * n, k))
            self.host = {"dispatch": d, "w": w_bits}
            self.bound = "hbm"   # 452 flop/B: below the MFMA/HBM ridge (~629 flop/B)
            tokens = X[0].shape[0]
            m_total = int(d["offsets"][-1])
            real = int(rows.sum())
            off = torch.from_numpy(d["offsets"].astype("int32")).cuda()
            rws = torch.from_numpy(rows.astype("int32")).cuda()
            dst = torch.from_numpy(d["dst_rows"]).cuda()
            xq, xs = empty((m_total, k), u8), empty((k // 128, m_total), f32)
            wq, ws = empty((E * n, k), u8), empty((E * n // 128, k // 128), f32)
            y = empty((m_total, n), bf16)
            self.flops = 2.0 * real * n * k   # real rows only
            nb = E * (n // 128) * (k // 128)
            self.launches = [
                # tokens read once; every route writes its codes and scales
                Launch("quant_act_scatter", lambda r: fq.fp8_quantize_act_scatter(
                    X[r], dst, m_total, q=xq, scale=xs),
                       2 * tokens * k + real * (k + 4 * k // 128)),
                Launch("quant_weight", lambda r: fq.fp8_quantize_weight(w, q=wq, scale=ws),
                       3 * E * n * k + 4 * nb),
                # real rows of A read; every padded row of C written (padding rows are zeroed)
                Launch("gemm", lambda r: fq.fp8_grouped_gemm(
                    off, rws, xq, xs, wq.view(E, n, k), ws.view(E, n // 128, k // 128), bf16, out=y,
                    workspace=gws),
                       gemm_bytes(real, E * n, k, nb, 2, 0) + 2 * m_total * n, self.flops),
            ]
            self.desc = {"workload": name, "experts": E, "tokens": tokens, "top_k": 8,
                         "rows_real": real, "rows_padded": m_total, "n": n, "k": k,
                         "x": "bf16 tokens, quantized 1x128 before dispatch", "out": "bf16"}
        self.rotate, self.count = rotate, 0
        self.desc["input_sets"] = rotate
        # streams == 2: the two operand quantizations are independent, so the
        # second can run on a side stream (default priority) beside the first;
        # the GEMM waits for both. The side stream's work of a step starts
        # after everything the main stream enqueued before it (the previous
        # step's GEMM included), so no buffer is overwritten while in use.
        assert self.launches[-1].label == "gemm"
        if streams == 2 and len(self.launches) != 3:
            raise SystemExit("--streams 2 overlaps two quantization launches; %s quantizes in %d"
                             % (name, len(self.launches) - 1))
        self.side = torch.cuda.Stream() if streams == 2 else None
        self.mark = torch.cuda.Event()
        self.done = torch.cuda.Event()
        self.desc["streams"] = streams
        torch.cuda.synchronize()

    def step(self, ev=None):
        """One pass over the next input set; ev (per launch, a (begin, end)
        event pair or None) brackets the chosen launches on the stream each
        runs on."""
        torch = self.torch
        r = self.count % self.rotate
        self.count += 1
        main = torch.cuda.current_stream()
        if self.side is not None:
            self.mark.record(main)
            self.side.wait_event(self.mark)
        for i, ln in enumerate(self.launches):
            s = self.side if (self.side is not None and i == 1) else main
            if ln.label == "gemm" and self.side is not None:
                main.wait_event(self.done)
            pair = ev[i] if ev is not None else None
            with torch.cuda.stream(s):
                if pair is not None:
                    pair[0].record(s)
                ln.fn(r)
                if pair is not None:
                    pair[1].record(s)
            if s is not main:
                self.done.record(s)


def cpu_model() -> str:
    """The host CPU's model name (reported with the oracle timing)."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def tiny_one_thread(min_seconds: float = 1.0) -> dict:
    """The oracle's whole Tiny Fprop step (128x256x512) on one thread: every
    OpenMP and BLAS pool limited to 1 for the duration."""
    import oracle
    import workloads as wl
    from threadpoolctl import threadpool_limits
    d = wl.tiny_fprop()
    m, k = d["x"].shape
    n = d["w"].shape[0]
    with threadpool_limits(limits=1):
        steps, t0 = 0, time.perf_counter()
        while True:
            a_q, a_s = oracle.quant_act_1x128(d["x"])
            b_q, b_s = oracle.quant_weight_128x128(d["w"])
            oracle.gemm(a_q, a_s, b_q, b_s, "block")
            steps += 1
            dt = time.perf_counter() - t0
            if dt >= min_seconds:
                break
    return {"threads": 1, "steps": steps, "ms_per_step": round(1e3 * dt / steps, 4),
            "gflops": round(2.0 * m * n * k * steps / dt / 1e9, 4)}


def _oracle_threads() -> int:
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # pragma: no cover - informational only
        blas_threads = 1
    omp = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    return max(omp, blas_threads)


def cpu_baseline(wl_obj: Workload, min_seconds: float = 10.0, max_steps: int = 200) -> dict:
    """The oracle, as it stands, on the same inputs as the GPU step: whole
    steps repeated until at least min_seconds of CPU work (at least one)."""
    import oracle
    if wl_obj.name == "grouped_fprop":
        return cpu_baseline_grouped(wl_obj, min_seconds)
    d = wl_obj.host
    m, k = d["x"].shape
    n = d["w"].shape[0]
    # Whole oracle steps (quantize X, quantize W, float64 GEMM) on the same
    # inputs, repeated until at least min_seconds of CPU work.
    steps, t0 = 0, time.perf_counter()
    while True:
        a_q, a_s = oracle.quant_act_1x128(d["x"])
        b_q, b_s = oracle.quant_weight_128x128(d["w"])
        c = oracle.gemm(a_q, a_s, b_q, b_s, "block")
        del c
        steps += 1
        dt = time.perf_counter() - t0
        if dt >= min_seconds or steps >= max_steps:
            break
    return {
        "value": round(2.0 * m * n * k * steps / dt / 1e12, 4),
        "unit": "TFLOP/s",
        "cores": _oracle_threads(),
        "kind": "oracle",
        "seconds": round(dt, 3),
        "steps": steps,
        "sample": "%d full steps of the workload (X %dx%d 1x128 quantize, W %dx%d 128x128 "
                  "quantize, float64 dequantize + GEMM): scalar C quantizers with OpenMP and "
                  "numpy float64 matmul" % (steps, m, k, n, k),
        "cpu_model": cpu_model(),
        "tiny_fprop_one_thread": tiny_one_thread(),
    }


def cpu_baseline_grouped(wl_obj: Workload, min_seconds: float = 10.0) -> dict:
    """The oracle's whole grouped MoE Fprop step on the same routed inputs:
    quantize the 8192 tokens before dispatch and scatter them to their
    expert-sorted rows, quantize the 32 expert weights in 128x128 blocks,
    then the float64 per-expert GEMM over the real rows. Whole steps until
    at least min_seconds (one step is several seconds on the host)."""
    import numpy as np

    import oracle
    d, w = wl_obj.host["dispatch"], wl_obj.host["w"]
    rows, off = d["rows"], d["offsets"]
    m_total = int(off[-1])
    E, n, k = w.shape
    flops = 2.0 * float(rows.sum()) * n * k
    b_q = np.empty((E, n, k), np.uint8)
    b_s = np.empty((E, n // 128, k // 128), np.float32)
    steps, t0 = 0, time.perf_counter()
    while True:
        a_q, a_s, _ = oracle.quant_act_scatter(d["x"], d["dst_rows"], m_total)
        for e in range(E):
            b_q[e], b_s[e] = oracle.quant_weight_128x128(w[e])
        c = oracle.grouped_gemm(off, rows, a_q, a_s, b_q, b_s)
        del c
        steps += 1
        dt = time.perf_counter() - t0
        if dt >= min_seconds:
            break
    return {
        "value": round(flops * steps / dt / 1e12, 4),
        "unit": "TFLOP/s",
        "cores": _oracle_threads(),
        "kind": "oracle",
        "seconds": round(dt, 3),
        "steps": steps,
        "sample": "%d full steps of the grouped workload (8192 tokens x %d quantized 1x128 and "
                  "scattered to %d expert-sorted rows, %d expert weights %dx%d quantized 128x128, "
                  "float64 per-expert GEMM over %d real rows): scalar C quantizers with OpenMP and "
                  "numpy float64 matmul" % (steps, k, m_total, E, n, k, int(rows.sum())),
        "cpu_model": cpu_model(),
        "tiny_fprop_one_thread": tiny_one_thread(),
    }


# ---------------------------------------------------------------- counters

def _read_counter_csv(path: str, counter: str):
    """Dispatches of one rocprofv3 counter CSV: [(dispatch_id, kernel, KiB)]."""
    rows = {}
    with open(path, newline="") as f:
        for r in csv.DictReader(f):
            if r["Counter_Name"] != counter:
                continue
            did = int(r["Dispatch_Id"])
            name, val = r["Kernel_Name"], float(r["Counter_Value"])
            rows[did] = (did, name, rows.get(did, (0, name, 0.0))[2] + val)
    return [rows[d] for d in sorted(rows)]


def pmc_summary(fetch_csv: str, write_csv: str, config: str, probe_mib: int, out_json: str,
                wl_obj: Workload) -> dict:
    """Per-launch HBM bytes of every kernel of the step from FETCH_SIZE and
    WRITE_SIZE (KiB per dispatch), each scaled by the factor that maps what
    the counter reads for the calibration copy onto the copy's true bytes."""
    probe = probe_mib * (1 << 20)
    res = {"kernel_source": kernel_source_digest(), "copy_probe_bytes": probe,
           "fetch_csv": os.path.basename(fetch_csv), "write_csv": os.path.basename(write_csv)}
    for counter, path, key in (("FETCH_SIZE", fetch_csv, "fetch"), ("WRITE_SIZE", write_csv, "write")):
        rows = _read_counter_csv(path, counter)
        copies = [r for r in rows if "copyBuffer" in r[1]]
        if not copies:
            raise SystemExit("no calibration copy in %s (run with --copy-probe-mib)" % path)
        factor = probe / (copies[0][2] * 1024.0)
        res[key + "_factor"] = round(factor, 4)
        step_labels = {ln.label for ln in wl_obj.launches}
        for label, frags in KERNEL_NAMES.items():
            if label not in step_labels:
                continue  # e.g. set-up dispatches outside the step (the FP8 cache)
            frags = (frags,) if isinstance(frags, str) else frags
            # per launch: for each kernel the launch dispatches, the average
            # over its dispatches times the dispatches one launch makes
            per = max(ln.dispatches for ln in wl_obj.launches if ln.label == label)
            total, seen = 0.0, 0
            for frag in frags:
                vals = [r[2] for r in rows if frag in r[1]]
                if vals:
                    total += sum(vals) / len(vals) * per
                    seen += len(vals)
            if seen:
                ent = res.setdefault("kernels", {}).setdefault(label, {})
                ent[key + "_bytes"] = round(total * 1024.0 * factor)
                ent["dispatches"] = seen
    for label, ent in res.get("kernels", {}).items():
        ent["traffic_bytes"] = ent.get("fetch_bytes", 0) + ent.get("write_bytes", 0)
        alg = [ln.bytes for ln in wl_obj.launches if ln.label == label]
        ent["algorithmic_bytes"] = round(sum(alg) / len(alg))
        ent["ratio"] = round(ent["traffic_bytes"] / ent["algorithmic_bytes"], 3)
    data = {}
    try:
        with open(out_json) as f:
            data = json.load(f)
    except (OSError, ValueError):
        pass
    data[config] = res
    with open(out_json, "w") as f:
        json.dump(data, f, indent=1, sort_keys=True)
        f.write("\n")
    return res


MI355X_CUS = 256
MI355X_SIMDS = MI355X_CUS * 4   # 4 SIMDs per CU
PEAK_CLOCK_HZ = 2.4e9


def counter_table(path: str, wl_obj: Workload) -> str:
    """Markdown table of one rocprofv3 counter CSV of this script: for each
    kernel of the step, its dispatch count, mean duration and the mean of every
    counter over its dispatches. Derived columns where their counters are
    present:
    * MFMA busy at peak clock: SQ_VALU_MFMA_BUSY_CYCLES (MFMA pipe cycles,
      summed over the SIMDs) / (SIMDs x duration x 2.4 GHz);
    * waiting: SQ_WAIT_INST_ANY / SQ_WAVE_CYCLES, the share of wave cycles
      spent in s_waitcnt (SQ_WAIT_INST_LDS likewise, waits on LDS);
    * the memory path: the mean L1 -> L2 read latency in cycles
      (TCP_TCC_READ_REQ_LATENCY / TCP_TCC_READ_REQ), the L2 hit rate
      (TCC_HIT / (TCC_HIT + TCC_MISS)) and the share of L1 cycles stalled on
      data pending from L2 (TCP_PENDING_STALL_CYCLES over 256 L1s x duration x
      2.4 GHz, a lower bound when the clock runs below its peak)."""
    disp = {}
    with open(path, newline="") as f:
        for r in csv.DictReader(f):
            d = disp.setdefault(int(r["Dispatch_Id"]), {
                "name": r["Kernel_Name"], "ns": int(r["End_Timestamp"]) - int(r["Start_Timestamp"]), "c": {}})
            d["c"][r["Counter_Name"]] = d["c"].get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    counters = sorted({c for d in disp.values() for c in d["c"]})
    step_labels = [ln.label for ln in wl_obj.launches]
    head = ["kernel", "dispatches", "mean us"] + counters
    derived = []
    if "SQ_VALU_MFMA_BUSY_CYCLES" in counters:
        derived.append("MFMA busy at 2.4 GHz")
    if "SQ_WAIT_INST_ANY" in counters and "SQ_WAVE_CYCLES" in counters:
        derived.append("waiting (s_waitcnt)")
    if "SQ_WAIT_INST_LDS" in counters and "SQ_WAVE_CYCLES" in counters:
        derived.append("waiting on LDS")
    if "TCP_TCC_READ_REQ_LATENCY_sum" in counters and "TCP_TCC_READ_REQ_sum" in counters:
        derived.append("L1->L2 read latency (cycles)")
    if "TCC_HIT_sum" in counters and "TCC_MISS_sum" in counters:
        derived.append("L2 hit rate")
    if "TCP_PENDING_STALL_CYCLES_sum" in counters:
        derived.append("L1 stalled on L2 data")
    out = ["| " + " | ".join(head + derived) + " |", "|" + "---|" * (len(head) + len(derived))]
    rows = []
    for label, frags in KERNEL_NAMES.items():
        if label not in step_labels:
            continue
        frags = (frags,) if isinstance(frags, str) else frags
        for j, frag in enumerate(frags):   # one row per kernel the launch dispatches
            rows.append((label if j == 0 else "%s: %s" % (label, frag), frag))
    for label, frag in rows:
        ds = [d for d in disp.values() if frag in d["name"]]
        if not ds:
            continue
        ns = sum(d["ns"] for d in ds) / len(ds)
        mean = {c: sum(d["c"].get(c, 0.0) for d in ds) / len(ds) for c in counters}
        row = [label, str(len(ds)), "%.2f" % (ns / 1e3)] + ["%.0f" % mean[c] for c in counters]
        if "MFMA busy at 2.4 GHz" in derived:
            row.append("%.3f" % (mean["SQ_VALU_MFMA_BUSY_CYCLES"] / (MI355X_SIMDS * ns * 1e-9 * PEAK_CLOCK_HZ)))
        if "waiting (s_waitcnt)" in derived:
            row.append("%.3f" % (mean["SQ_WAIT_INST_ANY"] / max(mean["SQ_WAVE_CYCLES"], 1.0)))
        if "waiting on LDS" in derived:
            row.append("%.3f" % (mean["SQ_WAIT_INST_LDS"] / max(mean["SQ_WAVE_CYCLES"], 1.0)))
        if "L1->L2 read latency (cycles)" in derived:
            row.append("%.0f" % (mean["TCP_TCC_READ_REQ_LATENCY_sum"] / max(mean["TCP_TCC_READ_REQ_sum"], 1.0)))
        if "L2 hit rate" in derived:
            row.append("%.3f" % (mean["TCC_HIT_sum"] / max(mean["TCC_HIT_sum"] + mean["TCC_MISS_sum"], 1.0)))
        if "L1 stalled on L2 data" in derived:
            row.append("%.3f" % (mean["TCP_PENDING_STALL_CYCLES_sum"] / (MI355X_CUS * ns * 1e-9 * PEAK_CLOCK_HZ)))
        out.append("| " + " | ".join(row) + " |")
    return "\n".join(out)


def stored_traffic(path: str, config: str):
    """Counter figures for this config, or None when absent or taken on other kernels."""
    try:
        with open(path) as f:
            ent = json.load(f).get(config)
    except (OSError, ValueError):
        return None
    if not ent or ent.get("kernel_source") != kernel_source_digest():
        return None
    return ent.get("kernels")


# ------------------------------------------------------------------ device

HIP_ATTR_CLOCK_RATE_KHZ = 5        # hipDeviceAttributeClockRate
FP8_FLOP_PER_CLK_PER_CU = 8192     # dense FP8 MFMA: 4 SIMDs x 2048 FLOP per clock


def device_info() -> dict:
    """CU count, peak engine clock and the dense FP8 peak they imply (the
    reported roofline peak stays the published 5.0 PFLOP/s)."""
    import ctypes

    import torch
    props = torch.cuda.get_device_properties(0)
    info = {"name": props.name, "arch": props.gcnArchName, "cus": props.multi_processor_count}
    try:
        hip = ctypes.CDLL("libamdhip64.so")
        val = ctypes.c_int(0)
        if hip.hipDeviceGetAttribute(ctypes.byref(val), HIP_ATTR_CLOCK_RATE_KHZ,
                                     torch.cuda.current_device()) == 0:
            info["max_sclk_mhz"] = val.value / 1000.0
            info["fp8_peak_from_clock_tflops"] = round(
                info["cus"] * val.value * 1e3 * FP8_FLOP_PER_CLK_PER_CU / 1e12, 1)
    except OSError:
        pass
    return info


# -------------------------------------------------------------------- main

def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)
    import torch

    if args.counter_table:
        wl_obj = Workload(args.config, 1) if torch.cuda.is_available() else None
        if wl_obj is None:
            raise SystemExit("--counter-table needs the workload shapes, which are built on the GPU")
        print(counter_table(args.counter_table, wl_obj))
        return

    if args.pmc_summary:
        wl_obj = Workload(args.config, 1) if torch.cuda.is_available() else None
        if wl_obj is None:
            raise SystemExit("--pmc-summary needs the workload shapes, which are built on the GPU")
        print(json.dumps(pmc_summary(args.pmc_summary[0], args.pmc_summary[1], args.config,
                                     args.copy_probe_mib or 256, args.traffic_json, wl_obj)))
        return

    if args.copy_probe_mib:
        src = torch.ones(args.copy_probe_mib << 20, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    wl_obj = Workload(args.config, max(1, args.rotate), args.streams)
    stream = torch.cuda.current_stream()
    # Untimed pre-warm: the GPU ramps its clocks over the first tens of
    # milliseconds of sustained work; run steps for a while before the W
    # warmup steps so the timed steps see steady-state clocks.
    t_pre = time.perf_counter()
    while time.perf_counter() - t_pre < args.prewarm_s:
        for _ in range(10):
            wl_obj.step()
        torch.cuda.synchronize()
    for _ in range(args.warmup):
        wl_obj.step()
    torch.cuda.synchronize()

    nl = len(wl_obj.launches)
    gi = [ln.label for ln in wl_obj.launches].index("gemm")

    def pair():
        return (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))

    # Timed region: K steps. Only the dominant kernel (the GEMM) is bracketed
    # by an event pair, for its roofline; every pair costs the step GPU time
    # (measured ~5 us), so the other launches are not bracketed here.
    evs = [[pair() if i == gi else None for i in range(nl)] for _ in range(args.steps)]
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    start.record(stream)
    for i in range(args.steps):
        wl_obj.step(evs[i])
    t_host = time.perf_counter() - t_wall
    stop.record(stream)
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall
    ms = start.elapsed_time(stop) / args.steps
    gemm_timed = sorted(e[gi][0].elapsed_time(e[gi][1]) for e in evs)
    gemm_ms = sum(gemm_timed) / len(gemm_timed)

    # Per-launch figures: a second pass of K steps, outside the timed region,
    # with every launch bracketed.
    evs_all = [[pair() for _ in range(nl)] for _ in range(args.steps)]
    for i in range(args.steps):
        wl_obj.step(evs_all[i])
    torch.cuda.synchronize()
    per_launch = [sorted(e[i][0].elapsed_time(e[i][1]) for e in evs_all) for i in range(nl)]
    launch_ms = [sum(v) / len(v) for v in per_launch]

    value = wl_obj.flops / (ms * 1e-3) / 1e12
    traffic = stored_traffic(args.traffic_json, args.config)
    kernels = {}
    for ln, t, v in zip(wl_obj.launches, launch_ms, per_launch):
        key = ln.label if ln.label not in kernels else ln.label + "_b"
        ent = {"ms": round(t, 4), "ms_median": round(v[len(v) // 2], 4), "ms_min": round(v[0], 4),
               "algorithmic_bytes": int(ln.bytes),
               "hbm_gbs": round(ln.bytes / (t * 1e-3) / 1e9, 1),
               "hbm_frac": round(ln.bytes / (t * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
        if ln.flops:
            ent["tflops"] = round(ln.flops / (t * 1e-3) / 1e12, 2)
        single = sum(1 for o in wl_obj.launches if o.label == ln.label) == 1
        if traffic and single and ln.label in traffic:
            ent["traffic_bytes"] = traffic[ln.label]["traffic_bytes"]
        kernels[key] = ent
    gemm = (wl_obj.launches[gi], gemm_ms)   # from the timed region
    gemm_tflops = gemm[0].flops / (gemm[1] * 1e-3) / 1e12
    gemm_gbs = gemm[0].bytes / (gemm[1] * 1e-3) / 1e9

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
        "dtype": "fp8-e4m3 x fp8-e4m3 -> fp32 accumulate, " + (
            "fp32 out" if args.config in ("wgrad", "wgrad_cached", "grouped_wgrad", "grouped_wgrad_cached")
            else "bf16 out"),
        "data": "synthetic (seeded; see workloads/)",
        "config": wl_obj.desc,
        "pct_of_fp8_peak": round(100.0 * value / FP8_DENSE_PEAK_TFLOPS, 2),
        "roofline": dict(({
            "bound": "mfma",
            "achieved": round(gemm_tflops, 2),
            "peak": FP8_DENSE_PEAK_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(gemm_tflops / FP8_DENSE_PEAK_TFLOPS, 4),
        } if wl_obj.bound == "mfma" else {
            "bound": "hbm",
            "achieved": round(gemm_gbs, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(gemm_gbs / HBM_PEAK_GBS, 4),
        }), **{
            "traffic": traffic["gemm"]["traffic_bytes"] if traffic and "gemm" in traffic else None,
            "kernel": "gemm_kernel" + ({"grouped_fprop": " (grouped over M) + grouped_fixup_kernel",
                                        "grouped_dgrad": " (grouped over M) + grouped_fixup_kernel",
                                        "grouped_wgrad": " (grouped over K)",
                                        "grouped_wgrad_cached": " (grouped over K)",
                                        "mx_fprop": " (microscaling)"}.get(args.config, "")),
            "algorithmic_bytes": int(gemm[0].bytes),
            "algorithmic_flops": int(gemm[0].flops),
            # both roofs, whichever binds: dense FP8 MFMA and HBM
            "mfma": {"achieved": round(gemm_tflops, 2), "peak": FP8_DENSE_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(gemm_tflops / FP8_DENSE_PEAK_TFLOPS, 4)},
            "hbm": {"achieved": round(gemm_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": round(gemm_gbs / HBM_PEAK_GBS, 4)},
            "ms": round(gemm_ms, 4),
            "ms_median": round(gemm_timed[len(gemm_timed) // 2], 4),
            "timing": "event pair around every GEMM launch of the timed steps",
        }),
        # every launch of a second, untimed pass of the same steps, each
        # bracketed by its own event pair
        "kernels": kernels,
        "device": device_info(),
        "wall_s": round(t_wall, 3),
        "host_enqueue_ms_per_step": round(t_host * 1e3 / args.steps, 4),
    }
    if not args.no_cpu_baseline and wl_obj.host is not None:
        out["cpu_baseline"] = cpu_baseline(wl_obj)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
