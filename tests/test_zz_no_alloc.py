"""The allocation-free grouped GEMM (fp8_grouped_gemm_noalloc, through the C
ABI) against fp8_grouped_gemm with a full workspace: two calls in a row on
the library's scratch, the second with a smaller input, each bit-identical
to the workspace entry point (same kernels, same K-split of the last round);
the small case also against the oracle. Collected last: it leaves the GPU's
scratch in use by the library."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import fine_grained_fp8_quantize_amd as fq
import oracle
import workloads as wl
from gpu_util import assert_grouped_close, dev_codes, dev_f32, host_out, nan_out

pytestmark = pytest.mark.gpu


def _inputs(rows, n, k, on_host):
    """Expert-sorted codes of the seeded grouped config, quantized on the host
    by the oracle (small case) or on the GPU (the MoE config)."""
    rows = np.asarray(rows, dtype=np.int64)
    g = wl.grouped_fprop(3, n=n, k=k, experts=len(rows), rows=rows)
    E = len(rows)
    if on_host:
        a_q, a_s = oracle.quant_act_1x128(g["x"])
        b_q = np.empty((E, n, k), np.uint8)
        b_s = np.empty((E, n // 128, k // 128), np.float32)
        for e in range(E):
            b_q[e], b_s[e] = oracle.quant_weight_128x128(g["w"][e])
        dev = (dev_codes(a_q), dev_f32(a_s), dev_codes(b_q), dev_f32(b_s))
        host = (a_q, a_s, b_q, b_s)
    else:
        x = torch.from_numpy(g["x"].view(np.int16)).cuda().view(torch.bfloat16)
        w = torch.from_numpy(g["w"].reshape(E * n, k).view(np.int16)).cuda().view(torch.bfloat16)
        a_q, a_s = fq.fp8_quantize_act(x)
        b_q, b_s = fq.fp8_quantize_weight(w)
        dev = (a_q, a_s, b_q.view(E, n, k), b_s.view(E, n // 128, k // 128))
        host = None
    off = g["offsets"]
    return rows, off, dev, host


def test_noalloc_matches_workspace_entry_point():
    full = torch.empty(fq.GROUPED_WORKSPACE_BYTES, dtype=torch.uint8, device="cuda")
    # the MoE config (816 tiles: a last round of 48, split into 5 K pieces),
    # then a smaller one (14 tiles, 4 pieces each) on the scratch the first left
    for rows, n, k, on_host in ((wl.moe_rows(0), 4096, 7168, False),
                                ([300, 5, 0, 128, 257, 40], 384, 18 * 128, True)):
        rows, off, (a_q, a_s, b_q, b_s), host = _inputs(rows, n, k, on_host)
        off_d = torch.from_numpy(off.astype(np.int32)).cuda()
        rows_d = torch.from_numpy(rows.astype(np.int32)).cuda()
        m_total = int(off[-1])
        c_ws = nan_out((m_total, n), torch.bfloat16)
        c_na = nan_out((m_total, n), torch.bfloat16)
        fq.fp8_grouped_gemm(off_d, rows_d, a_q, a_s, b_q, b_s, torch.bfloat16, out=c_ws, workspace=full)
        fq.fp8_grouped_gemm_noalloc(off_d, rows_d, a_q, a_s, b_q, b_s, torch.bfloat16, out=c_na)
        torch.cuda.synchronize()
        print("no-alloc call: %d experts, n=%d, k=%d, %d padded rows" % (len(rows), n, k, m_total), flush=True)
        assert torch.equal(c_na.view(torch.int16), c_ws.view(torch.int16)), "differs from fp8_grouped_gemm"
        if host is not None:
            ref = oracle.grouped_gemm(off, rows, *host)
            assert_grouped_close(host_out(c_na), ref, off, rows, "no-alloc grouped GEMM")
