"""GPU parity of the per-tensor GEMM (fp8_gemm_tensor, whole-K accumulation
in the MFMA accumulators) and the accumulation study at K = 4096.

Parity: against the exact float64 oracle (oracle.gemm_tensor), to the same
tolerance as the block-scaled GEMM. Study: every arm stays close to the
exact sum (see tests/accum_study.py for the arms and metrics).
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import accum_study
import fine_grained_fp8_quantize_amd as fq
import oracle
from gpu_util import assert_gemm_close, dev_codes, host_out, nan_out

pytestmark = pytest.mark.gpu


def _codes(seed, rows, k):
    rng = np.random.default_rng(seed)
    finite = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], np.uint8)
    return rng.choice(finite, size=(rows, k)).astype(np.uint8)


@pytest.mark.parametrize("m,n,k", [(300, 200, 384), (17, 129, 128), (256, 256, 1024), (513, 7, 256)])
@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float32])
def test_gemm_tensor_ragged(m, n, k, out_dtype):
    qa, qb = _codes(m + k, m, k), _codes(n + k + 1, n, k)
    sa, sb = np.float32(3.7e-3), np.float32(0.021)
    ldc = (n + 7) // 8 * 8                                   # output rows 16-byte aligned
    c = torch.full((m, ldc), float("nan"), dtype=out_dtype, device="cuda")
    fq.fp8_gemm_tensor(dev_codes(qa), torch.tensor([sa], device="cuda"), dev_codes(qb),
                       torch.tensor([sb], device="cuda"), out_dtype, out=c[:, :n])
    torch.cuda.synchronize()
    got = host_out(c)
    assert np.all(np.isnan(got[:, n:])), "columns past n written"
    assert_gemm_close(got[:, :n], oracle.gemm_tensor(qa, sa, qb, sb), "tensor %dx%dx%d" % (m, n, k))


def test_gemm_tensor_full_size():
    """The Dense Fprop shape (4096 x 4096 x 7168), every element."""
    qa, qb = _codes(5, 4096, 7168), _codes(6, 4096, 7168)
    c = fq.fp8_gemm_tensor(dev_codes(qa), torch.tensor([0.5], device="cuda"), dev_codes(qb),
                           torch.tensor([0.25], device="cuda"), torch.bfloat16,
                           out=nan_out((4096, 4096), torch.bfloat16))
    torch.cuda.synchronize()
    assert_gemm_close(host_out(c), oracle.gemm_tensor(qa, 0.5, qb, 0.25), "tensor full size")


def test_gemm_tensor_k0_writes_zeros():
    c = torch.full((40, 24), 5.0, dtype=torch.float32, device="cuda")
    a = torch.empty((40, 0), dtype=torch.uint8, device="cuda")
    b = torch.empty((24, 0), dtype=torch.uint8, device="cuda")
    s = torch.ones(1, dtype=torch.float32, device="cuda")
    fq.fp8_gemm_tensor(a, s, b, s, torch.float32, out=c)
    torch.cuda.synchronize()
    assert torch.all(c == 0)


@pytest.mark.parametrize("positive", [False, True])
def test_accumulation_study_k4096(positive):
    """Each arm's FP32 result of a K = 4096 GEMM of random FP8 matrices is
    within a few FP32 roundings of the exact sum: far from the H800 figure."""
    r = accum_study.run(1024, 1024, 4096, positive)
    print(r)
    for arm, e in r["arms"].items():
        assert e["normwise"] < 1e-4, (arm, e)
        assert e["max_rel_cond"] < 1e-3, (arm, e)
    # promotion every slab buys nothing over chaining the MFMA accumulator
    chain, slab = r["arms"]["mfma_chain"]["normwise"], r["arms"]["slab_promotion"]["normwise"]
    assert abs(chain - slab) <= 0.1 * slab, (chain, slab)


def test_gemm_tensor_224_wide_tiles():
    """N = 7168 makes the launcher pick 224-wide n tiles (32 x 224)."""
    qa, qb = _codes(11, 512, 256), _codes(12, 7168, 256)
    c = fq.fp8_gemm_tensor(dev_codes(qa), torch.tensor([0.75], device="cuda"), dev_codes(qb),
                           torch.tensor([1.5], device="cuda"), torch.float32,
                           out=nan_out((512, 7168), torch.float32))
    torch.cuda.synchronize()
    assert_gemm_close(host_out(c), oracle.gemm_tensor(qa, 0.75, qb, 1.5), "tensor 224-wide")
