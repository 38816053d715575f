"""The allocation-free GEMM entry point (puro_fp8_gemm_noalloc), through the C ABI.

It takes no workspace: split-K partial sums go to the library's fixed device
array (PURO_NOALLOC_SCRATCH_BYTES per GPU).  Two calls in a row, the second
smaller, on products whose plans split K, must give exactly the bytes of
puro_fp8_gemm with a caller workspace (same plan and kernels), and stay within
the oracle's 2e-6 relative Frobenius bound; a plan needing more than the array
is rejected before anything is enqueued.
"""
import ctypes

import numpy as np
import pytest
import torch

import blockwise_fp8_gemm_amd as pf
import oracle
import synth
from helpers import host, rel_frobenius, to_dev

pytestmark = pytest.mark.gpu

SCRATCH = 64 << 20


def _noalloc(layout, A, sA, B, sB, bgran, C):
    """Direct C-ABI call; returns the status."""
    M, N, K = pf.gemm_dims(layout, A, B)
    L = pf.lib()
    return L.puro_fp8_gemm_noalloc(pf.LAYOUTS[layout], M, N, K, A.data_ptr(), A.stride(0), sA.data_ptr(),
                                   B.data_ptr(), B.stride(0), sB.data_ptr(), pf.BGRAN[bgran], C.data_ptr(),
                                   pf.PURO_BF16 if C.dtype == torch.bfloat16 else pf.PURO_F32, C.stride(0),
                                   ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))


def _weight_gradient_operands(M, N, K, seed):
    """Token-blocked copies of dY^T [M][K] and X^T [N][K] (1x128 along the tokens)."""
    dY = synth.normal((K, M), 1e-3, seed, "bf16")
    X = synth.normal((K, N), 1.0, seed + 1, "bf16")
    host_ops = oracle.quant_transpose(dY, True) + oracle.quant_transpose(X, True)
    dev_ops = pf.puro_fp8_quant_transpose(to_dev(dY), True) + pf.puro_fp8_quant_transpose(to_dev(X), True)
    return host_ops, dev_ops


@pytest.mark.parametrize("out", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
def test_two_calls_match_the_workspace_entry_point(dev, out):
    # the k projection's weight gradient (1024 x 2048, K = 8192), then a smaller product
    for (M, N, K), seed in (((1024, 2048, 8192), 7001), ((256, 384, 4096), 7011)):
        need = pf.puro_fp8_gemm_workspace_size("NT", M, N, K, "1x128")
        assert 0 < need <= SCRATCH, (M, N, K, need)
        (qa, sa, qb, sb), (dqa, dsa, dqb, dsb) = _weight_gradient_operands(M, N, K, seed)
        C = torch.full((M, N), float("nan"), dtype=out, device=dev)
        assert _noalloc("NT", dqa, dsa, dqb, dsb, "1x128", C) == pf.PURO_OK
        want = pf.puro_fp8_gemm("NT", dqa, dsa, dqb, dsb, bgran="1x128", out_dtype=out)
        torch.cuda.synchronize()
        got = host(C)
        assert np.array_equal(got.view(np.uint16 if out == torch.bfloat16 else np.uint32),
                              host(want).view(np.uint16 if out == torch.bfloat16 else np.uint32)), (M, N, K)
        if out == torch.float32:
            rng = np.random.default_rng(seed)
            ms, ns = rng.integers(0, M, 2000), rng.integers(0, N, 2000)
            ref = oracle.gemm_entries("NT", qa, sa, qb, sb, "1x128", ms, ns)
            assert rel_frobenius(got[ms, ns].astype(np.float64), ref) <= 2e-6


def test_plan_above_the_scratch_is_rejected(dev):
    M, N, K = 384, 5504, 16384
    assert pf.puro_fp8_gemm_workspace_size("NT", M, N, K, "1x128") > SCRATCH
    A = torch.zeros((M, K), dtype=torch.uint8, device=dev)
    B = torch.zeros((N, K), dtype=torch.uint8, device=dev)
    sA = torch.zeros((M, K // 128), dtype=torch.float32, device=dev)
    sB = torch.zeros((N, K // 128), dtype=torch.float32, device=dev)
    C = torch.full((M, N), 7.0, dtype=torch.float32, device=dev)
    assert _noalloc("NT", A, sA, B, sB, "1x128", C) == 5   # PURO_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert bool((C == 7.0).all())     # nothing was enqueued


def test_unsplit_products_and_the_binding(dev):
    # no split: the fixed array is not used; the Python wrapper marshals the same call
    M, N, K = 1024, 1024, 512
    (qa, sa, qb, sb), (dqa, dsa, dqb, dsb) = _weight_gradient_operands(M, N, K, 7021)
    assert pf.puro_fp8_gemm_workspace_size("NT", M, N, K, "1x128") == 0
    C = torch.empty((M, N), dtype=torch.float32, device=dev)
    pf.puro_fp8_gemm_noalloc("NT", dqa, dsa, dqb, dsb, C, bgran="1x128")
    torch.cuda.synchronize()
    assert rel_frobenius(host(C).astype(np.float64), oracle.gemm("NT", qa, sa, qb, sb, "1x128")) <= 2e-6
