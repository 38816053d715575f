"""GPU parity of puro_fp8_gemm_native: the recipe's amax/448 codes and scales,
block partials on the native FP8 matrix cores, promoted into FP32 per block.

The FP8 matrix cores add each run of 8 consecutive products in fixed point,
keeping bits down to about 13 places below the run's largest product
(measured on gfx950; the library header states it), so a block partial is not
FP32-exact.  Per element the truncation is below 8 * 2^-13 * max|product| <=
2^-10 * (sum of |products|) per run, and FP32 promotion adds at most
(KB + 4) 2^-23 C_abs.  The test bound is the one the power-of-two variant
uses, twice the truncation term plus four times the FP32 term:
    |C - C_ref| <= 2^-9 C_abs + (4 KB + 4) 2^-23 C_abs
with C_abs the oracle's blockwise product of |codes| and |scales|, plus one
BF16 rounding for BF16 outputs; and a relative Frobenius error of at most
1e-3 for FP32 outputs.  The FP32-exact entry point (puro_fp8_gemm) on the same
operands stays within 2e-6.
"""
import numpy as np
import pytest
import torch

import blockwise_fp8_gemm_amd as pf
import oracle
import synth
from helpers import bf16_to_f64, first_mismatch, host, rel_frobenius, to_dev

pytestmark = pytest.mark.gpu


def _same(t, ref, what):
    got = host(t)
    if got.dtype == np.float32:
        got, ref = got.view(np.uint32), np.asarray(ref).view(np.uint32)
    assert first_mismatch(got, ref) is None, (what, first_mismatch(got, ref))


def _operands(layout, bgran, X, W):
    """amax/448 quantisation of logical X [M][K] and W [N][K] into the storage form of
    `layout`, on the host (oracle) and on the device (library, checked byte-exact)."""
    if layout == "NT":
        host_ops = oracle.quant_act(X) + (oracle.quant_weight(W) if bgran == "128x128" else oracle.quant_act(W))
        dev_ops = pf.puro_fp8_quant_act(to_dev(X)) + (
            pf.puro_fp8_quant_weight(to_dev(W)) if bgran == "128x128" else pf.puro_fp8_quant_act(to_dev(W)))
    else:
        Wkn = np.ascontiguousarray(W.T)
        if layout == "NN":
            ha, da = oracle.quant_act(X), pf.puro_fp8_quant_act(to_dev(X))
        else:
            Xkm = np.ascontiguousarray(X.T)
            ha = oracle.quant_transpose(Xkm, False)
            da = pf.puro_fp8_quant_transpose(to_dev(Xkm), False)
        if bgran == "128x128":
            hb, db = oracle.quant_weight(Wkn), pf.puro_fp8_quant_weight(to_dev(Wkn))
        else:
            hb = oracle.quant_transpose(Wkn, False)
            db = pf.puro_fp8_quant_transpose(to_dev(Wkn), False)
        host_ops, dev_ops = ha + hb, da + db
    torch.cuda.synchronize()
    for t, r in zip(dev_ops, host_ops):
        _same(t, r, "operand")
    return host_ops, dev_ops


def _bound(c_abs, K):
    return (2.0 ** -9 + (4 * (K // 128) + 4) * 2.0 ** -23) * c_abs


SHAPES = [(256, 256, 512), (384, 128, 1024), (128, 256, 128), (256, 128, 4096), (256, 256, 16384)]


@pytest.mark.parametrize("out", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
@pytest.mark.parametrize("bgran", ["1x128", "128x128"])
@pytest.mark.parametrize("layout", ["NT", "NN", "TN"])
@pytest.mark.parametrize("M,N,K", SHAPES, ids=["%dx%dx%d" % s for s in SHAPES])
def test_native_gemm_within_the_matrix_core_bound(dev, M, N, K, layout, bgran, out):
    X = synth.normal((M, K), 1.0, 6100 + M + K)
    W = synth.normal((N, K), 0.02, 6200 + N + K)
    (qa, sa, qb, sb), dev_ops = _operands(layout, bgran, X, W)
    C = pf.puro_fp8_gemm(layout, *dev_ops, bgran=bgran, out_dtype=out, native=True)
    torch.cuda.synchronize()
    C_ref = oracle.gemm(layout, qa, sa, qb, sb, bgran)
    E = _bound(oracle.gemm(layout, qa & 0x7F, np.abs(sa), qb & 0x7F, np.abs(sb), bgran), K)
    if out == torch.float32:
        got = host(C).astype(np.float64)
        assert rel_frobenius(got, C_ref) <= 1e-3
    else:
        got = bf16_to_f64(host(C))
        E = E + 2.0 ** -8 * (np.abs(C_ref) + E)
    bad = np.argwhere(np.abs(got - C_ref) > E)
    assert bad.size == 0, ("element bound", tuple(bad[0]))


def test_native_gemm_outliers_and_zero_blocks(dev):
    """Dynamic range: outlier channels, lognormal magnitudes and zero blocks (the
    outlier-stress recipe at a reduced token count)."""
    T, C_in, C_out = 1024, 768, 256
    X, _ = synth.outlier_activations(T, C_in, 6301)
    dY = synth.lognormal_gradients(T, C_out, 6302)
    (qa, sa, qb, sb), dev_ops = _operands("NT", "1x128", np.ascontiguousarray(dY.T), np.ascontiguousarray(X.T))
    C = pf.puro_fp8_gemm("NT", *dev_ops, bgran="1x128", out_dtype=torch.float32, native=True)
    torch.cuda.synchronize()
    C_ref = oracle.gemm("NT", qa, sa, qb, sb, "1x128")
    E = _bound(oracle.gemm("NT", qa & 0x7F, np.abs(sa), qb & 0x7F, np.abs(sb), "1x128"), T)
    got = host(C).astype(np.float64)
    bad = np.argwhere(np.abs(got - C_ref) > E)
    assert bad.size == 0, ("element bound", tuple(bad[0]))


@pytest.mark.parametrize("bgran", ["1x128", "128x128"])
def test_native_gemm_large_tiles(dev, bgran):
    """8192 x 2048 x 2048, the shape of the o projection's forward product, for which the
    planner takes 256 x 256 workgroup tiles: 3,000 sampled entries and the four corners."""
    M, N, K = 8192, 2048, 2048
    X = synth.normal((M, K), 1.0, 6401)
    W = synth.normal((N, K), 0.02, 6402)
    (qa, sa, qb, sb), dev_ops = _operands("NT", bgran, X, W)
    C = pf.puro_fp8_gemm("NT", *dev_ops, bgran=bgran, out_dtype=torch.float32, native=True)
    torch.cuda.synchronize()
    rng = np.random.default_rng(6403)
    ms, ns = rng.integers(0, M, 3000), rng.integers(0, N, 3000)
    ms[:4], ns[:4] = [0, 0, M - 1, M - 1], [0, N - 1, 0, N - 1]
    ref = oracle.gemm_entries("NT", qa, sa, qb, sb, bgran, ms, ns)
    E = _bound(oracle.gemm_entries("NT", qa & 0x7F, np.abs(sa), qb & 0x7F, np.abs(sb), bgran, ms, ns), K)
    got = host(C)[ms, ns].astype(np.float64)
    bad = np.flatnonzero(np.abs(got - ref) > E)
    assert bad.size == 0, ("entry", int(ms[bad[0]]), int(ns[bad[0]]), got[bad[0]], ref[bad[0]])
    assert rel_frobenius(got, ref) <= 1e-3


def test_exact_path_on_large_tiles(dev):
    """The FP32-exact entry point on a product its planner runs on 256 x 256 tiles
    (NT, 128x128 B scales, K = 4096): 3,000 sampled entries within its per-element
    bound (KB + 4) 2^-23 C_abs and 2e-6 relative Frobenius."""
    M, N, K = 4096, 4096, 4096
    X = synth.normal((M, K), 1.0, 6501)
    W = synth.normal((N, K), 0.02, 6502)
    (qa, sa, qb, sb), dev_ops = _operands("NT", "128x128", X, W)
    for out in (torch.float32, torch.bfloat16):
        C = pf.puro_fp8_gemm("NT", *dev_ops, bgran="128x128", out_dtype=out)
        torch.cuda.synchronize()
        rng = np.random.default_rng(6503)
        ms, ns = rng.integers(0, M, 3000), rng.integers(0, N, 3000)
        ms[:4], ns[:4] = [0, 0, M - 1, M - 1], [0, N - 1, 0, N - 1]
        ref = oracle.gemm_entries("NT", qa, sa, qb, sb, "128x128", ms, ns)
        c_abs = oracle.gemm_entries("NT", qa & 0x7F, np.abs(sa), qb & 0x7F, np.abs(sb), "128x128", ms, ns)
        E = (K // 128 + 4) * 2.0 ** -23 * c_abs
        if out == torch.float32:
            got = host(C)[ms, ns].astype(np.float64)
            assert rel_frobenius(got, ref) <= 2e-6
        else:
            got = bf16_to_f64(host(C)[ms, ns])
            E = E + 2.0 ** -8 * (np.abs(ref) + E)
        bad = np.flatnonzero(np.abs(got - ref) > E)
        assert bad.size == 0, ("entry", out, int(ms[bad[0]]), int(ns[bad[0]]), got[bad[0]], ref[bad[0]])


def test_native_gemm_agrees_with_the_exact_path(dev):
    M, N, K = 512, 384, 2048
    X = synth.normal((M, K), 1.0, 6601)
    W = synth.normal((N, K), 0.02, 6602)
    (qa, sa, qb, sb), dev_ops = _operands("NT", "128x128", X, W)
    C1 = pf.puro_fp8_gemm("NT", *dev_ops, bgran="128x128", out_dtype=torch.float32)
    C2 = pf.puro_fp8_gemm("NT", *dev_ops, bgran="128x128", out_dtype=torch.float32, native=True)
    torch.cuda.synchronize()
    C_ref = oracle.gemm("NT", qa, sa, qb, sb, "128x128")
    assert rel_frobenius(host(C1).astype(np.float64), C_ref) <= 2e-6
    c_abs = oracle.gemm("NT", qa & 0x7F, np.abs(sa), qb & 0x7F, np.abs(sb), "128x128")
    E = _bound(c_abs, K) + (K // 128 + 4) * 2.0 ** -23 * c_abs
    assert (np.abs(host(C1).astype(np.float64) - host(C2).astype(np.float64)) <= E).all()
