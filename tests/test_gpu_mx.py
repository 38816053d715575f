"""GPU parity of the power-of-two scale variant (the scaled FP8 matrix cores).

Quantisers: byte-exact against the oracle's power-of-two rule (codes and scale
bits), on workload shapes, ragged shapes, zero blocks and blocks at the low end
of the E8M0 range.

GEMM (puro_fp8_gemm_mx): the oracle's FP64 blockwise product of the same codes
and scales.  The FP8 matrix cores add each run of 8 products in fixed point,
keeping bits down to 13 places below the run's largest product (measured on
gfx950, see the library header), so per element the error is below
8 * 2^-13 * max|product| <= 2^-10 * (sum of |products|) per run, plus FP32
accumulation.  The test bound is twice that:
    |C - C_ref| <= 2^-9 * C_abs + (4 KB + 4) 2^-23 * C_abs
with C_abs the oracle's product of |codes| and |scales|, plus one BF16
rounding for BF16 outputs.
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


def _inputs(rows, cols, seed, kind):
    x = synth.normal((rows, cols), 1.0, seed)
    if kind == "zeros_and_tiny":
        x[: rows // 2, : min(cols, 128)] = 0.0
        x[rows // 2:, : min(cols, 128)] *= np.float32(1e-38)   # amax/448 below 2^-127: range limit
    elif kind == "outliers":
        x[:, 3] *= 1e4
    return x


QSHAPES = [(256, 512), (200, 136), (8192, 2048), (130, 1000)]


@pytest.mark.parametrize("kind", ["normal", "zeros_and_tiny", "outliers"])
@pytest.mark.parametrize("rows,cols", QSHAPES, ids=["%dx%d" % s for s in QSHAPES])
def test_pow2_quantisers_bit_exact(dev, rows, cols, kind):
    x = _inputs(rows, cols, 5000 + rows + cols, kind)
    xb = synth.f32_to_bf16_bits(x)
    for xin, what in ((x, "f32"), (xb, "bf16")):
        d = to_dev(xin, ld=(cols + 15) // 16 * 16)
        q, s = pf.puro_fp8_quant_act(d, pow2=True)
        _same(q, oracle.quant_act(xin, rule="pow2")[0], ("act q", what))
        _same(s, oracle.quant_act(xin, rule="pow2")[1], ("act s", what))
        for tr in (True, False):
            rq, rs = oracle.quant_transpose(xin, tr, rule="pow2")
            q, s = pf.puro_fp8_quant_transpose(d, tr, pow2=True)
            _same(q, rq, ("transpose q", tr, what))
            _same(s, rs, ("transpose s", tr, what))
            qr, sr, qt, st = pf.puro_fp8_quant_dual(d, tr, pow2=True)
            ra = oracle.quant_act(xin, rule="pow2")
            for t_, r_, w_ in ((qr, ra[0], "dual q_row"), (sr, ra[1], "dual s_row"), (qt, rq, "dual q_tok"),
                               (st, rs, "dual s_tok")):
                _same(t_, r_, (w_, tr, what))
    rq, rs = oracle.quant_weight(x, rule="pow2")
    q, s = pf.puro_fp8_quant_weight(to_dev(x, ld=(cols + 15) // 16 * 16), pow2=True)
    _same(q, rq, "weight q")
    _same(s, rs, "weight s")


def _operands(layout, bgran, X, W):
    """Power-of-two quantisation of logical X [M][K] and W [N][K] into the storage form of
    `layout`, on the host (oracle) and on the device (library, checked byte-exact)."""
    if layout == "NT":
        host_ops = oracle.quant_act(X, rule="pow2") + (oracle.quant_weight(W, rule="pow2") if bgran == "128x128"
                                                         else oracle.quant_act(W, rule="pow2"))
        dev_ops = pf.puro_fp8_quant_act(to_dev(X), pow2=True) + (
            pf.puro_fp8_quant_weight(to_dev(W), pow2=True) if bgran == "128x128"
            else pf.puro_fp8_quant_act(to_dev(W), pow2=True))
    else:
        Wkn = np.ascontiguousarray(W.T)
        if layout == "NN":
            ha, da = oracle.quant_act(X, rule="pow2"), pf.puro_fp8_quant_act(to_dev(X), pow2=True)
        else:
            Xkm = np.ascontiguousarray(X.T)
            ha = oracle.quant_transpose(Xkm, False, rule="pow2")
            da = pf.puro_fp8_quant_transpose(to_dev(Xkm), False, pow2=True)
        if bgran == "128x128":
            hb, db = oracle.quant_weight(Wkn, rule="pow2"), pf.puro_fp8_quant_weight(to_dev(Wkn), pow2=True)
        else:
            hb = oracle.quant_transpose(Wkn, False, rule="pow2")
            db = pf.puro_fp8_quant_transpose(to_dev(Wkn), False, pow2=True)
        host_ops, dev_ops = ha + hb, da + db
    torch.cuda.synchronize()
    for t, r in zip(dev_ops, host_ops):
        _same(t, r, "operand")
    return host_ops, dev_ops


MX_SHAPES = [(256, 256, 512), (384, 128, 1024), (128, 256, 128), (256, 128, 4096)]


@pytest.mark.parametrize("out", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
@pytest.mark.parametrize("bgran", ["1x128", "128x128"])
@pytest.mark.parametrize("layout", ["NT", "NN", "TN"])
@pytest.mark.parametrize("M,N,K", MX_SHAPES, ids=["%dx%dx%d" % s for s in MX_SHAPES])
def test_mx_gemm_within_the_matrix_core_bound(dev, M, N, K, layout, bgran, out):
    X = synth.normal((M, K), 1.0, 5100 + M + K)
    W = synth.normal((N, K), 0.02, 5200 + N + K)
    (qa, sa, qb, sb), dev_ops = _operands(layout, bgran, X, W)
    C = pf.puro_fp8_gemm(layout, *dev_ops, bgran=bgran, out_dtype=out, mx=True)
    torch.cuda.synchronize()
    C_ref = oracle.gemm(layout, qa, sa, qb, sb, bgran)
    c_abs = oracle.gemm(layout, qa & 0x7F, np.abs(sa), qb & 0x7F, np.abs(sb), bgran)
    E = (2.0 ** -9 + (4 * (K // 128) + 4) * 2.0 ** -23) * c_abs
    if out == torch.float32:
        got = host(C).astype(np.float64)
        assert rel_frobenius(got, C_ref) <= 1e-3
    else:
        got = bf16_to_f64(host(C))
        E = E + 2.0 ** -8 * (np.abs(C_ref) + E)
    bad = np.argwhere(np.abs(got - C_ref) > E)
    assert bad.size == 0, ("element bound", tuple(bad[0]))


@pytest.mark.parametrize("bgran", ["1x128", "128x128"])
@pytest.mark.parametrize("layout", ["NT", "NN", "TN"])
def test_mx_gemm_large_tiles(dev, layout, bgran):
    """A product large enough for the 256 x 256 workgroup tiles (4096 x 4096 x 256): 3,000
    sampled entries, including the four corners, within the same matrix-core bound."""
    M, N, K = 4096, 4096, 256
    X = synth.normal((M, K), 1.0, 5401)
    W = synth.normal((N, K), 0.02, 5402)
    (qa, sa, qb, sb), dev_ops = _operands(layout, bgran, X, W)
    C = pf.puro_fp8_gemm(layout, *dev_ops, bgran=bgran, out_dtype=torch.float32, mx=True)
    torch.cuda.synchronize()
    rng = np.random.default_rng(5403)
    ms, ns = rng.integers(0, M, 3000), rng.integers(0, N, 3000)
    ms[:4], ns[:4] = [0, 0, M - 1, M - 1], [0, N - 1, 0, N - 1]
    ref = oracle.gemm_entries(layout, qa, sa, qb, sb, bgran, ms, ns)
    c_abs = oracle.gemm_entries(layout, qa & 0x7F, np.abs(sa), qb & 0x7F, np.abs(sb), bgran, ms, ns)
    E = (2.0 ** -9 + (4 * (K // 128) + 4) * 2.0 ** -23) * c_abs
    got = host(C)[ms, ns].astype(np.float64)
    bad = np.flatnonzero(np.abs(got - ref) > E)
    assert bad.size == 0, ("entry", int(ms[bad[0]]), int(ns[bad[0]]), got[bad[0]], ref[bad[0]])
    assert rel_frobenius(got, ref) <= 1e-3


def test_mx_gemm_agrees_with_the_promoting_path(dev):
    # the same power-of-two codes and scales through puro_fp8_gemm (FP32-exact block
    # partials) and puro_fp8_gemm_mx: both within the matrix-core bound of each other
    M, N, K = 512, 384, 2048
    X = synth.normal((M, K), 1.0, 5301)
    W = synth.normal((N, K), 0.02, 5302)
    (qa, sa, qb, sb), dev_ops = _operands("NT", "128x128", X, W)
    C1 = pf.puro_fp8_gemm("NT", *dev_ops, bgran="128x128", out_dtype=torch.float32)
    C2 = pf.puro_fp8_gemm("NT", *dev_ops, bgran="128x128", out_dtype=torch.float32, mx=True)
    torch.cuda.synchronize()
    C_ref = oracle.gemm("NT", qa, sa, qb, sb, "128x128")
    assert rel_frobenius(host(C1).astype(np.float64), C_ref) <= 2e-6
    c_abs = oracle.gemm("NT", qa & 0x7F, np.abs(sa), qb & 0x7F, np.abs(sb), "128x128")
    E = (2.0 ** -9 + 2 * (4 * (K // 128) + 4) * 2.0 ** -23) * c_abs
    assert (np.abs(host(C1).astype(np.float64) - host(C2).astype(np.float64)) <= E).all()
