"""GPU parity of the grouped launcher on the two FP8-matrix-core datapaths
(puro_fp8_gemm_grouped_mx, puro_fp8_gemm_grouped_native): several products,
K-segment sums and an accumulate-into output in one call, each against the
oracle's FP64 blockwise product (oracle.gemm_segments) of the same codes and
scales, within the matrix-core bound of the single-call variants:
    |C - C_ref| <= 2^-9 C_abs + (4 KB + 4) 2^-23 C_abs (+ 2^-23 |C_old| with accumulate)
with C_abs the oracle's blockwise product of |codes| and |scales| summed over the
segments and KB the problem's total K blocks, plus one BF16 rounding for BF16
outputs.  MX takes the power-of-two quantisers' codes and scales, native the
amax / 448 ones.  The group mixes 128x128-tile problems with ones eligible for
256x256 tiles, and its equally deep single-segment problems exercise the
launch-wide split of tiles over the XCDs.
"""
import numpy as np
import pytest
import torch

import blockwise_fp8_gemm_amd as pf
import oracle
import synth
from helpers import bf16_to_f64, first_mismatch, host, rel_frobenius, to_dev

pytestmark = pytest.mark.gpu

RULE = {"mx": "pow2", "native": "amax448"}


def _operands(layout, bgran, X, W, dp):
    """Quantise logical X [M][K] and W [N][K] into `layout`'s storage, on the host (oracle)
    and on the device (library; byte-exact, checked)."""
    p2 = dp == "mx"
    rule = {"rule": "pow2"} if p2 else {}
    if layout == "NT":
        ha = oracle.quant_act(X, **rule)
        da = pf.puro_fp8_quant_act(to_dev(X), pow2=p2)
        hb = oracle.quant_weight(W, **rule) if bgran == "128x128" else oracle.quant_act(W, **rule)
        db = (pf.puro_fp8_quant_weight(to_dev(W), pow2=p2) if bgran == "128x128"
              else pf.puro_fp8_quant_act(to_dev(W), pow2=p2))
    else:
        Wkn = np.ascontiguousarray(W.T)
        if layout == "NN":
            ha, da = oracle.quant_act(X, **rule), pf.puro_fp8_quant_act(to_dev(X), pow2=p2)
        else:
            Xkm = np.ascontiguousarray(X.T)
            ha = oracle.quant_transpose(Xkm, False, **rule)
            da = pf.puro_fp8_quant_transpose(to_dev(Xkm), False, pow2=p2)
        if bgran == "128x128":
            hb, db = oracle.quant_weight(Wkn, **rule), pf.puro_fp8_quant_weight(to_dev(Wkn), pow2=p2)
        else:
            hb = oracle.quant_transpose(Wkn, False, **rule)
            db = pf.puro_fp8_quant_transpose(to_dev(Wkn), False, pow2=p2)
    torch.cuda.synchronize()
    hosts, devs = tuple(ha) + tuple(hb), tuple(da) + tuple(db)
    for t, r in zip(devs, hosts):
        got = host(t)
        if got.dtype == np.float32:
            got, r = got.view(np.uint32), np.asarray(r).view(np.uint32)
        assert first_mismatch(got, r) is None, "operand"
    return hosts, devs


# (M, N, segment Ks, accumulate): equally deep single-segment problems (tile count a
# multiple of 8 on 128x128 tiles), a 256x256-eligible one, a two-segment sum, an
# accumulate-into output
GROUP = [(256, 256, (512,), False), (384, 128, (512,), False), (128, 256, (512,), False),
         (512, 512, (256,), False), (256, 128, (256, 384), False), (256, 256, (384,), True)]


@pytest.mark.parametrize("out", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
@pytest.mark.parametrize("bgran", ["1x128", "128x128"])
@pytest.mark.parametrize("layout", ["NT", "NN", "TN"])
@pytest.mark.parametrize("dp", ["mx", "native"])
def test_grouped_fp8_datapaths_within_the_matrix_core_bound(dev, dp, layout, bgran, out):
    probs, refs = [], []
    for i, (M, N, ks, acc) in enumerate(GROUP):
        hs, ds = [], []
        for j, K in enumerate(ks):
            X = synth.normal((M, K), 1.0, 7100 + 10 * i + j)
            W = synth.normal((N, K), 0.02, 7200 + 10 * i + j)
            h, d = _operands(layout, bgran, X, W, dp)
            hs.append(h)
            ds.append(d)
        c_old = None
        prob = {"segments": ds}
        if acc:
            c_old = synth.normal((M, N), 1.0, 7300 + i)
            if out == torch.bfloat16:
                bits = synth.f32_to_bf16_bits(c_old)
                c_old = bf16_to_f64(bits)
                prob["C"] = to_dev(bits)
            else:
                prob["C"] = to_dev(c_old.astype(np.float32))
                c_old = c_old.astype(np.float32).astype(np.float64)
            prob["accumulate"] = True
        probs.append(prob)
        refs.append((hs, c_old, sum(ks) // 128))
    Cs = pf.puro_fp8_gemm_grouped(layout, probs, bgran=bgran, out_dtype=out, mx=dp == "mx", native=dp == "native")
    torch.cuda.synchronize()
    for (hs, c_old, KB), C in zip(refs, Cs):
        C_ref = oracle.gemm_segments(layout, hs, bgran, c_init=c_old)
        c_abs = oracle.gemm_segments(layout, [(qa & 0x7F, np.abs(sa), qb & 0x7F, np.abs(sb))
                                              for qa, sa, qb, sb in hs], bgran)
        E = (2.0 ** -9 + (4 * KB + 4) * 2.0 ** -23) * c_abs
        if c_old is not None:
            E = E + 2.0 ** -23 * np.abs(c_old)
        if out == torch.float32:
            got = host(C).astype(np.float64)
            assert rel_frobenius(got, C_ref) <= 1e-3
        else:
            got = bf16_to_f64(host(C))
            E = E + 2.0 ** -8 * (np.abs(C_ref) + E)
        bad = np.argwhere(np.abs(got - C_ref) > E)
        assert bad.size == 0, ("element bound", tuple(bad[0]))


@pytest.mark.parametrize("dp", ["mx", "native"])
def test_grouped_fp8_datapaths_equal_the_single_calls(dev, dp):
    """Grouped products equal the same products through the single-call entry point
    within the sum of both calls' bounds (both on the same datapath)."""
    ops = []
    for i, (M, N, K) in enumerate([(512, 512, 512), (256, 768, 512), (768, 256, 512)]):
        X = synth.normal((M, K), 1.0, 7400 + i)
        W = synth.normal((N, K), 0.02, 7500 + i)
        ops.append(_operands("NT", "128x128", X, W, dp))
    Cs = pf.puro_fp8_gemm_grouped("NT", [d for _, d in ops], bgran="128x128", out_dtype=torch.float32,
                                  mx=dp == "mx", native=dp == "native")
    for (hs, ds), C in zip(ops, Cs):
        C1 = pf.puro_fp8_gemm("NT", *ds, bgran="128x128", out_dtype=torch.float32, mx=dp == "mx",
                              native=dp == "native")
        torch.cuda.synchronize()
        qa, sa, qb, sb = hs
        c_abs = oracle.gemm("NT", qa & 0x7F, np.abs(sa), qb & 0x7F, np.abs(sb), "128x128")
        E = 2 * (2.0 ** -9 + (4 * 4 + 4) * 2.0 ** -23) * c_abs
        bad = np.argwhere(np.abs(host(C).astype(np.float64) - host(C1).astype(np.float64)) > E)
        assert bad.size == 0, tuple(bad[0])
