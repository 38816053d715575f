"""GPU parity of the SiLU-gated activation fused into the dual quantiser.

h = BF16(silu(g) * u) is evaluated in FP32 by the kernel, so h is compared with
the oracle's FP64 value through the library's stated bound: every h must be
the BF16 rounding of some value within 2^-20 |h_exact| + 2^-149 (|g u| + 1) of
the exact one, and all but a sliver (values within that distance of a BF16
rounding midpoint) must equal the correctly rounded h_exact.  The codes and
scales are then bit-exact against the oracle's quantisers applied to the
kernel's own h: the quantisation decision is taken on the same BF16 values on
both sides.

Inputs: gate and up as the two halves of one [tokens][2 cols] product, N(0, 1)
like the gate/up projections of a Qwen3-1.7B layer (X ~ N(0, 1), W ~ N(0, 0.02),
K = 2048), a wide-gate case (N(0, 8)), every finite BF16 gate value, ragged
extents with padded rows, both token-copy layouts and both scale rules.
"""
import numpy as np
import pytest
import torch

import blockwise_fp8_gemm_amd as pf
import oracle
import synth
from helpers import bf16_to_f64, first_mismatch, host, to_dev

pytestmark = pytest.mark.gpu

EPS = 2.0 ** -20
ABS = 2.0 ** -149


def _check_h(h_bits, g_bits, u_bits, what, max_off=1e-3):
    exact = oracle.swiglu(g_bits, u_bits)
    gu = np.abs(bf16_to_f64(g_bits) * bf16_to_f64(u_bits))
    r = EPS * np.abs(exact) + ABS * (gu + 1.0)
    lo = bf16_to_f64(oracle.bf16_rne(exact - r))
    hi = bf16_to_f64(oracle.bf16_rne(exact + r))
    hv = bf16_to_f64(h_bits)
    bad = ~((hv >= lo) & (hv <= hi))
    if bad.any():
        i = np.argwhere(bad)[0]
        t = tuple(i)
        raise AssertionError("%s: h%s = %r outside [%r, %r] (exact %r, g %r, u %r)" % (
            what, t, hv[t], lo[t], hi[t], exact[t], bf16_to_f64(g_bits)[t], bf16_to_f64(u_bits)[t]))
    off = np.mean(bf16_to_f64(oracle.bf16_rne(exact)) != hv)
    assert off <= max_off, (what, "fraction not correctly rounded", off)


def _check_codes(h_bits, transpose_out, qr, sr, qt, st, what, rule="amax"):
    qr_ref, sr_ref = oracle.quant_act(h_bits, rule=rule)
    qt_ref, st_ref = oracle.quant_transpose(h_bits, transpose_out=transpose_out, rule=rule)
    for (q, s, q_ref, s_ref, part) in ((qr, sr, qr_ref, sr_ref, "rows"), (qt, st, qt_ref, st_ref, "tokens")):
        qg, sg = host(q), host(s)
        assert qg.shape == q_ref.shape and sg.shape == s_ref.shape, (what, part)
        assert first_mismatch(sg.view(np.uint32), s_ref.view(np.uint32)) is None, (
            what, part, "scale", first_mismatch(sg.view(np.uint32), s_ref.view(np.uint32)))
        assert first_mismatch(qg, q_ref) is None, (what, part, "codes", first_mismatch(qg, q_ref))


def _halves(tokens, cols, std, seed):
    """gate and up as the halves of one BF16 [tokens][2 cols] product."""
    gu = synth.normal((tokens, 2 * cols), std, seed, "bf16")
    return gu, gu[:, :cols], gu[:, cols:]


def _dev_halves(g, u):
    """gate and up side by side in one device buffer of padded rows (NaN in every gap), up
    starting at the first 16-element boundary after gate."""
    tokens, cols = g.shape
    off = (cols + 15) // 16 * 16
    ld = (off + cols + 15) // 16 * 16 + 16
    buf = torch.empty((tokens, ld), dtype=torch.int16, device="cuda:0").fill_(0x7FC0)
    buf[:, :cols] = torch.from_numpy(np.ascontiguousarray(g).view(np.int16)).to("cuda:0")
    buf[:, off:off + cols] = torch.from_numpy(np.ascontiguousarray(u).view(np.int16)).to("cuda:0")
    b = buf.view(torch.bfloat16)
    return b[:, :cols], b[:, off:off + cols]


def _all_finite_bf16_gates(seed):
    g = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    g[(g & 0x7F80) == 0x7F80] = 0        # Inf / NaN patterns -> 0 (inputs must be finite)
    u = np.clip(synth.normal((256, 256), 0.6, seed), -1.0, 1.0)   # |g u| stays finite
    return g.reshape(256, 256), synth.f32_to_bf16_bits(u)


CASES = [
    # name, tokens, cols, gate std, seed
    ("layer_halves", 1024, 6144, 1.0, synth.seed_of(5, 0, 1)),
    ("wide_gate", 512, 1024, 8.0, 301),
    ("ragged", 300, 200, 2.0, 302),
    ("one_tile_ragged", 129, 130, 1.0, 303),
]


@pytest.mark.parametrize("rule", ["amax", "pow2"])
@pytest.mark.parametrize("transpose_out", [True, False])
@pytest.mark.parametrize("name,tokens,cols,std,seed", CASES, ids=[c[0] for c in CASES])
def test_swiglu_quant_dual(dev, name, tokens, cols, std, seed, transpose_out, rule):
    gu, g, u = _halves(tokens, cols, std, seed)
    g_d, u_d = _dev_halves(g, u)
    h, qr, sr, qt, st = pf.puro_fp8_swiglu_quant_dual(g_d, u_d, transpose_out, pow2=(rule == "pow2"))
    torch.cuda.synchronize()
    hb = host(h)
    _check_h(hb, g, u, name)
    _check_codes(hb, transpose_out, qr, sr, qt, st, name, rule)


def test_swiglu_every_finite_gate(dev):
    """All 65,280 finite BF16 gate values (subnormals, +-0, the largest) against the bound."""
    g, u = _all_finite_bf16_gates(304)
    for u_bits in (u, np.full_like(u, 0x3F80)):          # random |u| <= 1, and u = 1
        h, qr, sr, qt, st = pf.puro_fp8_swiglu_quant_dual(to_dev(g), to_dev(u_bits), True)
        torch.cuda.synchronize()
        hb = host(h)
        _check_h(hb, g, u_bits, "every finite gate")
        _check_codes(hb, True, qr, sr, qt, st, "every finite gate")


def test_swiglu_without_h_and_padding_untouched(dev):
    """h = NULL gives the same codes; a padded h buffer is written only inside its rows."""
    tokens, cols = 384, 200
    gu, g, u = _halves(tokens, cols, 1.5, 305)
    gu_d = to_dev(gu)
    g_d, u_d = gu_d[:, :cols], gu_d[:, cols:]
    hbuf = torch.full((tokens, 208), 0, dtype=torch.int16, device="cuda:0")
    hbuf.fill_(0x5A5A)
    h_view = hbuf.view(torch.bfloat16)[:, :cols]
    for transpose_out in (True, False):
        h1, qr1, sr1, qt1, st1 = pf.puro_fp8_swiglu_quant_dual(g_d, u_d, transpose_out, h=h_view)
        n, qr2, sr2, qt2, st2 = pf.puro_fp8_swiglu_quant_dual(g_d, u_d, transpose_out, store_h=False)
        torch.cuda.synchronize()
        assert n is None
        assert (hbuf[:, cols:] == 0x5A5A).all()
        for a, b in ((qr1, qr2), (sr1, sr2), (qt1, qt2), (st1, st2)):
            assert torch.equal(a, b)
        hb = host(h1)
        _check_h(hb, g, u, "h view")
        _check_codes(hb, transpose_out, qr1, sr1, qt1, st1, "h view")


def test_swiglu_separate_buffers_equal_plain_dual(dev):
    """gate and up in separate tensors; the codes equal puro_fp8_quant_dual of the returned h."""
    tokens, cols = 512, 768
    g = synth.normal((tokens, cols), 1.0, 306, "bf16")
    u = synth.normal((tokens, cols), 1.0, 307, "bf16")
    h, qr, sr, qt, st = pf.puro_fp8_swiglu_quant_dual(to_dev(g), to_dev(u), True)
    qr2, sr2, qt2, st2 = pf.puro_fp8_quant_dual(h, True)
    torch.cuda.synchronize()
    for a, b in ((qr, qr2), (sr, sr2), (qt, qt2), (st, st2)):
        assert torch.equal(a, b)
    _check_h(host(h), g, u, "separate buffers")


def test_swiglu_full_size(dev):
    """The down projection's input of a Qwen3-1.7B layer at 8,192 tokens: gate and up as the
    halves of the [8192][12288] gate/up product; whole tensors checked."""
    tokens, cols = 8192, 6144
    gu, g, u = _halves(tokens, cols, 1.0, synth.seed_of(5, 0, 2))
    gu_d = to_dev(gu)
    h, qr, sr, qt, st = pf.puro_fp8_swiglu_quant_dual(gu_d[:, :cols], gu_d[:, cols:], True)
    torch.cuda.synchronize()
    hb = host(h)
    _check_h(hb, g, u, "full size")
    _check_codes(hb, True, qr, sr, qt, st, "full size")
