"""Seeded random configurations of the quantisers against the oracle, byte for byte.

Each case draws extents from a list mixing tile multiples with ragged values,
the input type (FP32 or BF16), padded or tight leading dimensions, the scale
rule (the recipe's amax / 448 or the power-of-two one) and the value
distribution (normal, lognormal with zero blocks, or outlier channels), and runs
every quantiser entry point on the same input.
"""
import os

import numpy as np
import pytest
import torch

import blockwise_fp8_gemm_amd as pf
import oracle
import synth
from helpers import first_mismatch, host, to_dev

pytestmark = pytest.mark.gpu

EXTENTS = [1, 5, 16, 127, 128, 129, 200, 256, 300, 384, 640]
# number of seeded cases (a wider sweep: set PURO_RANDOM_CASES, e.g. 400)
CASES = int(os.environ.get("PURO_RANDOM_CASES", "24"))


def _same(t, ref, what):
    got = host(t)
    ref = np.asarray(ref)
    if got.dtype == np.float32:
        got, ref = got.view(np.uint32), ref.view(np.uint32)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    assert first_mismatch(got, ref) is None, (what, first_mismatch(got, ref))


def _input(rng, rows, cols, seed):
    kind = int(rng.integers(3))
    if kind == 0:
        x = synth.normal((rows, cols), float(10.0 ** rng.integers(-3, 3)), seed)
    elif kind == 1:
        x = np.exp(np.log(1e-6) + 2.0 * synth.normal((rows, cols), 1.0, seed).astype(np.float64)).astype(np.float32)
        if rows >= 128 and cols >= 128:
            synth.zero_blocks(x, seed + 1, 0.05)
    else:
        x = synth.normal((rows, cols), 1.0, seed)
        x[:, rng.integers(0, cols, max(1, cols // 64))] *= np.float32(100.0)
    return x


@pytest.mark.parametrize("seed", range(CASES))
def test_random_quantisers(dev, seed):
    rng = np.random.default_rng(9100 + seed)
    rows, cols = int(rng.choice(EXTENTS)), int(rng.choice(EXTENTS))
    bf16 = bool(rng.integers(2))
    rule = ["amax", "pow2"][rng.integers(2)]
    pow2 = rule == "pow2"
    x = _input(rng, rows, cols, 9200 + seed)
    if bf16:
        x = synth.f32_to_bf16_bits(x)
    ld = (cols + 15) // 16 * 16 + int(rng.integers(2)) * 16
    d = to_dev(x, ld=ld)
    q, s = pf.puro_fp8_quant_act(d, pow2=pow2)
    torch.cuda.synchronize()
    qr, sr = oracle.quant_act(x, rule=rule)
    _same(q, qr, "act q")
    _same(s, sr, "act s")
    q, s = pf.puro_fp8_quant_weight(d, pow2=pow2)
    torch.cuda.synchronize()
    qw, sw = oracle.quant_weight(x, rule=rule)
    _same(q, qw, "weight q")
    _same(s, sw, "weight s")
    for tr in (True, False):
        q, s = pf.puro_fp8_quant_transpose(d, tr, pow2=pow2)
        qd = pf.puro_fp8_quant_dual(d, tr, pow2=pow2)
        torch.cuda.synchronize()
        qt, st = oracle.quant_transpose(x, tr, rule=rule)
        _same(q, qt, ("transpose q", tr))
        _same(s, st, ("transpose s", tr))
        for t_, r_, w_ in zip(qd, (qr, sr, qt, st), ("dual q_row", "dual s_row", "dual q_tok", "dual s_tok")):
            _same(t_, r_, (w_, tr))
    # the weight quantiser's transposed copy
    (o,) = pf.puro_fp8_quant_weight_grouped([d], pow2=pow2, transposed=True)
    torch.cuda.synchronize()
    _same(o[0], qw, "grouped q")
    _same(o[1], sw, "grouped s")
    _same(o[2], np.ascontiguousarray(qw.T), "grouped qt")
    _same(o[3], np.ascontiguousarray(sw.T), "grouped st")
