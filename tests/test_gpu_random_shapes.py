"""Seeded random configurations of the GEMM entry points against the oracle.

Each case draws a layout, a B-scale granularity, an output type, extents from a
list that mixes tile multiples with ragged values (1, 7, 127, 129, ...), and
padded or tight leading dimensions; the grouped cases draw several problems of
1 to 3 K segments, some accumulating into an existing output.  Operands come
from the oracle's and the library's quantisers (byte-compared first); products
are held to the bounds of the fixed-shape tests (FP32: 2e-6 relative Frobenius
and the per-element accumulation bound; BF16: that bound plus one rounding).
"""
import os

import numpy as np
import pytest
import torch

import blockwise_fp8_gemm_amd as pf
import synth
from helpers import to_dev
from test_gpu_gemm import _check_product, _check_sum, _quantise_both

pytestmark = pytest.mark.gpu

EXTENTS = [1, 7, 64, 127, 128, 129, 200, 256, 383, 384, 512, 640]
KS = [1, 100, 128, 129, 255, 256, 384, 1000, 1024, 2048]
# number of seeded cases (a wider sweep: set PURO_RANDOM_CASES, e.g. 400)
CASES = int(os.environ.get("PURO_RANDOM_CASES", "24"))


def _case(seed):
    rng = np.random.default_rng(seed)
    layout = ["NT", "NN", "TN"][rng.integers(3)]
    bgran = ["1x128", "128x128"][rng.integers(2)]
    out = [torch.float32, torch.bfloat16][rng.integers(2)]
    M, N, K = int(rng.choice(EXTENTS)), int(rng.choice(EXTENTS)), int(rng.choice(KS))
    pad = int(rng.integers(2)) * 16
    return layout, bgran, out, M, N, K, pad


@pytest.mark.parametrize("seed", range(CASES))
def test_random_gemm(dev, seed):
    layout, bgran, out, M, N, K, pad = _case(8100 + seed)
    X = synth.normal((M, K), 1.0, 8200 + seed)
    W = synth.normal((N, K), 0.02, 8300 + seed)
    ld = (K + 15) // 16 * 16 + pad
    hostops, devops = _quantise_both(layout, bgran, X, W, ldx=ld, ldw=ld)
    _check_product(layout, bgran, hostops, devops, out)


@pytest.mark.parametrize("seed", range(max(1, CASES // 3)))
def test_random_grouped(dev, seed):
    """1-5 NT problems in one grouped call, 1-3 K segments each, some adding into C."""
    rng = np.random.default_rng(8400 + seed)
    bgran = ["1x128", "128x128"][rng.integers(2)]
    out = [torch.float32, torch.bfloat16][rng.integers(2)]
    probs, checks = [], []
    for p in range(int(rng.integers(1, 6))):
        M, N = int(rng.choice(EXTENTS)), int(rng.choice(EXTENTS))
        segs_host, segs_dev = [], []
        for s in range(int(rng.integers(1, 4))):
            K = int(rng.choice(KS))
            X = synth.normal((M, K), 1.0, 8500 + 100 * seed + 10 * p + s)
            W = synth.normal((N, K), 0.02, 8600 + 100 * seed + 10 * p + s)
            h, d = _quantise_both("NT", bgran, X, W, ldx=(K + 15) // 16 * 16, ldw=(K + 15) // 16 * 16)
            segs_host.append(h)
            segs_dev.append(d)
        accumulate = bool(rng.integers(2))
        c_old = None
        C = None
        if accumulate:
            c_old_f = synth.normal((M, N), 1.0, 8700 + 100 * seed + p)
            if out == torch.bfloat16:
                bits = synth.f32_to_bf16_bits(c_old_f)
                C = to_dev(bits, ld=(N + 15) // 16 * 16)
                c_old = (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
            else:
                C = to_dev(c_old_f, ld=(N + 15) // 16 * 16)
                c_old = c_old_f.astype(np.float64)
        prob = {"segments": segs_dev, "accumulate": accumulate}
        if C is not None:
            prob["C"] = C
        probs.append(prob)
        checks.append((segs_host, c_old))
    Cs = pf.puro_fp8_gemm_grouped("NT", probs, bgran=bgran, out_dtype=out)
    torch.cuda.synchronize()
    for (segs_host, c_old), C in zip(checks, Cs):
        _check_sum("NT", bgran, segs_host, C, out, c_old=c_old)
