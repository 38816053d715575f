"""Pins for the oracle's E4M3 codec (CPU only).

The codec follows the E4M3 definition of the FP8-formats paper (Micikevicius
et al., 2022) cited by the Puro-2B report.  It is pinned against
  * that paper's table of reference points (tests/golden/e4m3_format.txt),
  * PyTorch's float8_e4m3fn conversions, an independent library routine:
    decoding of all 256 codes, and encoding of every finite FP32 value with
    |y| <= 512 (exhaustive) once inputs are clamped to +-448 (torch's cast is
    round-to-nearest-even but not saturating), and
  * values that follow from the definition by hand (ties to even, saturation).
"""
import math
import os

import numpy as np
import pytest
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "e4m3_format.txt")


def _golden():
    rows = []
    with open(GOLDEN) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            name, code, value = line.split()
            rows.append((name, int(code, 16), float(value)))
    return rows


def test_golden_reference_points_decode():
    for name, code, value in _golden():
        got = oracle.e4m3_decode(np.array([code], np.uint8))[0]
        if math.isnan(value):
            assert math.isnan(got), name
        else:
            assert got == value and math.copysign(1, got) == math.copysign(1, value), name


def test_golden_reference_points_encode():
    for name, code, value in _golden():
        if math.isnan(value):
            continue
        got = oracle.e4m3_encode(np.array([value], np.float32))[0]
        assert got == code, (name, hex(got))


def test_decode_all_codes_vs_torch():
    codes = np.arange(256, dtype=np.uint8)
    ours = oracle.e4m3_decode(codes)
    theirs = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(theirs)
    assert (np.isnan(ours) == nan).all()
    assert (np.flatnonzero(nan) == [0x7F, 0xFF]).all()
    np.testing.assert_array_equal(ours[~nan], theirs[~nan])
    assert np.nanmax(ours) == 448.0


def test_encode_exhaustive_vs_torch():
    """Every FP32 bit pattern from +0 up to 512.0, and its negation."""
    top = np.float32(512.0).view(np.uint32)
    step = 1 << 24
    for start in range(0, int(top) + 1, step):
        bits = np.arange(start, min(start + step, int(top) + 1), dtype=np.uint32)
        for sign in (0, 0x80000000):
            y = (bits | np.uint32(sign)).view(np.float32)
            ours = oracle.e4m3_encode(y)
            ref = torch.from_numpy(y).clamp(-448.0, 448.0).to(torch.float8_e4m3fn)
            ref = ref.view(torch.uint8).numpy()
            bad = np.flatnonzero(ours != ref)
            assert bad.size == 0, "first mismatch at y=%r: ours 0x%02x torch 0x%02x" % (
                float(y[bad[0]]), ours[bad[0]], ref[bad[0]])


def test_encode_saturates_above_448():
    rng = np.random.default_rng(1)
    big = np.concatenate([np.float32([448.0, 449.0, 464.0, 465.0, 480.0, 1e6, 3.4e38]),
                          rng.uniform(448, 1e30, 1000).astype(np.float32)])
    assert (oracle.e4m3_encode(big) == 0x7E).all()
    assert (oracle.e4m3_encode(-big) == 0xFE).all()


@pytest.mark.parametrize("value,code", [
    (432.0, 0x7E),            # midpoint of 416 (odd mantissa 5) and 448 (even 6): to 448
    (2.0 ** -10, 0x00),       # midpoint of 0 and the smallest subnormal: to 0
    (3 * 2.0 ** -11, 0x01),   # 1.5 * 2^-10 is past half the subnormal spacing 2^-9: to 2^-9
    (1.0625, 0x38),           # midpoint of 1 (0x38) and 1.125 (0x39): to even 0x38
    (1.1875, 0x3A),           # midpoint of 1.125 (0x39) and 1.25 (0x3A): to even 0x3A
    (17.0, 0x58),             # midpoint of 16 (0x58) and 18 (0x59): to even 0x58
    (-0.0, 0x80),             # the sign of zero is kept
    (-1e-30, 0x80),           # negative values that round to zero keep the sign
])
def test_encode_by_hand(value, code):
    assert oracle.e4m3_encode(np.array([value], np.float32))[0] == code


def test_round_trip_all_finite_codes():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
    vals = oracle.e4m3_decode(codes).astype(np.float32)
    assert (oracle.e4m3_encode(vals) == codes).all()


def test_bf16_rne_matches_torch_on_fp32_inputs():
    """For FP32-representable inputs the double-to-BF16 rounding equals torch's FP32->BF16 cast."""
    rng = np.random.default_rng(2)
    x = np.concatenate([rng.standard_normal(200000).astype(np.float32) * 10.0 ** rng.integers(-30, 30, 200000),
                        np.float32([0.0, -0.0, 1.0, 65504.0, 3e38, 1e-40, -1e-40])]).astype(np.float32)
    ours = oracle.bf16_rne(x.astype(np.float64))
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(ours, ref)


def test_bf16_rne_ties_and_double_inputs():
    # exact midpoints between neighbouring BF16 values go to the even pattern
    lo = np.arange(0x3F80, 0x3F80 + 64, dtype=np.uint32)
    a = (lo << 16).view(np.float32).astype(np.float64)
    b = ((lo + 1) << 16).view(np.float32).astype(np.float64)
    mid = (a + b) / 2
    got = oracle.bf16_rne(mid)
    want = np.where(lo % 2 == 0, lo, lo + 1).astype(np.uint16)
    np.testing.assert_array_equal(got, want)
    # a double just above a midpoint rounds up, just below rounds down (no FP32 double rounding)
    up = oracle.bf16_rne(np.nextafter(mid, np.inf))
    down = oracle.bf16_rne(np.nextafter(mid, -np.inf))
    np.testing.assert_array_equal(up, (lo + 1).astype(np.uint16))
    np.testing.assert_array_equal(down, lo.astype(np.uint16))
