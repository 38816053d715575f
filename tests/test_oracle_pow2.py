"""Pins for the oracle's power-of-two scale rule (CPU only).

A variant for gfx950's scaled matrix cores, whose block scales are E8M0
powers of two: per block s = 2^k, k the smallest integer with 448 * 2^k >=
amax (k limited to [-127, 127]), q = E4M3(x / s).  Pinned by what that
definition fixes:
  * s is a power of two; for blocks not at the range limit, 224 < amax / s <= 448,
    and s equals the recipe's fl32(amax / 448) rounded up to a power of two;
  * the codes equal an independent cast: torch's float8_e4m3fn conversion of the
    exact quotient x / s (x / s <= 448, so no saturation is involved);
  * blocks built from E4M3 values times 2^k with a +-448 * 2^k element come back
    exactly (s = 2^k, codes unchanged);
  * multiplying a block by 2^j multiplies s by 2^j and keeps every code;
  * a zero block, and a block too small for the range, get s = 2^-127.
"""
import numpy as np
import pytest
import torch

import oracle
import synth


def _is_pow2(s):
    m, _ = np.frexp(s.astype(np.float64))
    return (m == 0.5).all()


@pytest.mark.parametrize("kind", ["act", "weight", "transpose"])
def test_scales_are_the_smallest_power_of_two_above_amax_over_448(kind):
    x = synth.normal((300, 392), 1.0, 7001) * np.float32(3.0)
    if kind == "act":
        q, s = oracle.quant_act(x, rule="pow2")
        amax = np.stack([np.abs(x[:, b * 128:(b + 1) * 128]).max(axis=1) for b in range(4)], axis=1)
        q_amax, s_amax = oracle.quant_act(x)
    elif kind == "weight":
        q, s = oracle.quant_weight(x, rule="pow2")
        amax = np.array([[np.abs(x[i * 128:(i + 1) * 128, j * 128:(j + 1) * 128]).max() for j in range(4)]
                         for i in range(3)])
        q_amax, s_amax = oracle.quant_weight(x)
    else:
        q, s = oracle.quant_transpose(x, True, rule="pow2")
        amax = np.stack([np.abs(x[b * 128:(b + 1) * 128, :]).max(axis=0) for b in range(3)], axis=1)
        q_amax, s_amax = oracle.quant_transpose(x, True)
    assert _is_pow2(s)
    r = amax.astype(np.float64) / s
    assert (r > 224).all() and (r <= 448).all()
    # the recipe's scale rounded up to a power of two (never below it)
    assert (s >= s_amax).all() and (s < 2 * s_amax.astype(np.float64)).all()


def test_codes_equal_torch_cast_of_exact_quotient():
    x = synth.normal((64, 512), 1.0, 7002)
    x[:, 5] *= 1e4
    x[3, 128:256] *= 1e-30
    q, s = oracle.quant_act(x, rule="pow2")
    y = x.astype(np.float64) / np.repeat(s.astype(np.float64), 128, axis=1)
    assert np.abs(y).max() <= 448
    ref = torch.from_numpy(y.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert (q == ref).all()


def test_exact_blocks_round_trip():
    rng = np.random.default_rng(7003)
    finite = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
    codes = rng.choice(finite, size=(32, 256))
    codes[:, 7] = 0x7E
    codes[:, 130] = 0xFE
    k = rng.integers(-40, 40, size=(32, 2))
    x = (oracle.e4m3_decode(codes) * np.repeat(np.ldexp(1.0, k), 128, axis=1)).astype(np.float32)
    q, s = oracle.quant_act(x, rule="pow2")
    assert (s == np.ldexp(1.0, k).astype(np.float32)).all()
    assert (q == codes).all()


@pytest.mark.parametrize("j", [-30, -1, 1, 25])
def test_power_of_two_scaling(j):
    x = synth.normal((16, 256), 1.0, 7004)
    q0, s0 = oracle.quant_act(x, rule="pow2")
    q1, s1 = oracle.quant_act((x * np.float32(2.0 ** j)).astype(np.float32), rule="pow2")
    assert (q0 == q1).all()
    assert (s1.astype(np.float64) == s0.astype(np.float64) * 2.0 ** j).all()


def test_zero_and_tiny_blocks_get_the_smallest_scale():
    x = np.zeros((2, 256), np.float32)
    x[0, 3] = -0.0
    x[1, 128:] = np.float32(1e-40)          # 448 * 2^-127 > 1e-40: at the range limit
    q, s = oracle.quant_act(x, rule="pow2")
    assert (s == np.float32(2.0 ** -127)).all()
    assert q[0, 3] == 0x80 and (q[0, :3] == 0).all()
    # 1e-40 / 2^-127 = 1.7: a normal E4M3 value
    assert (q[1, 128:] == torch.tensor([1e-40 / 2.0 ** -127]).to(torch.float8_e4m3fn).view(torch.uint8).item()).all()
