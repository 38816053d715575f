"""Pins for the oracle's gated activation h = silu(g) * u (CPU only).

The model card's configuration table names the Qwen3-1.7B configuration, whose
feed-forward block gates the up projection with SiLU of the gate projection
(SwiGLU with Swish parameter 1).  The oracle evaluates g * u / (1 + e^-g) in
FP64.  It is pinned against
  * closed forms: sigmoid(ln 3) = 3/4 and sigmoid(ln 7) = 7/8, so h is a known
    multiple of ln 3 or ln 7; silu(0) = 0; the asymptotes silu(g) -> g and
    silu(-g) -> -g e^-g;
  * the identity sigmoid(g) + sigmoid(-g) = 1, i.e. h(g) - h(-g) = g u;
  * the minimum of silu, -W(1/e) at g = -1 - W(1/e) (W = Lambert's W, from
    scipy), a fact of the mathematics the formula must reproduce;
  * two independent library routines: numpy's tanh through
    sigmoid(g) = (1 + tanh(g/2)) / 2, and torch's FP64 SiLU.
"""
import math

import numpy as np
import pytest
import scipy.special
import torch

import oracle


def test_closed_forms():
    ln3, ln7 = math.log(3.0), math.log(7.0)
    g = np.array([ln3, -ln3, ln7, -ln7])
    u = np.array([2.0, -3.0, 0.5, 4.0])
    want = np.array([0.75 * ln3 * 2.0, -0.25 * ln3 * -3.0, 0.875 * ln7 * 0.5, -0.125 * ln7 * 4.0])
    np.testing.assert_allclose(oracle.swiglu(g, u), want, rtol=4e-16, atol=0)


def test_zero_and_asymptotes():
    assert oracle.swiglu(np.array([0.0]), np.array([5.0]))[0] == 0.0
    assert oracle.swiglu(np.array([3.0]), np.array([0.0]))[0] == 0.0
    # 1 + e^-50 rounds to 1 in FP64: h is g u exactly
    assert oracle.swiglu(np.array([50.0]), np.array([-1.5]))[0] == -75.0
    # far negative: h = g u e^g (1 - e^g + ...) with e^g below 2^-53
    g = np.array([-40.0, -50.0, -300.0])
    u = np.array([1.0, 2.0, -3.0])
    np.testing.assert_allclose(oracle.swiglu(g, u), g * u * np.exp(g), rtol=4e-16, atol=0)
    # beyond e^709 the denominator is infinite: a zero with the sign of g u
    h = oracle.swiglu(np.array([-800.0, -800.0]), np.array([1.0, -1.0]))
    assert h[0] == 0.0 and math.copysign(1.0, h[0]) < 0
    assert h[1] == 0.0 and math.copysign(1.0, h[1]) > 0


def test_odd_part_identity():
    rng = np.random.default_rng(7)
    g = rng.standard_normal(20000) * 6.0
    u = rng.standard_normal(20000)
    diff = oracle.swiglu(g, u) - oracle.swiglu(-g, u)
    np.testing.assert_allclose(diff, g * u, rtol=1e-14, atol=1e-300)


def test_minimum_is_minus_lambert_w_of_inverse_e():
    w = float(np.real(scipy.special.lambertw(1.0 / math.e)))
    g_star = -1.0 - w
    h_star = oracle.swiglu(np.array([g_star]), np.array([1.0]))[0]
    assert abs(h_star + w) <= 4e-16
    side = oracle.swiglu(np.array([g_star - 1e-3, g_star + 1e-3]), np.array([1.0, 1.0]))
    assert (side > h_star).all()


def test_tanh_form():
    rng = np.random.default_rng(11)
    g = np.concatenate([rng.standard_normal(50000) * 8.0, np.linspace(-30, 30, 6001)])
    u = rng.standard_normal(g.size) * 10.0 ** rng.integers(-3, 4, g.size)
    alt = g * u * 0.5 * (1.0 + np.tanh(0.5 * g))
    # 1 + tanh(g/2) loses relative precision for negative g: compare against |g u|
    assert (np.abs(oracle.swiglu(g, u) - alt) <= 1e-15 * np.abs(g * u) + 1e-300).all()


def test_torch_silu_fp64():
    rng = np.random.default_rng(13)
    g = rng.standard_normal(100000) * 5.0
    u = rng.standard_normal(100000)
    ref = (torch.nn.functional.silu(torch.from_numpy(g)) * torch.from_numpy(u)).numpy()
    np.testing.assert_allclose(oracle.swiglu(g, u), ref, rtol=1e-14, atol=1e-300)


def test_bf16_inputs_and_rounding():
    # BF16 bit patterns are read as their exact values; the BF16 result is one rounding
    g = np.array([0x3F80, 0xBF80, 0x4040, 0x0000], np.uint16)     # 1, -1, 3, 0
    u = np.array([0x4000, 0x4000, 0xBF00, 0x3F80], np.uint16)     # 2, 2, -0.5, 1
    gv, uv = np.array([1.0, -1.0, 3.0, 0.0]), np.array([2.0, 2.0, -0.5, 1.0])
    np.testing.assert_array_equal(oracle.swiglu(g, u), oracle.swiglu(gv, uv))
    np.testing.assert_array_equal(oracle.swiglu_bf16(g, u), oracle.bf16_rne(oracle.swiglu(gv, uv)))
    with pytest.raises(ValueError):
        oracle.swiglu(np.zeros(3), np.zeros(4))
