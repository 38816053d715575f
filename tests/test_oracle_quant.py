"""Pins for the oracle's blockwise quantisers (CPU only).

Reading of the pages (Puro-2B-Base model card, setup paragraph: main linear
GEMMs in blockwise E4M3; technical report part 7/7: DeepSeek-V3-style FP8):
per block s = fl32(amax/448), q = E4M3_RNE_sat(fl32(x/s)), zero blocks give
s = 0 and signed zero codes.  Pinned by properties that this definition fixes:
  (i)   blocks built from E4M3 values times a power-of-two scale, holding a
        +-448*s element, give back exactly that scale and those codes;
  (ii)  every block's amax element encodes to +-448 (0x7E / 0xFE);
  (iii) multiplying a block by 2^k multiplies s by 2^k and keeps every code;
  (iv)  q(-x) = q(x) ^ 0x80 with the same s;
  (v)   codes are monotone in x within a block;
  (vi)  |x/s - value(q)| <= half an E4M3 spacing plus the FP32 division error;
  (vii) zero blocks give s = 0 and codes 0x00 / 0x80 by sign;
plus layout identities between the three quantisers and the ragged-tail rule.
"""
import numpy as np
import pytest

import oracle
import synth

FINITE = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
VALS = oracle.e4m3_decode(FINITE)


def _rng(seed):
    return np.random.default_rng(seed)


def _exact_blocks(rows, cols, seed, block="row"):
    """x = value(code) * 2^k with a +-448 element in every 1x128 row block (block='row'),
    128x128 tile (block='tile') or 128x1 column block (block='col'); returns x, codes, scales."""
    rng = _rng(seed)
    codes = rng.choice(FINITE, size=(rows, cols))
    x = oracle.e4m3_decode(codes)
    if block == "row":
        nb = (cols + 127) // 128
        k = rng.integers(-20, 20, size=(rows, nb))
        for b in range(nb):
            c0 = b * 128
            pos = c0 + rng.integers(0, min(128, cols - c0), size=rows)
            sign = rng.choice([0, 0x80], size=rows)
            codes[np.arange(rows), pos] = 0x7E | sign
        x = oracle.e4m3_decode(codes)
        scale = np.ldexp(1.0, k)
        x = x * np.repeat(scale, 128, axis=1)[:, :cols]
    elif block == "col":
        nb = (rows + 127) // 128
        k = rng.integers(-20, 20, size=(nb, cols))
        for b in range(nb):
            r0 = b * 128
            pos = r0 + rng.integers(0, min(128, rows - r0), size=cols)
            codes[pos, np.arange(cols)] = 0x7E | rng.choice([0, 0x80], size=cols)
        x = oracle.e4m3_decode(codes)
        scale = np.ldexp(1.0, k)
        x = x * np.repeat(scale, 128, axis=0)[:rows, :]
    else:
        rb, cb = (rows + 127) // 128, (cols + 127) // 128
        k = rng.integers(-20, 20, size=(rb, cb))
        for i in range(rb):
            for j in range(cb):
                r = i * 128 + rng.integers(0, min(128, rows - i * 128))
                c = j * 128 + rng.integers(0, min(128, cols - j * 128))
                codes[r, c] = 0x7E | rng.choice([0, 0x80])
        x = oracle.e4m3_decode(codes)
        scale = np.ldexp(1.0, k)
        x = x * np.repeat(np.repeat(scale, 128, axis=0), 128, axis=1)[:rows, :cols]
    return x.astype(np.float32), codes, scale.astype(np.float32)


@pytest.mark.parametrize("rows,cols", [(64, 512), (33, 200)])
def test_i_exact_blocks_round_trip_act(rows, cols):
    x, codes, scale = _exact_blocks(rows, cols, 10)
    q, s = oracle.quant_act(x)
    np.testing.assert_array_equal(s, scale)
    np.testing.assert_array_equal(q, codes)


@pytest.mark.parametrize("rows,cols", [(256, 384), (200, 130)])
def test_i_exact_blocks_round_trip_weight(rows, cols):
    x, codes, scale = _exact_blocks(rows, cols, 11, block="tile")
    q, s = oracle.quant_weight(x)
    np.testing.assert_array_equal(s, scale)
    np.testing.assert_array_equal(q, codes)


@pytest.mark.parametrize("tokens,cols", [(384, 48), (300, 20)])
def test_i_exact_blocks_round_trip_transpose(tokens, cols):
    x, codes, scale = _exact_blocks(tokens, cols, 12, block="col")
    q, s = oracle.quant_transpose(x, transpose_out=False)
    np.testing.assert_array_equal(s, scale)
    np.testing.assert_array_equal(q, codes)
    qt, st = oracle.quant_transpose(x, transpose_out=True)
    np.testing.assert_array_equal(st, scale.T)
    np.testing.assert_array_equal(qt, codes.T)


def _random_act(rows, cols, seed, spread=True):
    x = synth.normal((rows, cols), 1.0, seed)
    if spread:  # per-row magnitudes over many binades
        x *= np.float32(2.0) ** _rng(seed).integers(-60, 60, size=(rows, 1)).astype(np.float32)
    return x


def test_ii_amax_maps_to_448():
    x = _random_act(300, 1024, 20)
    q, s = oracle.quant_act(x)
    blocks = np.abs(x).reshape(300, 8, 128)
    amax = blocks.max(axis=2, keepdims=True)
    at_max = blocks == amax
    qb = q.reshape(300, 8, 128)
    assert ((qb & 0x7F)[at_max] == 0x7E).all()
    assert ((qb & 0x7F)[~at_max] <= 0x7E).all()


@pytest.mark.parametrize("k", [-7, -1, 1, 5, 30])
def test_iii_power_of_two_scaling(k):
    x = _random_act(64, 512, 21)
    q0, s0 = oracle.quant_act(x)
    q1, s1 = oracle.quant_act((x * np.float32(2.0 ** k)).astype(np.float32))
    np.testing.assert_array_equal(q1, q0)
    np.testing.assert_array_equal(s1, (s0 * np.float32(2.0 ** k)).astype(np.float32))
    w = synth.normal((256, 256), 0.02, 22)
    qw0, sw0 = oracle.quant_weight(w)
    qw1, sw1 = oracle.quant_weight((w * np.float32(2.0 ** k)).astype(np.float32))
    np.testing.assert_array_equal(qw1, qw0)
    np.testing.assert_array_equal(sw1, (sw0 * np.float32(2.0 ** k)).astype(np.float32))


def test_iv_sign_symmetry():
    x = _random_act(64, 512, 23)
    q0, s0 = oracle.quant_act(x)
    q1, s1 = oracle.quant_act(-x)
    np.testing.assert_array_equal(s0, s1)
    np.testing.assert_array_equal(q1, q0 ^ 0x80)


def test_v_monotone_within_block():
    x = _random_act(32, 128, 24)
    q, s = oracle.quant_act(x)
    for r in range(32):
        order = np.argsort(x[r], kind="stable")
        v = oracle.e4m3_decode(q[r][order])
        assert (np.diff(v) >= 0).all()


def test_vi_error_bound():
    x = _random_act(256, 1024, 25)
    q, s = oracle.quant_act(x)
    y = x.astype(np.float64) / np.repeat(s.astype(np.float64), 128, axis=1)
    v = oracle.e4m3_decode(q)
    half_spacing = np.where(np.abs(v) >= 2.0 ** -6, 2.0 ** -4 * np.abs(v), 2.0 ** -10)
    # |y| here is x/s in exact arithmetic; fl32 adds at most 2^-24 |y|
    assert (np.abs(y - v) <= half_spacing + 2.0 ** -24 * np.abs(y)).all()


def test_vii_zero_blocks():
    x = _random_act(8, 512, 26)
    x[3, 128:256] = 0.0
    x[5, 0:128] = -0.0
    x[6, 384:512] = np.where(np.arange(128) % 2 == 0, 0.0, -0.0).astype(np.float32)
    q, s = oracle.quant_act(x)
    assert s[3, 1] == 0 and s[5, 0] == 0 and s[6, 3] == 0
    assert (q[3, 128:256] == 0x00).all()
    assert (q[5, 0:128] == 0x80).all()
    assert (q[6, 384:512] == np.where(np.arange(128) % 2 == 0, 0x00, 0x80)).all()
    assert (s[~np.isin(np.arange(8), [3, 5, 6])] > 0).all()


def test_vii_underflowing_scale_is_a_zero_block():
    # amax / 448 underflows to 0 in FP32: treated as a zero block
    x = np.zeros((1, 128), np.float32)
    x[0, 5] = np.float32(1e-45)
    x[0, 6] = np.float32(-1e-45)
    q, s = oracle.quant_act(x)
    assert s[0, 0] == 0
    assert q[0, 5] == 0x00 and q[0, 6] == 0x80


def test_subnormal_scales_and_inputs():
    # amax small enough that s is an FP32 subnormal; the definition still applies
    x = synth.normal((4, 256), 1.0, 27) * np.float32(1e-37)
    q, s = oracle.quant_act(x.astype(np.float32))
    assert (s > 0).all() and (s < np.finfo(np.float32).tiny).all()
    yy = x.astype(np.float32) / np.repeat(s, 128, axis=1)
    np.testing.assert_array_equal(q, oracle.e4m3_encode(yy.astype(np.float32)))


def test_ragged_tail_block_uses_only_its_elements():
    x = _random_act(16, 200, 28)
    q, s = oracle.quant_act(x)
    q_tail, s_tail = oracle.quant_act(np.ascontiguousarray(x[:, 128:]))
    np.testing.assert_array_equal(q[:, 128:], q_tail)
    np.testing.assert_array_equal(s[:, 1:], s_tail)
    w = synth.normal((130, 260), 0.02, 29)
    qw, sw = oracle.quant_weight(w)
    qe, se = oracle.quant_weight(np.ascontiguousarray(w[128:, 256:]))
    np.testing.assert_array_equal(qw[128:, 256:], qe)
    assert sw[1, 2] == se[0, 0]


def test_layout_identities_between_quantisers():
    x = synth.normal((384, 96), 1.0, 30, dtype="bf16")
    qt, st = oracle.quant_transpose(x, transpose_out=True)
    qn, sn = oracle.quant_transpose(x, transpose_out=False)
    qa, sa = oracle.quant_act(np.ascontiguousarray(x.T))
    np.testing.assert_array_equal(qt, qa)
    np.testing.assert_array_equal(st, sa)
    np.testing.assert_array_equal(qn, qa.T)
    np.testing.assert_array_equal(sn, sa.T)


def test_bf16_input_equals_widened_fp32_input():
    xb = synth.normal((64, 384), 1.0, 31, dtype="bf16")
    xf = synth.bf16_bits_to_f32(xb)
    for fn in (oracle.quant_act, oracle.quant_weight):
        qb, sb = fn(xb)
        qf, sf = fn(xf)
        np.testing.assert_array_equal(qb, qf)
        np.testing.assert_array_equal(sb, sf)
    wb = synth.normal((256, 128), 0.02, 32, dtype="bf16")
    np.testing.assert_array_equal(oracle.quant_weight(wb)[0], oracle.quant_weight(synth.bf16_bits_to_f32(wb))[0])


def test_empty_inputs():
    q, s = oracle.quant_act(np.zeros((0, 256), np.float32))
    assert q.shape == (0, 256) and s.shape == (0, 2)
    q, s = oracle.quant_act(np.zeros((5, 0), np.float32))
    assert q.shape == (5, 0) and s.shape == (5, 0)
    q, s = oracle.quant_transpose(np.zeros((0, 7), np.float32))
    assert q.shape == (7, 0) and s.shape == (7, 0)
