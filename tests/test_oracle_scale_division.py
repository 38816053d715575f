"""Independent pin of the oracle's block scale and quotient (CPU only).

The scale rule read from the Puro-2B-Base model card's setup paragraph
("blockwise E4M3" for the main linear-layer GEMMs) is s = fl32(amax / 448) and
q = E4M3_RNE_sat(fl32(x / s)): two IEEE binary32 divisions.  A reciprocal
multiply (amax * RN(1/448), x * RN(1/s)) is a plausible slip that the
invariant pins in test_oracle_quant.py do not see: it agrees with division on
every block whose amax is 448 * 2^k and keeps the amax element at 0x7E.

Here the oracle's scales and codes are compared, on 10^5 blocks whose amax is
not 448 * 2^k, spread over binades 2^-140 .. 2^120 (FP32-subnormal scales
included), with a computation that shares nothing with it:
  * s: numpy's float32 division np.float32(amax) / np.float32(448), which is
    IEEE binary32 division (round to nearest even, subnormals kept);
  * q: numpy's float32 quotient np.float32(x) / s, saturated at +-448 and cast
    by torch's float8_e4m3fn conversion (round to nearest even).
Half of each block's elements are placed within a few FP32 ulps of an E4M3
rounding midpoint, so that a quotient off by one ulp changes the code.  The
tests also check that the data separates the two forms: the reciprocal forms
give different scales, and different codes, on many blocks.
"""
import numpy as np
import pytest
import torch

import oracle

FINITE_POS = np.arange(0x7F, dtype=np.uint8)             # codes 0x00 .. 0x7E
POS_VALS = oracle.e4m3_decode(FINITE_POS)
MIDPOINTS = 0.5 * (POS_VALS[:-1] + POS_VALS[1:])         # between adjacent codes, all < 448


def _adversarial_blocks(nblocks, seed, lo_exp=-140, hi_exp=120, n=128):
    """nblocks rows of n float32 values.  Row b: one element +-amax_b (amax_b
    with a random non-trivial mantissa, exponent uniform in [lo_exp, hi_exp]),
    n/2 - 1 elements near E4M3 midpoints times fl32(amax_b/448), n/2 elements
    uniform in (-amax_b, amax_b)."""
    rng = np.random.default_rng(seed)
    h = n // 2
    mant = rng.uniform(1.0, 2.0, size=nblocks)
    mant[mant == 1.0] = 1.5
    amax = np.ldexp(mant, rng.integers(lo_exp, hi_exp, size=nblocks)).astype(np.float32)
    # keep amax a normal or subnormal nonzero float32, not a power-of-two multiple of 448
    amax = np.where(amax == 0, np.float32(1e-40), amax).astype(np.float32)
    s = amax / np.float32(448.0)
    x = np.empty((nblocks, n), np.float32)
    x[:, :h] = (rng.uniform(-1.0, 1.0, size=(nblocks, h)) * amax[:, None]).astype(np.float32)
    mid = MIDPOINTS[rng.integers(0, MIDPOINTS.size, size=(nblocks, h - 1))]
    near = (mid * s[:, None].astype(np.float64)).astype(np.float32)
    # move by -2 .. +2 ulps so that x / s lands on both sides of the midpoint
    steps = rng.integers(-2, 3, size=(nblocks, h - 1))
    for k in (1, 2):
        near = np.where(steps >= k, np.nextafter(near, np.float32(np.inf)), near)
        near = np.where(steps <= -k, np.nextafter(near, np.float32(-np.inf)), near)
    near = np.minimum(np.abs(near), amax[:, None]).astype(np.float32)
    sign = rng.choice(np.array([-1.0, 1.0], np.float32), size=(nblocks, h - 1))
    x[:, h:n - 1] = near * sign
    x[:, n - 1] = amax * rng.choice(np.array([-1.0, 1.0], np.float32), size=nblocks)
    # shuffle positions inside each block
    perm = np.argsort(rng.random((nblocks, n)), axis=1)
    return np.take_along_axis(x, perm, axis=1)


def _torch_e4m3(y):
    """torch's E4M3 cast of float32 values, saturated at +-448 first."""
    t = torch.from_numpy(np.ascontiguousarray(y, np.float32)).clamp(-448.0, 448.0)
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def _independent(xb):
    """(s, codes) of every 128-element row of xb by numpy division and torch's cast."""
    amax = np.abs(xb).max(axis=1)
    s = (amax.astype(np.float32) / np.float32(448.0)).astype(np.float32)
    with np.errstate(divide="ignore", invalid="ignore"):
        y = (xb / s[:, None]).astype(np.float32)
    codes = np.where(s[:, None] > 0, _torch_e4m3(np.where(s[:, None] > 0, y, 0.0)),
                     np.where(np.signbit(xb), 0x80, 0x00)).astype(np.uint8)
    return s, codes


@pytest.fixture(scope="module")
def blocks():
    return _adversarial_blocks(100_000, 4242)


def test_scale_bits_equal_ieee_division(blocks):
    q, s = oracle.quant_act(blocks)
    s_ind, _ = _independent(blocks)
    assert s.shape == (blocks.shape[0], 1)
    np.testing.assert_array_equal(s[:, 0].view(np.uint32), s_ind.view(np.uint32))
    # the data has FP32-subnormal scales and spans the binades
    assert ((s > 0) & (s < np.finfo(np.float32).tiny)).sum() > 1000
    assert s.max() > 2.0 ** 100 and s[s > 0].min() < 2.0 ** -140


def test_codes_equal_ieee_quotient_cast_by_torch(blocks):
    q, s = oracle.quant_act(blocks)
    _, codes_ind = _independent(blocks)
    bad = np.argwhere(q != codes_ind)
    assert bad.size == 0, "first mismatch at %s" % (tuple(bad[0]),)


def test_data_separates_division_from_reciprocal(blocks):
    """The reciprocal forms a plausible implementation might use give other
    scales and other codes on this data, so the two tests above would fail."""
    amax = np.abs(blocks).max(axis=1)
    s_div = amax / np.float32(448.0)
    s_rcp = amax * (np.float32(1.0) / np.float32(448.0))
    assert (s_div != s_rcp).sum() > 10_000
    y_div = blocks / s_div[:, None]
    with np.errstate(over="ignore", invalid="ignore"):
        r = (np.float32(1.0) / s_div).astype(np.float32)
        y_rcp = (blocks * r[:, None]).astype(np.float32)
    ok = np.isfinite(r)
    changed = _torch_e4m3(y_div[ok]) != _torch_e4m3(np.where(np.isfinite(y_rcp[ok]), y_rcp[ok], 448.0))
    assert changed.sum() > 1000


def test_weight_tiles_and_token_blocks_follow_the_same_rule():
    """The 128x128 and 128-token quantisers use the same block rule."""
    # 128x128 tiles: 48 blocks of 16,384 elements, each laid out as one tile
    tiles = _adversarial_blocks(48, 78, lo_exp=-135, hi_exp=100, n=128 * 128).reshape(48, 128, 128)
    amax = np.abs(tiles).reshape(48, -1).max(axis=1)
    w = tiles.transpose(1, 0, 2).reshape(128, 48 * 128)   # 1 x 48 tiles side by side
    qw, sw = oracle.quant_weight(np.ascontiguousarray(w))
    s_ind = (amax / np.float32(448.0)).astype(np.float32)
    np.testing.assert_array_equal(sw[0].view(np.uint32), s_ind.view(np.uint32))
    with np.errstate(divide="ignore", invalid="ignore"):
        y = (w.reshape(128, 48, 128) / s_ind[None, :, None]).astype(np.float32)
    want = _torch_e4m3(y).reshape(128, 48 * 128)
    np.testing.assert_array_equal(qw, want)
    # 128-token blocks, transposed output: columns of a [tokens][channels] tensor
    x = _adversarial_blocks(3000, 79).T.copy()            # [128 tokens][3000 channels]
    qt, st = oracle.quant_transpose(x, transpose_out=True)
    s_c, codes_c = _independent(np.ascontiguousarray(x.T))
    np.testing.assert_array_equal(st[:, 0].view(np.uint32), s_c.view(np.uint32))
    np.testing.assert_array_equal(qt, codes_c)
