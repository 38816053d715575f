"""GPU parity of the three quantisers against the oracle: codes and scales bit-exact.

Inputs: the workload shapes (config-1 FP32 X / W; Qwen3-1.7B layer tensors at
reduced token counts), ragged extents with padded rows, and adversarial
blocks (exact E4M3 midpoints, +-0, zero blocks, outlier channels, FP32
subnormal scales, lognormal gradients).
"""
import numpy as np
import pytest
import torch

import blockwise_fp8_gemm_amd as pf
import oracle
import synth
from helpers import first_mismatch, host, to_dev

pytestmark = pytest.mark.gpu


def _assert_same(q_gpu, s_gpu, q_ref, s_ref, what):
    qg, sg = host(q_gpu), host(s_gpu)
    assert qg.shape == q_ref.shape and sg.shape == s_ref.shape, what
    assert first_mismatch(sg.view(np.uint32), s_ref.view(np.uint32)) is None, (
        what, "scale", first_mismatch(sg.view(np.uint32), s_ref.view(np.uint32)))
    assert first_mismatch(qg, q_ref) is None, (what, "codes", first_mismatch(qg, q_ref))


def _adversarial(rows, cols, seed):
    """FP32 rows mixing the hard cases of the codec and of the scale rule."""
    rng = np.random.default_rng(seed)
    x = synth.normal((rows, cols), 1.0, seed)
    nb = cols // 128
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
    vals = oracle.e4m3_decode(codes)
    pos = np.sort(np.unique(np.abs(vals)))
    mids = (pos[:-1] + pos[1:]) / 2                    # exact E4M3 midpoints
    for r in range(rows):
        b = rng.integers(0, nb)
        kind = r % 8
        seg = slice(b * 128, b * 128 + 128)
        if kind == 0:     # amax exactly 448: s = 1, every midpoint is a tie
            m = rng.choice(mids, 128) * rng.choice([-1, 1], 128)
            m[rng.integers(0, 128)] = 448.0
            x[r, seg] = m.astype(np.float32)
        elif kind == 1:   # zero block with mixed signed zeros
            x[r, seg] = np.where(rng.random(128) < 0.5, 0.0, -0.0).astype(np.float32)
        elif kind == 2:   # tiny block: FP32 subnormal scale
            x[r, seg] *= np.float32(1e-38)
        elif kind == 3:   # huge dynamic range inside one block
            x[r, seg] *= (np.float32(2.0) ** rng.integers(-40, 10, 128)).astype(np.float32)
        elif kind == 4:   # scaled midpoints: power-of-two scale, ties after division
            k = rng.integers(-30, 30)
            m = rng.choice(mids, 128) * rng.choice([-1, 1], 128)
            m[0] = -448.0
            x[r, seg] = (m * 2.0 ** k).astype(np.float32)
        elif kind == 5:   # one outlier channel
            x[r, b * 128 + rng.integers(0, 128)] *= np.float32(1e4)
        elif kind == 6:   # -0.0 and values that round to zero
            x[r, seg] = (rng.standard_normal(128) * 1e-9).astype(np.float32)
            x[r, b * 128] = 1.0
            x[r, b * 128 + 1] = -0.0
        else:             # scales either side of 2^-80 (where the kernels stop using the reciprocal)
            x[r, seg] *= np.float32(2.0) ** rng.integers(-76, -62)
            x[r, seg][rng.integers(0, 128, 8)] *= np.float32(2.0 ** -20)
    return x


ACT_CASES = [
    ("config1_x_f32", lambda: synth.normal((256, 512), 1.0, synth.seed_of(1, 0, 0)), None),
    ("layer_x_bf16", lambda: synth.normal((1024, 2048), 1.0, synth.seed_of(2, 0, 0), "bf16"), None),
    ("down_in_bf16", lambda: synth.normal((512, 6144), 1.0, synth.seed_of(2, 0, 6), "bf16"), None),
    ("dy_bf16", lambda: synth.normal((512, 4096), 1e-3, synth.seed_of(3, 0, 8), "bf16"), None),
    ("adversarial_f32", lambda: _adversarial(256, 1024, 77), None),
    ("adversarial_bf16", lambda: synth.f32_to_bf16_bits(_adversarial(256, 1024, 78)), None),
    ("ragged_f32", lambda: synth.normal((77, 300), 1.0, 79), 304),
    ("ragged_bf16", lambda: synth.normal((130, 1000), 1.0, 80, "bf16"), 1024),
    ("single_short_row", lambda: synth.normal((1, 5), 1.0, 81), None),
]


@pytest.mark.parametrize("name,make,ld", ACT_CASES, ids=[c[0] for c in ACT_CASES])
def test_quant_act_bit_exact(dev, name, make, ld):
    x = make()
    q_ref, s_ref = oracle.quant_act(x)
    q, s = pf.puro_fp8_quant_act(to_dev(x, ld=ld))
    torch.cuda.synchronize()
    _assert_same(q, s, q_ref, s_ref, name)


WEIGHT_CASES = [
    ("config1_w_f32", lambda: synth.normal((256, 512), 1.0, synth.seed_of(1, 0, 1)), None),
    ("qkv_w_f32", lambda: synth.normal((4096, 2048), 0.02, synth.seed_of(2, 0, 1)), None),
    ("down_w_f32", lambda: synth.normal((2048, 6144), 0.02, synth.seed_of(2, 0, 7)), None),
    ("w_bf16", lambda: synth.normal((512, 1024), 0.02, 90, "bf16"), None),
    ("adversarial_f32", lambda: _adversarial(256, 512, 91), None),
    ("ragged_f32", lambda: synth.normal((200, 333), 0.02, 92), 336),
    ("ragged_bf16", lambda: synth.normal((129, 130), 0.02, 93, "bf16"), 144),
]


@pytest.mark.parametrize("name,make,ld", WEIGHT_CASES, ids=[c[0] for c in WEIGHT_CASES])
def test_quant_weight_bit_exact(dev, name, make, ld):
    w = make()
    q_ref, s_ref = oracle.quant_weight(w)
    q, s = pf.puro_fp8_quant_weight(to_dev(w, ld=ld))
    torch.cuda.synchronize()
    _assert_same(q, s, q_ref, s_ref, name)


@pytest.mark.parametrize("transposed", [False, True], ids=["plain", "transposed"])
@pytest.mark.parametrize("rule", ["amax", "pow2"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_quant_weight_grouped_bit_exact(dev, dtype, rule, transposed):
    """Several weights in grouped launches: each equal to the oracle's weight quantiser,
    and with transposed, its transposed copy equal to the oracle's codes and scales
    transposed (padded rows of the copy untouched).

    21 weights (two launches of at most 16): a layer's seven projections at
    reduced size, ragged extents with padded rows, an adversarial weight and
    empty ones in between.
    """
    def f(x):
        return synth.f32_to_bf16_bits(x) if dtype == "bf16" else x
    shapes = [(512, 256), (256, 256), (256, 256), (256, 256), (768, 256), (768, 256), (256, 768),
              (200, 333), (129, 130), (1, 16), (128, 128), (0, 256), (384, 640), (256, 0)]
    ws, lds = [], []
    for i, (r, c) in enumerate(shapes):
        ws.append(f(synth.normal((r, c), 0.02, 5200 + i)))
        lds.append((c + 15) // 16 * 16 + (16 if i % 3 == 0 else 0))
    ws.append(f(_adversarial(256, 512, 5250)))
    lds.append(512)
    for i in range(6):
        ws.append(f(synth.normal((128 * (i + 1), 128), 1.0 + i, 5260 + i)))
        lds.append(128)
    devs = [to_dev(w, ld=ld) for w, ld in zip(ws, lds)]
    given, bufs = None, []
    if transposed:   # transposed copies in buffers with 16 spare codes per row, marked 0x5A
        given = []
        for w in ws:
            r, c = w.shape
            buf = torch.full((c, (r + 15) // 16 * 16 + 16), 0x5A, dtype=torch.uint8, device="cuda:0")
            bufs.append((buf, r))
            given.append((None, None, buf[:, :r], None))
    outs = pf.puro_fp8_quant_weight_grouped(devs, outs=given, pow2=(rule == "pow2"), transposed=transposed)
    torch.cuda.synchronize()
    assert len(outs) == len(ws) == 21
    for i, (w, o) in enumerate(zip(ws, outs)):
        q_ref, s_ref = oracle.quant_weight(w, rule=rule)
        _assert_same(o[0], o[1], q_ref, s_ref, "grouped weight %d %s" % (i, w.shape))
        if transposed:
            _assert_same(o[2], o[3], np.ascontiguousarray(q_ref.T), np.ascontiguousarray(s_ref.T),
                         "grouped weight %d %s transposed" % (i, w.shape))
            buf, r = bufs[i]
            assert (buf[:, r:] == 0x5A).all(), "transposed copy %d wrote past its rows" % i


TRANSPOSE_CASES = [
    ("layer_x_bf16", lambda: synth.normal((1024, 2048), 1.0, synth.seed_of(3, 0, 0), "bf16"), None),
    ("dy_bf16", lambda: synth.normal((1024, 1024), 1e-3, synth.seed_of(3, 0, 9), "bf16"), None),
    ("outlier_bf16", lambda: synth.outlier_activations(512, 768, 95)[0], None),
    ("lognormal_bf16", lambda: synth.lognormal_gradients(512, 256, 96, random_sign=True), None),
    ("adversarial_f32", lambda: np.ascontiguousarray(_adversarial(256, 512, 97).T), None),
    ("ragged_bf16", lambda: synth.normal((300, 100), 1.0, 98, "bf16"), 112),
    ("ragged_f32", lambda: synth.normal((129, 65), 1.0, 99), 80),
]


@pytest.mark.parametrize("transpose_out", [True, False])
@pytest.mark.parametrize("name,make,ld", TRANSPOSE_CASES, ids=[c[0] for c in TRANSPOSE_CASES])
def test_quant_transpose_bit_exact(dev, name, make, ld, transpose_out):
    x = make()
    q_ref, s_ref = oracle.quant_transpose(x, transpose_out=transpose_out)
    q, s = pf.puro_fp8_quant_transpose(to_dev(x, ld=ld), transpose_out)
    torch.cuda.synchronize()
    _assert_same(q, s, q_ref, s_ref, name)


def test_quantisers_deterministic(dev):
    x = to_dev(synth.normal((512, 2048), 1.0, 100, "bf16"))
    a = [pf.puro_fp8_quant_act(x) for _ in range(2)]
    b = [pf.puro_fp8_quant_transpose(x, True) for _ in range(2)]
    torch.cuda.synchronize()
    for (q0, s0), (q1, s1) in (a, b):
        assert torch.equal(q0, q1) and torch.equal(s0.view(torch.int32), s1.view(torch.int32))


def test_padding_is_untouched(dev):
    """Bytes beyond the row length of a padded output stay as they were."""
    x = synth.normal((64, 200), 1.0, 101)
    buf = torch.full((64, 208), 0x5A, dtype=torch.uint8, device=dev)
    q = buf[:, :200]
    pf.puro_fp8_quant_act(to_dev(x, ld=208), q=q)
    torch.cuda.synchronize()
    assert (buf[:, 200:] == 0x5A).all()


DUAL_CASES = [
    ("layer_x_bf16", lambda: synth.normal((1024, 2048), 1.0, synth.seed_of(3, 0, 1), "bf16"), None),
    ("dy_bf16", lambda: synth.normal((512, 6144), 1e-3, synth.seed_of(3, 0, 10), "bf16"), None),
    ("outlier_bf16", lambda: synth.outlier_activations(512, 768, 195)[0], None),
    ("lognormal_bf16", lambda: synth.lognormal_gradients(384, 256, 196, random_sign=True), None),
    ("adversarial_f32", lambda: _adversarial(256, 512, 197), None),
    ("adversarial_bf16", lambda: synth.f32_to_bf16_bits(_adversarial(256, 1024, 198)), None),
    ("ragged_bf16", lambda: synth.normal((300, 200), 1.0, 199, "bf16"), 208),
    ("ragged_f32", lambda: synth.normal((129, 65), 1.0, 200), 80),
]


@pytest.mark.parametrize("transpose_out", [True, False])
@pytest.mark.parametrize("name,make,ld", DUAL_CASES, ids=[c[0] for c in DUAL_CASES])
def test_quant_dual_bit_exact(dev, name, make, ld, transpose_out):
    """One read, two outputs: equal to the oracle's row quantiser and token quantiser."""
    x = make()
    qr_ref, sr_ref = oracle.quant_act(x)
    qt_ref, st_ref = oracle.quant_transpose(x, transpose_out=transpose_out)
    qr, sr, qt, st = pf.puro_fp8_quant_dual(to_dev(x, ld=ld), transpose_out)
    torch.cuda.synchronize()
    _assert_same(qr, sr, qr_ref, sr_ref, name + " rows")
    _assert_same(qt, st, qt_ref, st_ref, name + " tokens")
