"""GPU parity of puro_fp8_gemm against the oracle.

The oracle takes the E4M3 codes and scales produced by the oracle quantisers
from the same seeded inputs; the GPU takes the codes and scales from the GPU
quantisers (bit-identical, checked first).  Tolerances:
  * FP32 output: relative Frobenius error <= 2e-6 against the FP64 oracle, and
    per element |C - C_ref| <= E = (KB + 4) 2^-23 C_abs, the FP32 accumulation
    bound for KB block promotions, where C_abs is the same blockwise product
    of |a|, |b| (so E bounds rounding in the sum of absolute terms);
  * BF16 output: per element |C - C_ref| <= E + 2^-8 (|C_ref| + E) (the FP32
    bound plus one BF16 rounding), and at least 99% of elements equal to the
    oracle's FP64 result rounded to BF16.
"""
import numpy as np
import pytest
import torch

import blockwise_fp8_gemm_amd as pf
import oracle
import synth
from helpers import bf16_to_f64, first_mismatch, host, rel_frobenius, to_dev

pytestmark = pytest.mark.gpu

FROB_TOL = 2e-6


def _quantise_both(layout, bgran, X, W, ldx=None, ldw=None):
    """Quantise logical X [M][K] and W [N][K] into the storage form of `layout`, on the
    host (oracle) and on the device (library).  Returns (host operands, device operands)."""
    if layout == "NT":
        qa, sa = oracle.quant_act(X)
        dqa, dsa = pf.puro_fp8_quant_act(to_dev(X, ld=ldx))
        if bgran == "128x128":
            qb, sb = oracle.quant_weight(W)
            dqb, dsb = pf.puro_fp8_quant_weight(to_dev(W, ld=ldw))
        else:
            qb, sb = oracle.quant_act(W)
            dqb, dsb = pf.puro_fp8_quant_act(to_dev(W, ld=ldw))
    else:
        Wkn = np.ascontiguousarray(W.T)
        if layout == "NN":
            qa, sa = oracle.quant_act(X)
            dqa, dsa = pf.puro_fp8_quant_act(to_dev(X, ld=ldx))
        else:
            Xkm = np.ascontiguousarray(X.T)
            qa, sa = oracle.quant_transpose(Xkm, transpose_out=False)
            dqa, dsa = pf.puro_fp8_quant_transpose(to_dev(Xkm, ld=_pad(Xkm.shape[1])), False)
        if bgran == "128x128":
            qb, sb = oracle.quant_weight(Wkn)
            dqb, dsb = pf.puro_fp8_quant_weight(to_dev(Wkn, ld=_pad(Wkn.shape[1])))
        else:
            qb, sb = oracle.quant_transpose(Wkn, transpose_out=False)
            dqb, dsb = pf.puro_fp8_quant_transpose(to_dev(Wkn, ld=_pad(Wkn.shape[1])), False)
    torch.cuda.synchronize()
    for a, b in ((dqa, qa), (dsa, sa), (dqb, qb), (dsb, sb)):
        assert first_mismatch(host(a), b) is None
    return (qa, sa, qb, sb), (dqa, dsa, dqb, dsb)


def _pad(n):
    return (n + 15) // 16 * 16


def _elem_bound(layout, bgran, qa, sa, qb, sb, K):
    """Per-element FP32 accumulation bound (KB + 4) 2^-23 sum|terms| from the oracle on |codes|."""
    c_abs = oracle.gemm(layout, qa & 0x7F, np.abs(sa), qb & 0x7F, np.abs(sb), bgran)
    return ((K + 127) // 128 + 4) * 2.0 ** -23 * c_abs


def _check_product(layout, bgran, hostops, devops, out, C=None):
    """Compare C (computed here by puro_fp8_gemm unless given) with the oracle."""
    qa, sa, qb, sb = hostops
    C_ref = oracle.gemm(layout, qa, sa, qb, sb, bgran)
    K = qa.shape[0] if layout == "TN" else qa.shape[1]
    E = _elem_bound(layout, bgran, qa, sa, qb, sb, K)
    if C is None:
        C = pf.puro_fp8_gemm(layout, *devops[:2], *devops[2:], bgran=bgran, out_dtype=out)
    torch.cuda.synchronize()
    if out == torch.float32:
        got = host(C).astype(np.float64)
        err = rel_frobenius(got, C_ref)
        assert err <= FROB_TOL, err
        bad = np.argwhere(np.abs(got - C_ref) > E)
        assert bad.size == 0, ("element bound", tuple(bad[0]))
    else:
        bits = host(C)
        got = bf16_to_f64(bits)
        bad = np.argwhere(np.abs(got - C_ref) > E + 2.0 ** -8 * (np.abs(C_ref) + E))
        assert bad.size == 0, ("element bound", tuple(bad[0]))
        exact = (bits == oracle.bf16_rne(C_ref)).mean()
        assert exact >= 0.99, exact
    return C_ref


SHAPES = [
    ("config1", 256, 256, 512),
    ("aligned_2x3", 512, 384, 768),
    ("tiles_3x2", 384, 256, 640),
    ("ragged", 200, 136, 300),
    ("ragged_thin", 130, 7, 1000),
    ("k_tail_only", 128, 128, 200),
    ("split_k", 256, 128, 2048),
    ("split_k_wide", 256, 256, 4096),
]


@pytest.mark.parametrize("out", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
@pytest.mark.parametrize("bgran", ["1x128", "128x128"])
@pytest.mark.parametrize("layout", ["NT", "NN", "TN"])
@pytest.mark.parametrize("name,M,N,K", SHAPES, ids=[s[0] for s in SHAPES])
def test_gemm_matches_oracle(dev, name, M, N, K, layout, bgran, out):
    X = synth.normal((M, K), 1.0, 1000 + M + K)
    W = synth.normal((N, K), 0.02 if name != "config1" else 1.0, 2000 + N + K)
    hostops, devops = _quantise_both(layout, bgran, X, W, ldx=_pad(K), ldw=_pad(K))
    _check_product(layout, bgran, hostops, devops, out)


def test_config1_single_forward(dev):
    """X 256x512, W 256x512, both N(0,1) FP32; X 1x128, W 128x128; FP32 output."""
    X = synth.normal((256, 512), 1.0, synth.seed_of(1, 0, 0))
    W = synth.normal((256, 512), 1.0, synth.seed_of(1, 0, 1))
    hostops, devops = _quantise_both("NT", "128x128", X, W)
    _check_product("NT", "128x128", hostops, devops, torch.float32)


def test_layer_shapes_reduced_tokens(dev):
    """The four fused projection shapes of one layer at 512 tokens, forward and data gradient."""
    for g, (name, n_out, k_in) in enumerate(synth.FUSED_GEMMS):
        X = synth.normal((512, k_in), 1.0, synth.seed_of(2, 0, 2 * g), "bf16")
        W = synth.normal((n_out, k_in), 0.02, synth.seed_of(2, 0, 2 * g + 1))
        Xf = synth.bf16_bits_to_f32(X)
        hostops, devops = _quantise_both("NT", "128x128", Xf, W)
        _check_product("NT", "128x128", hostops, devops, torch.float32)
        dY = synth.bf16_bits_to_f32(synth.normal((512, n_out), 1e-3, synth.seed_of(3, 0, 8 + g), "bf16"))
        # data gradient dX = dY W: logical A = dY [M][N_out], logical B^T = W^T [K_in][N_out]
        hostops, devops = _quantise_both("NN", "128x128", dY, np.ascontiguousarray(W.T))
        _check_product("NN", "128x128", hostops, devops, torch.float32)


def test_weight_gradient_nt_and_tn_agree(dev):
    T, Nout, Kin = 1024, 256, 384
    dY = synth.normal((T, Nout), 1e-3, 3001, "bf16")
    X = synth.normal((T, Kin), 1.0, 3002, "bf16")
    ddY, dX = to_dev(dY), to_dev(X)
    qa, sa = pf.puro_fp8_quant_transpose(ddY, True)
    qb, sb = pf.puro_fp8_quant_transpose(dX, True)
    C_nt = pf.puro_fp8_gemm("NT", qa, sa, qb, sb, bgran="1x128", out_dtype=torch.float32)
    qa2, sa2 = pf.puro_fp8_quant_transpose(ddY, False)
    qb2, sb2 = pf.puro_fp8_quant_transpose(dX, False)
    C_tn = pf.puro_fp8_gemm("TN", qa2, sa2, qb2, sb2, bgran="1x128", out_dtype=torch.float32)
    torch.cuda.synchronize()
    ra, rsa = oracle.quant_transpose(dY, True)
    rb, rsb = oracle.quant_transpose(X, True)
    C_ref = oracle.gemm("NT", ra, rsa, rb, rsb, "1x128")
    assert rel_frobenius(host(C_nt), C_ref) <= FROB_TOL
    assert rel_frobenius(host(C_tn), C_ref) <= FROB_TOL


def test_k_zero_writes_zeros(dev):
    A = torch.empty((64, 0), dtype=torch.uint8, device=dev)
    B = torch.empty((32, 0), dtype=torch.uint8, device=dev)
    sA = torch.empty((64, 0), dtype=torch.float32, device=dev)
    sB = torch.empty((32, 0), dtype=torch.float32, device=dev)
    C = torch.full((64, 32), 7.0, dtype=torch.float32, device=dev)
    pf.puro_fp8_gemm("NT", A, sA, B, sB, bgran="1x128", out_dtype=torch.float32, C=C)
    torch.cuda.synchronize()
    assert (C == 0).all()


def test_zero_blocks_and_outliers(dev):
    """Outlier channels x100 and all-zero 128-blocks in both operands (down-proj shape, 512 tokens)."""
    X, _ = synth.outlier_activations(512, 6144, 4001)
    W = synth.normal((2048, 6144), 0.02, 4002)
    hostops, devops = _quantise_both("NT", "128x128", synth.bf16_bits_to_f32(X), W)
    assert (hostops[1] == 0).any()
    _check_product("NT", "128x128", hostops, devops, torch.float32)


def test_output_padding_untouched(dev):
    X = synth.normal((200, 256), 1.0, 5001)
    W = synth.normal((100, 256), 0.02, 5002)
    hostops, devops = _quantise_both("NT", "128x128", X, W)
    buf = torch.full((200, 112), 123.0, dtype=torch.float32, device=dev)
    C = buf[:, :100]
    pf.puro_fp8_gemm("NT", devops[0], devops[1], devops[2], devops[3], bgran="128x128",
                     out_dtype=torch.float32, C=C)
    torch.cuda.synchronize()
    assert (buf[:, 100:] == 123.0).all()
    C_ref = oracle.gemm("NT", *hostops, "128x128")
    assert rel_frobenius(host(C), C_ref) <= FROB_TOL


def test_every_code_decodes_exactly(dev):
    """Each finite E4M3 code times 1.0, through both operand roles: the GEMM sees every value exactly."""
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
    M, K = codes.size, 128
    A = np.zeros((M, K), np.uint8)
    A[:, 0] = codes
    B = np.zeros((16, K), np.uint8)
    B[:, 0] = 0x38                      # 1.0
    sA = np.ones((M, 1), np.float32)
    sB = np.ones((16, 1), np.float32)
    want = oracle.e4m3_decode(codes)
    C = pf.puro_fp8_gemm("NT", to_dev(A), to_dev(sA), to_dev(B), to_dev(sB), bgran="1x128",
                         out_dtype=torch.float32)
    C2 = pf.puro_fp8_gemm("NT", to_dev(B), to_dev(sB), to_dev(A), to_dev(sA), bgran="1x128",
                          out_dtype=torch.float32)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(C)[:, 0].astype(np.float64), want)
    np.testing.assert_array_equal(host(C2)[0, :].astype(np.float64), want)
    assert (host(C)[:, 1:] == host(C)[:, :1]).all()


# Grouped launches: aligned problems (extents multiples of 128) share launches,
# the others (ragged, K tail) run on their own; empty ones are skipped.
GROUP = [(256, 384, 512), (200, 136, 300), (0, 128, 256), (128, 128, 1024), (128, 128, 200),
         (512, 256, 768), (384, 128, 128)]


@pytest.mark.parametrize("out", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
@pytest.mark.parametrize("bgran", ["1x128", "128x128"])
@pytest.mark.parametrize("layout", ["NT", "NN", "TN"])
def test_grouped_matches_oracle(dev, layout, bgran, out):
    ops = []
    for i, (M, N, K) in enumerate(GROUP):
        X = synth.normal((M, K), 1.0, 3000 + i)
        W = synth.normal((N, K), 0.02, 3100 + i)
        ops.append(_quantise_both(layout, bgran, X, W, ldx=_pad(K), ldw=_pad(K)))
    Cs = pf.puro_fp8_gemm_grouped(layout, [dv for _, dv in ops], bgran=bgran, out_dtype=out)
    for (hostops, devops), C in zip(ops, Cs):
        if C.numel():
            _check_product(layout, bgran, hostops, devops, out, C=C)


def test_grouped_more_problems_than_one_launch(dev):
    # 21 aligned problems (more than one launch holds) with mixed K
    ops = []
    for i in range(21):
        M, N, K = 128 * (1 + i % 3), 128 * (1 + i % 2), 128 * (1 + i % 5)
        X = synth.normal((M, K), 1.0, 3200 + i)
        W = synth.normal((N, K), 0.02, 3300 + i)
        ops.append(_quantise_both("NT", "128x128", X, W))
    Cs = pf.puro_fp8_gemm_grouped("NT", [dv for _, dv in ops], bgran="128x128", out_dtype=torch.float32)
    for (hostops, devops), C in zip(ops, Cs):
        _check_product("NT", "128x128", hostops, devops, torch.float32, C=C)


# Equally deep problems whose tile count is a multiple of 8: the launch hands
# each XCD a contiguous eighth of all its tiles, so eighths start and end inside
# problems (128x128 tiles: 6+6+5+4+3 = 24; 256x256-eligible extents: 16 tiles).
EQUAL_DEPTH = {
    "tiles128": ([(256, 384), (384, 256), (128, 640), (512, 128), (128, 384)], 640),
    "tiles256": ([(512, 512), (256, 768), (768, 256), (512, 512), (512, 256)], 1024),
}


@pytest.mark.parametrize("out", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
@pytest.mark.parametrize("group", sorted(EQUAL_DEPTH))
def test_grouped_equal_depth_xcd_eighths(dev, group, out):
    shapes, K = EQUAL_DEPTH[group]
    for bgran in ("1x128", "128x128"):
        ops = []
        for i, (M, N) in enumerate(shapes):
            X = synth.normal((M, K), 1.0, 3600 + i)
            W = synth.normal((N, K), 0.02, 3700 + i)
            ops.append(_quantise_both("NT", bgran, X, W))
        Cs = pf.puro_fp8_gemm_grouped("NT", [dv for _, dv in ops], bgran=bgran, out_dtype=out)
        for (hostops, devops), C in zip(ops, Cs):
            _check_product("NT", bgran, hostops, devops, out, C=C)


def test_grouped_layer_projections_reduced_tokens(dev):
    # the q, k, v projections of one input and the gate/up pair, 512 tokens:
    # grouped forward products equal the single calls' to the parity bound
    T = 512
    for names in (("q", "k", "v"), ("gate", "up")):
        gemms = [g for g in synth.LAYER_GEMMS if g[0] in names]
        K = gemms[0][2]
        X = synth.normal((T, K), 1.0, 3400 + K)
        ops = []
        for j, (g, n, k, src) in enumerate(gemms):
            W = synth.normal((n, k), 0.02, 3500 + j)
            ops.append(_quantise_both("NT", "128x128", X, W))
        Cs = pf.puro_fp8_gemm_grouped("NT", [dv for _, dv in ops], out_dtype=torch.bfloat16)
        for (hostops, devops), C in zip(ops, Cs):
            _check_product("NT", "128x128", hostops, devops, torch.bfloat16, C=C)


def _check_sum(layout, bgran, segs_host, C, out, c_old=None):
    """C against the oracle's segment sum (plus c_old): FP32 accumulation bound over all
    the segments' blocks, one more rounding for the addition of c_old, one BF16 rounding."""
    C_ref = oracle.gemm_segments(layout, segs_host, bgran, c_init=c_old)
    kb = sum(((qa.shape[0] if layout == "TN" else qa.shape[1]) + 127) // 128 for qa, _, _, _ in segs_host)
    c_abs = sum(oracle.gemm(layout, qa & 0x7F, np.abs(sa), qb & 0x7F, np.abs(sb), bgran)
                for qa, sa, qb, sb in segs_host)
    E = (kb + 4) * 2.0 ** -23 * c_abs
    if c_old is not None:
        E = E + 2.0 ** -23 * np.abs(c_old)
    torch.cuda.synchronize()
    if out == torch.float32:
        got = host(C).astype(np.float64)
        assert rel_frobenius(got, C_ref) <= FROB_TOL
        bad = np.argwhere(np.abs(got - C_ref) > E)
        assert bad.size == 0, ("element bound", tuple(bad[0]))
    else:
        bits = host(C)
        got = bf16_to_f64(bits)
        bad = np.argwhere(np.abs(got - C_ref) > E + 2.0 ** -8 * (np.abs(C_ref) + E))
        assert bad.size == 0, ("element bound", tuple(bad[0]))
        assert (bits == oracle.bf16_rne(C_ref)).mean() >= 0.99


# K-segment sums: (M, N, segment K's); aligned ones take the tile kernel, the others
# the bounds-checked one
SUMS = [(256, 384, (256, 384)), (200, 136, (300, 72)), (128, 128, (128, 256, 128, 512)), (256, 128, (200, 128))]


@pytest.mark.parametrize("out", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
@pytest.mark.parametrize("bgran", ["1x128", "128x128"])
@pytest.mark.parametrize("layout", ["NT", "NN", "TN"])
def test_grouped_segment_sums_match_oracle(dev, layout, bgran, out):
    probs, hosts = [], []
    for i, (M, N, ks) in enumerate(SUMS):
        hs, ds = [], []
        for j, K in enumerate(ks):
            X = synth.normal((M, K), 1.0, 3600 + 10 * i + j)
            W = synth.normal((N, K), 0.02, 3700 + 10 * i + j)
            h, d = _quantise_both(layout, bgran, X, W, ldx=_pad(K), ldw=_pad(K))
            hs.append(h)
            ds.append(d)
        probs.append({"segments": ds})
        hosts.append(hs)
    Cs = pf.puro_fp8_gemm_grouped(layout, probs, bgran=bgran, out_dtype=out)
    for hs, C in zip(hosts, Cs):
        _check_sum(layout, bgran, hs, C, out)


@pytest.mark.parametrize("out", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
@pytest.mark.parametrize("shape", [(256, 256, (512,)), (200, 136, (300,)), (128, 256, (256, 128))],
                         ids=["aligned", "ragged", "two_segments"])
def test_grouped_accumulate_into_output(dev, shape, out):
    M, N, ks = shape
    hs, ds = [], []
    for j, K in enumerate(ks):
        X = synth.normal((M, K), 1.0, 3800 + j)
        W = synth.normal((N, K), 0.02, 3900 + j)
        h, d = _quantise_both("NT", "1x128", X, W, ldx=_pad(K), ldw=_pad(K))
        hs.append(h)
        ds.append(d)
    C = to_dev(synth.normal((M, N), 0.5, 3999, "bf16" if out == torch.bfloat16 else "f32"), ld=_pad(N))
    # two passes, each checked against the oracle started from the output before it
    for _ in range(2):
        torch.cuda.synchronize()
        prev = host(C)
        prev = prev.astype(np.float64) if out == torch.float32 else bf16_to_f64(prev)
        pf.puro_fp8_gemm_grouped("NT", [{"segments": ds, "C": C, "accumulate": True}], bgran="1x128",
                                 out_dtype=out)
        _check_sum("NT", "1x128", hs, C, out, c_old=prev)
