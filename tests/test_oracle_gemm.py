"""Pins for the oracle's blockwise GEMM (CPU only).

The GEMM oracle is the definition
    C[m][n] = sum_kb sA(m,kb) sB(n,kb) sum_{k in kb} a(m,k) b(k,n)
in FP64.  It is pinned by
  * a library product of the unquantised inputs: when every block of X and W
    is an E4M3 value times a power of two and holds a +-448*2^k element, the
    quantisers are lossless, so quantise-then-GEMM must equal numpy's FP64
    matmul of X and W (a dropped scale, a transposed operand or a wrong block
    index all break this);
  * a brute-force dequantise-then-triple-loop on tiny shapes;
  * closed forms: constant blocks give C = K * alpha * beta; zero blocks
    contribute nothing; and the NT / TN weight-gradient layouts agree.
"""
import numpy as np
import pytest

import oracle
import synth

FINITE = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)


def _lossless(rows, cols, seed):
    """Every 1x128 row block, 128x1 column block and 128x128 tile holds a +-448*2^k element,
    with one power-of-two 2^k per 128x128 tile, so all three quantisers are exact on it."""
    rng = np.random.default_rng(seed)
    codes = rng.choice(FINITE, size=(rows, cols))
    rb, cb = (rows + 127) // 128, (cols + 127) // 128
    for ti in range(rb):
        for tj in range(cb):
            nr = min(128, rows - ti * 128)
            nc = min(128, cols - tj * 128)
            for i in range(nr):
                codes[ti * 128 + i, tj * 128 + (i % nc)] = 0x7E | rng.choice([0, 0x80])
            for j in range(nc):
                codes[ti * 128 + (j % nr), tj * 128 + j] = 0x7E | rng.choice([0, 0x80])
    k = rng.integers(-6, 6, size=(rb, cb))
    scale = np.repeat(np.repeat(np.ldexp(1.0, k), 128, axis=0), 128, axis=1)[:rows, :cols]
    return (oracle.e4m3_decode(codes) * scale).astype(np.float32)


def _quantise_operands(layout, bgran, X, W):
    """X is the logical [M][K] operand, W the logical [N][K]; returns storage-form operands."""
    if layout == "NT":
        qa, sa = oracle.quant_act(X)
        qb, sb = oracle.quant_weight(W) if bgran == "128x128" else oracle.quant_act(W)
    elif layout == "NN":
        qa, sa = oracle.quant_act(X)
        Wkn = np.ascontiguousarray(W.T)
        qb, sb = (oracle.quant_weight(Wkn) if bgran == "128x128"
                  else oracle.quant_transpose(Wkn, transpose_out=False))
    else:
        qa, sa = oracle.quant_transpose(np.ascontiguousarray(X.T), transpose_out=False)
        Wkn = np.ascontiguousarray(W.T)
        qb, sb = (oracle.quant_weight(Wkn) if bgran == "128x128"
                  else oracle.quant_transpose(Wkn, transpose_out=False))
    return qa, sa, qb, sb


CASES = [(256, 256, 512), (200, 136, 300), (128, 384, 128), (1, 1, 1), (130, 7, 1000)]


@pytest.mark.parametrize("layout", ["NT", "NN", "TN"])
@pytest.mark.parametrize("bgran", ["1x128", "128x128"])
@pytest.mark.parametrize("M,N,K", CASES)
def test_lossless_pipeline_equals_library_matmul(layout, bgran, M, N, K):
    X = _lossless(M, K, 100 + M + K)
    W = _lossless(N, K, 200 + N + K)
    qa, sa, qb, sb = _quantise_operands(layout, bgran, X, W)
    C = oracle.gemm(layout, qa, sa, qb, sb, bgran)
    ref = X.astype(np.float64) @ W.astype(np.float64).T
    denom = np.abs(X.astype(np.float64)) @ np.abs(W.astype(np.float64)).T + 1e-300
    assert (np.abs(C - ref) / denom <= 1e-13).all()


@pytest.mark.parametrize("layout", ["NT", "NN", "TN"])
@pytest.mark.parametrize("bgran", ["1x128", "128x128"])
@pytest.mark.parametrize("M,N,K", [(128, 128, 256), (256, 128, 512), (72, 200, 260)])
def test_blockwise_equals_brute_force(layout, bgran, M, N, K):
    X = synth.normal((M, K), 1.0, 300 + K)
    W = synth.normal((N, K), 0.02, 301 + K)
    qa, sa, qb, sb = _quantise_operands(layout, bgran, X, W)
    C = oracle.gemm(layout, qa, sa, qb, sb, bgran)
    Cb = oracle.gemm_brute(layout, qa, sa, qb, sb, bgran)
    np.testing.assert_allclose(C, Cb, rtol=1e-12, atol=1e-12 * np.abs(Cb).max())


@pytest.mark.parametrize("layout", ["NT", "NN", "TN"])
def test_constant_blocks_closed_form(layout):
    M, N, K = 128, 256, 384
    alpha = np.float32(0.37)
    beta = np.float32(-5.5)
    X = np.full((M, K), alpha, np.float32)
    W = np.full((N, K), beta, np.float32)
    qa, sa, qb, sb = _quantise_operands(layout, "128x128", X, W)
    assert (qa == 0x7E).all() and (qb == 0xFE).all()
    C = oracle.gemm(layout, qa, sa, qb, sb, "128x128")
    # every element: sum over K of (448 sA)(−448 sB) with 448 sA = fl(alpha/448)*448
    want = K * (448.0 * np.float64(sa.flat[0])) * (-448.0 * np.float64(sb.flat[0]))
    np.testing.assert_allclose(C, want, rtol=1e-15)
    np.testing.assert_allclose(C, K * np.float64(alpha) * np.float64(beta), rtol=1e-6)


def test_zero_blocks_contribute_nothing():
    M, N, K = 128, 128, 512
    X = synth.normal((M, K), 1.0, 400)
    W = synth.normal((N, K), 0.02, 401)
    qa, sa = oracle.quant_act(X)
    qb, sb = oracle.quant_weight(W)
    C_full = oracle.gemm("NT", qa, sa, qb, sb)
    X2 = X.copy()
    X2[:, 256:384] = 0.0
    qa2, sa2 = oracle.quant_act(X2)
    C2 = oracle.gemm("NT", qa2, sa2, qb, sb)
    # removing block 2 of K from A equals the product over the other blocks only
    keep = np.r_[0:256, 384:512]
    qa3, sa3 = oracle.quant_act(np.ascontiguousarray(X[:, keep]))
    qb3, sb3 = oracle.quant_weight(np.ascontiguousarray(W[:, keep]))
    # weight tiles over the kept columns are the same tiles as before (tile-aligned removal)
    np.testing.assert_array_equal(sb3, sb[:, [0, 1, 3]])
    C3 = oracle.gemm("NT", qa3, sa3, qb3, sb3)
    np.testing.assert_allclose(C2, C3, rtol=1e-14, atol=1e-14)
    assert np.abs(C2 - C_full).max() > 0


def test_weight_gradient_nt_equals_tn():
    T, Nout, Kin = 512, 128, 256
    dY = synth.normal((T, Nout), 1e-3, 500, dtype="bf16")
    X = synth.normal((T, Kin), 1.0, 501, dtype="bf16")
    qa_t, sa_t = oracle.quant_transpose(dY, transpose_out=True)    # [Nout][T]
    qb_t, sb_t = oracle.quant_transpose(X, transpose_out=True)     # [Kin][T]
    C_nt = oracle.gemm("NT", qa_t, sa_t, qb_t, sb_t, "1x128")
    qa_n, sa_n = oracle.quant_transpose(dY, transpose_out=False)   # [T][Nout]
    qb_n, sb_n = oracle.quant_transpose(X, transpose_out=False)    # [T][Kin]
    C_tn = oracle.gemm("TN", qa_n, sa_n, qb_n, sb_n, "1x128")
    np.testing.assert_array_equal(C_nt, C_tn)


def test_entries_equal_full_product():
    M, N, K = 200, 136, 300
    X = synth.normal((M, K), 1.0, 600)
    W = synth.normal((N, K), 0.02, 601)
    for layout in ("NT", "NN", "TN"):
        qa, sa, qb, sb = _quantise_operands(layout, "128x128", X, W)
        C = oracle.gemm(layout, qa, sa, qb, sb, "128x128")
        rng = np.random.default_rng(7)
        ms = rng.integers(0, M, 500)
        ns = rng.integers(0, N, 500)
        np.testing.assert_array_equal(oracle.gemm_entries(layout, qa, sa, qb, sb, "128x128", ms, ns),
                                      C[ms, ns])


def test_empty_and_k_zero():
    qa = np.zeros((4, 0), np.uint8)
    sa = np.zeros((4, 0), np.float32)
    qb = np.zeros((3, 0), np.uint8)
    sb = np.zeros((3, 0), np.float32)
    C = oracle.gemm("NT", qa, sa, qb, sb, "1x128")
    assert C.shape == (4, 3) and (C == 0).all()


# Sums over K segments (the partial products one input's gradient receives
# from several projections, and the accumulate-into output).  Pinned by the
# lossless pipeline: the segments of a split K range must give numpy's FP64
# product of the whole operands, whatever the split (ragged pieces included).
@pytest.mark.parametrize("layout", ["NT", "NN", "TN"])
@pytest.mark.parametrize("bgran", ["1x128", "128x128"])
@pytest.mark.parametrize("M,N,ks", [(256, 128, (256, 384)), (200, 136, (300, 72, 128)), (128, 256, (128,))])
def test_segments_equal_the_whole_product(layout, bgran, M, N, ks):
    segs, Xs, Ws = [], [], []
    for i, K in enumerate(ks):
        X = _lossless(M, K, 400 + i * 7 + K)
        W = _lossless(N, K, 500 + i * 7 + K)
        segs.append(_quantise_operands(layout, bgran, X, W))
        Xs.append(X)
        Ws.append(W)
    C = oracle.gemm_segments(layout, segs, bgran)
    X = np.concatenate(Xs, axis=1).astype(np.float64)
    W = np.concatenate(Ws, axis=1).astype(np.float64)
    ref = X @ W.T
    denom = np.abs(X) @ np.abs(W).T + 1e-300
    assert (np.abs(C - ref) / denom <= 1e-13).all()


def test_segments_accumulate_onto_c_init():
    M, N, K = 130, 128, 256
    X = _lossless(M, K, 601)
    W = _lossless(N, K, 602)
    seg = _quantise_operands("NT", "128x128", X, W)
    c0 = synth.normal((M, N), 3.0, 603).astype(np.float64)
    C = oracle.gemm_segments("NT", [seg], "128x128", c_init=c0)
    ref = c0 + X.astype(np.float64) @ W.astype(np.float64).T
    np.testing.assert_allclose(C, ref, rtol=1e-13, atol=1e-13 * np.abs(ref).max())
