"""GPU parity at the workload's full sizes, in the launch configurations the
benchmark uses, on sampled outputs.

Inputs are the seeded host tensors of the Qwen3-1.7B layer shapes (8,192
tokens; hidden 2,048, FFN 6,144, 16/8 heads) and of the outlier-stress
down-projection shape (16,384 tokens).  The oracle quantises the same inputs
(its codes and scales must equal the GPU's byte for byte over the whole
tensors) and computes sampled output entries one by one.  Sampled entries
must meet the per-element bound (KB + 4) 2^-23 sum|terms| (plus half a BF16
ulp for BF16 outputs) and the sampled relative Frobenius error must be
<= 2e-6.
"""
import numpy as np
import pytest
import torch

import blockwise_fp8_gemm_amd as pf
import oracle
import synth
from helpers import bf16_to_f64, first_mismatch, host, to_dev

pytestmark = pytest.mark.gpu

SAMPLES = 3000


def _same(dev_t, ref, what):
    got = host(dev_t)
    if got.dtype == np.float32:
        got, ref = got.view(np.uint32), ref.view(np.uint32)
    assert first_mismatch(got, ref) is None, (what, first_mismatch(got, ref))


def _check_sampled(layout, bgran, ops, C, K, seed, out):
    qa, sa, qb, sb = ops
    M, N = C.shape
    rng = np.random.default_rng(seed)
    ms = rng.integers(0, M, SAMPLES)
    ns = rng.integers(0, N, SAMPLES)
    ms[:4] = [0, 0, M - 1, M - 1]
    ns[:4] = [0, N - 1, 0, N - 1]
    ref = oracle.gemm_entries(layout, qa, sa, qb, sb, bgran, ms, ns)
    ref_abs = oracle.gemm_entries(layout, qa & 0x7F, np.abs(sa), qb & 0x7F, np.abs(sb), bgran, ms, ns)
    E = ((K + 127) // 128 + 4) * 2.0 ** -23 * ref_abs
    h = host(C)
    got = bf16_to_f64(h[ms, ns]) if out == torch.bfloat16 else h[ms, ns].astype(np.float64)
    tol = E + 2.0 ** -8 * (np.abs(ref) + E) if out == torch.bfloat16 else E
    bad = np.flatnonzero(np.abs(got - ref) > tol)
    assert bad.size == 0, ("entry", int(ms[bad[0]]), int(ns[bad[0]]), got[bad[0]], ref[bad[0]])
    if out == torch.float32:
        err = np.linalg.norm(got - ref) / np.linalg.norm(ref)
        assert err <= 2e-6, err


def _workspace(layout, M, N, K, bgran, dev):
    n = pf.puro_fp8_gemm_workspace_size(layout, M, N, K, bgran)
    return torch.empty(max(n, 256), dtype=torch.uint8, device=dev), n


LAYER = [(g, n, k) for g, n, k, _ in synth.LAYER_GEMMS if g in ("q", "k", "gate", "down")]


@pytest.mark.parametrize("g,n_out,k_in", LAYER, ids=[x[0] for x in LAYER])
def test_layer_gemm_full_size(dev, g, n_out, k_in):
    """Forward, data gradient and weight gradient of one projection at 8,192 tokens."""
    T = synth.TOKENS
    j = [x[0] for x in synth.LAYER_GEMMS].index(g)
    X = synth.normal((T, k_in), 1.0, synth.seed_of(2, 0, 100 + j), "bf16")
    W = synth.normal((n_out, k_in), 0.02, synth.seed_of(2, 0, 110 + j))
    dY = synth.normal((T, n_out), 1e-3, synth.seed_of(3, 0, 120 + j), "bf16")
    dX_, dW_, ddY = to_dev(X), to_dev(W), to_dev(dY)

    rqx, rsx = oracle.quant_act(X)
    rqw, rsw = oracle.quant_weight(W)
    rqd, rsd = oracle.quant_act(dY)
    rqdt, rsdt = oracle.quant_transpose(dY, True)
    rqxt, rsxt = oracle.quant_transpose(X, True)

    qx, sx = pf.puro_fp8_quant_act(dX_)
    qw, sw = pf.puro_fp8_quant_weight(dW_)
    qd, sd = pf.puro_fp8_quant_act(ddY)
    qdt, sdt = pf.puro_fp8_quant_transpose(ddY, True)
    qxt, sxt = pf.puro_fp8_quant_transpose(dX_, True)
    torch.cuda.synchronize()
    for t, r, w in ((qx, rqx, "qX"), (sx, rsx, "sX"), (qw, rqw, "qW"), (sw, rsw, "sW"), (qd, rqd, "qdY"),
                    (sd, rsd, "sdY"), (qdt, rqdt, "qdYt"), (sdt, rsdt, "sdYt"), (qxt, rqxt, "qXt"),
                    (sxt, rsxt, "sXt")):
        _same(t, r, w)

    ws, nws = _workspace("NT", T, n_out, k_in, "128x128", dev)
    Y = pf.puro_fp8_gemm("NT", qx, sx, qw, sw, "128x128", torch.bfloat16, workspace=ws if nws else None)
    ws, nws = _workspace("NN", T, k_in, n_out, "128x128", dev)
    dXg = pf.puro_fp8_gemm("NN", qd, sd, qw, sw, "128x128", torch.bfloat16, workspace=ws if nws else None)
    ws, nws = _workspace("NT", n_out, k_in, T, "1x128", dev)
    dWg = pf.puro_fp8_gemm("NT", qdt, sdt, qxt, sxt, "1x128", torch.float32, workspace=ws if nws else None)
    torch.cuda.synchronize()
    _check_sampled("NT", "128x128", (rqx, rsx, rqw, rsw), Y, k_in, 1, torch.bfloat16)
    _check_sampled("NN", "128x128", (rqd, rsd, rqw, rsw), dXg, n_out, 2, torch.bfloat16)
    _check_sampled("NT", "1x128", (rqdt, rsdt, rqxt, rsxt), dWg, T, 3, torch.float32)


@pytest.mark.parametrize("random_sign", [False, True], ids=["positive_dY", "random_sign_dY"])
def test_outlier_stress_full_size(dev, random_sign):
    """Down-projection shape at 16,384 tokens: 1% of channels x100, lognormal gradients
    (the literal positive ones, and the random-sign variant the outlier-stress row lists as a
    parity-only extra), all-zero 128-blocks; forward, data gradient, weight gradient (FP32
    outputs)."""
    T, K_in, N_out = 16384, 6144, 2048
    X, _ = synth.outlier_activations(T, K_in, synth.seed_of(5, 0, 0))
    dY = synth.lognormal_gradients(T, N_out, synth.seed_of(5, 0, 1), random_sign=random_sign)
    if random_sign:
        assert (synth.bf16_bits_to_f32(dY) < 0).mean() > 0.45
    W = synth.normal((N_out, K_in), 0.02, synth.seed_of(5, 0, 2))
    dX_, dW_, ddY = to_dev(X), to_dev(W), to_dev(dY)
    rqx, rsx = oracle.quant_act(X)
    rqw, rsw = oracle.quant_weight(W)
    rqd, rsd = oracle.quant_act(dY)
    rqdt, rsdt = oracle.quant_transpose(dY, True)
    rqxt, rsxt = oracle.quant_transpose(X, True)
    assert (rsx == 0).any() and (rsdt == 0).any()
    qx, sx = pf.puro_fp8_quant_act(dX_)
    qw, sw = pf.puro_fp8_quant_weight(dW_)
    qd, sd = pf.puro_fp8_quant_act(ddY)
    qdt, sdt = pf.puro_fp8_quant_transpose(ddY, True)
    qxt, sxt = pf.puro_fp8_quant_transpose(dX_, True)
    torch.cuda.synchronize()
    for t, r, w in ((qx, rqx, "qX"), (sx, rsx, "sX"), (qw, rqw, "qW"), (qd, rqd, "qdY"), (sd, rsd, "sdY"),
                    (qdt, rqdt, "qdYt"), (sdt, rsdt, "sdYt"), (qxt, rqxt, "qXt"), (sxt, rsxt, "sXt")):
        _same(t, r, w)
    outs = []
    for layout, A, sA, B, sB, bg, K in (("NT", qx, sx, qw, sw, "128x128", K_in),
                                        ("NN", qd, sd, qw, sw, "128x128", N_out),
                                        ("NT", qdt, sdt, qxt, sxt, "1x128", T)):
        M, N, _ = pf.gemm_dims(layout, A, B)
        ws, nws = _workspace(layout, M, N, K, bg, dev)
        outs.append(pf.puro_fp8_gemm(layout, A, sA, B, sB, bg, torch.float32, workspace=ws if nws else None))
    torch.cuda.synchronize()
    _check_sampled("NT", "128x128", (rqx, rsx, rqw, rsw), outs[0], K_in, 4, torch.float32)
    _check_sampled("NN", "128x128", (rqd, rsd, rqw, rsw), outs[1], N_out, 5, torch.float32)
    _check_sampled("NT", "1x128", (rqdt, rsdt, rqxt, rsxt), outs[2], T, 6, torch.float32)


def _check_sampled_sum(layout, bgran, segs, C, seed, out):
    """Sampled entries of a K-segment sum against the oracle (bound over all segments' blocks)."""
    M, N = C.shape
    rng = np.random.default_rng(seed)
    ms = rng.integers(0, M, SAMPLES)
    ns = rng.integers(0, N, SAMPLES)
    ms[:4] = [0, 0, M - 1, M - 1]
    ns[:4] = [0, N - 1, 0, N - 1]
    ref = np.zeros(SAMPLES)
    ref_abs = np.zeros(SAMPLES)
    kb = 0
    for qa, sa, qb, sb in segs:
        ref += oracle.gemm_entries(layout, qa, sa, qb, sb, bgran, ms, ns)
        ref_abs += oracle.gemm_entries(layout, qa & 0x7F, np.abs(sa), qb & 0x7F, np.abs(sb), bgran, ms, ns)
        kb += ((qa.shape[0] if layout == "TN" else qa.shape[1]) + 127) // 128
    E = (kb + 4) * 2.0 ** -23 * ref_abs
    h = host(C)
    got = bf16_to_f64(h[ms, ns]) if out == torch.bfloat16 else h[ms, ns].astype(np.float64)
    tol = E + 2.0 ** -8 * (np.abs(ref) + E) if out == torch.bfloat16 else E
    bad = np.flatnonzero(np.abs(got - ref) > tol)
    assert bad.size == 0, ("entry", int(ms[bad[0]]), int(ns[bad[0]]), got[bad[0]], ref[bad[0]])
    if out == torch.float32:
        assert np.linalg.norm(got - ref) / np.linalg.norm(ref) <= 2e-6


def test_layer_grouped_full_size(dev):
    """One whole layer at 8,192 tokens in the grouped launches the benchmark times: every
    input and output gradient quantised both ways in one read and the seven weights in one
    launch (byte-compared over the whole tensors), the forward products grouped (q/k/v, o, gate/up, down), the data gradients
    summed per input (K segments), and the seven weight gradients in one launch."""
    T = synth.TOKENS
    shape = {g: (n, k, src) for g, n, k, src in synth.LAYER_GEMMS}
    host_q, dev_q = {}, {}

    def dual(name, x):
        d = pf.puro_fp8_quant_dual(to_dev(x), True)
        r = oracle.quant_act(x) + oracle.quant_transpose(x, True)
        torch.cuda.synchronize()
        for t, ref, what in zip(d, r, ("q_row", "s_row", "q_tok", "s_tok")):
            _same(t, ref, (name, what))
        host_q[name], dev_q[name] = r, d

    for i, (name, c) in enumerate(synth.LAYER_INPUTS):
        dual(name, synth.normal((T, c), 1.0, synth.seed_of(4, 0, i), "bf16"))
    Ws = {}
    for j, (g, n, k, src) in enumerate(synth.LAYER_GEMMS):
        dual("dY_" + g, synth.normal((T, n), 1e-3, synth.seed_of(4, 0, 20 + j), "bf16"))
        Ws[g] = synth.normal((n, k), 0.02, synth.seed_of(4, 0, 10 + j))
    # the layer's seven weights in one grouped launch, as the benchmark does
    gs = [g for g, _, _, _ in synth.LAYER_GEMMS]
    qws = pf.puro_fp8_quant_weight_grouped([to_dev(Ws[g]) for g in gs])
    torch.cuda.synchronize()
    for g, (qw, sw) in zip(gs, qws):
        rw = oracle.quant_weight(Ws[g])
        _same(qw, rw[0], ("qW", g))
        _same(sw, rw[1], ("sW", g))
        host_q["W_" + g], dev_q["W_" + g] = rw, (qw, sw)

    seed = 10
    for gs in (("q", "k", "v"), ("o",), ("gate", "up"), ("down",)):
        src = shape[gs[0]][2]
        (hqx, hsx), (dqx, dsx) = host_q[src][:2], dev_q[src][:2]
        Ys = pf.puro_fp8_gemm_grouped("NT", [(dqx, dsx) + dev_q["W_" + g] for g in gs], out_dtype=torch.bfloat16)
        torch.cuda.synchronize()
        for g, Y in zip(gs, Ys):
            seed += 1
            _check_sampled("NT", "128x128", (hqx, hsx) + host_q["W_" + g], Y, shape[g][1], seed, torch.bfloat16)
    for gs in (("down",), ("gate", "up"), ("o",), ("q", "k", "v")):
        dsegs = [dev_q["dY_" + g][:2] + dev_q["W_" + g] for g in gs]
        hsegs = [host_q["dY_" + g][:2] + host_q["W_" + g] for g in gs]
        (dX,) = pf.puro_fp8_gemm_grouped("NN", [{"segments": dsegs}], out_dtype=torch.bfloat16)
        torch.cuda.synchronize()
        seed += 1
        _check_sampled_sum("NN", "128x128", hsegs, dX, seed, torch.bfloat16)
    gs = [g for g, _, _, _ in synth.LAYER_GEMMS]
    dWs = pf.puro_fp8_gemm_grouped("NT", [dev_q["dY_" + g][2:] + dev_q[shape[g][2]][2:] for g in gs],
                                   bgran="1x128", out_dtype=torch.float32)
    torch.cuda.synchronize()
    for g, dW in zip(gs, dWs):
        seed += 1
        _check_sampled("NT", "1x128", host_q["dY_" + g][2:] + host_q[shape[g][2]][2:], dW, T, seed, torch.float32)


def test_layer_adjacent_full_size(dev):
    """One whole layer at 8,192 tokens as the benchmark's step runs it: the q/k/v and gate/up
    weights quantised into adjacent rows of one buffer per group (each weight as an item, and
    each group's adjacent master weights as one item with its transposed copy: the same codes),
    each group's output gradient quantised both ways in one call, each group's forward product
    one GEMM, the data gradient of each input one NT GEMM over the group's concatenated K on the
    transposed codes, and the seven weight gradients, on row ranges of the groups' token-blocked
    copies, in one launch.  Codes and scales byte-compared over whole tensors; products on
    sampled entries against the oracle's NT / NN definitions."""
    T = synth.TOKENS
    shape = {g: (n, k, src) for g, n, k, src in synth.LAYER_GEMMS}
    inputs = dict(synth.LAYER_INPUTS)
    host_q, dev_q = {}, {}

    def dual(name, x):
        d = pf.puro_fp8_quant_dual(to_dev(x), True)
        r = oracle.quant_act(x) + oracle.quant_transpose(x, True)
        torch.cuda.synchronize()
        for t, ref, what in zip(d, r, ("q_row", "s_row", "q_tok", "s_tok")):
            _same(t, ref, (name, what))
        host_q[name], dev_q[name] = r, d

    for i, (name, c) in enumerate(synth.LAYER_INPUTS):
        dual(name, synth.normal((T, c), 1.0, synth.seed_of(4, 0, i), "bf16"))
    rows, width = {}, {}
    for G, members, _ in synth.PROJ_GROUPS:
        r0 = 0
        for g in members:
            rows[g] = (G, r0)
            r0 += shape[g][0]
        width[G] = r0
    for j, (G, _, _) in enumerate(synth.PROJ_GROUPS):
        dual("dY_" + G, synth.normal((T, width[G]), 1e-3, synth.seed_of(4, 0, 30 + j), "bf16"))
    # the seven weights in one launch, each into its rows of its group's buffers
    qwG = {G: torch.empty((width[G], inputs[src]), dtype=torch.uint8, device=dev) for G, _, src in synth.PROJ_GROUPS}
    swG = {G: torch.empty((width[G] // 128, inputs[src] // 128), dtype=torch.float32, device=dev)
           for G, _, src in synth.PROJ_GROUPS}
    Ws, outs, gs = {}, [], [g for g, _, _, _ in synth.LAYER_GEMMS]
    for j, (g, n, k, _) in enumerate(synth.LAYER_GEMMS):
        Ws[g] = synth.normal((n, k), 0.02, synth.seed_of(4, 0, 10 + j))
        G, r0 = rows[g]
        outs.append((qwG[G][r0:r0 + n], swG[G][r0 // 128:(r0 + n) // 128]))
    pf.puro_fp8_quant_weight_grouped([to_dev(Ws[g]) for g in gs], outs=outs)
    # the benchmark quantises each group's adjacent master weights as one weight, with the
    # transposed copy its data gradient reads: the same tiles, so the same codes and scales
    WG = {G: np.concatenate([Ws[g] for g in members]) for G, members, _ in synth.PROJ_GROUPS}
    G4 = [G for G, _, _ in synth.PROJ_GROUPS]
    tq = pf.puro_fp8_quant_weight_grouped([to_dev(WG[G]) for G in G4], transposed=True)
    torch.cuda.synchronize()
    hq, hs, qwtG, swtG = {}, {}, {}, {}
    for (G, members, _), (q4, s4, qt4, st4) in zip(synth.PROJ_GROUPS, tq):
        refs = [oracle.quant_weight(Ws[g]) for g in members]
        hq[G] = np.concatenate([r[0] for r in refs])
        hs[G] = np.concatenate([r[1] for r in refs])
        _same(qwG[G], hq[G], ("qW", G))
        _same(swG[G], hs[G], ("sW", G))
        _same(q4, hq[G], ("qW whole group", G))
        _same(s4, hs[G], ("sW whole group", G))
        _same(qt4, np.ascontiguousarray(hq[G].T), ("qW transposed", G))
        _same(st4, np.ascontiguousarray(hs[G].T), ("sW transposed", G))
        qwtG[G], swtG[G] = qt4, st4

    seed = 100
    for G, _, src in synth.PROJ_GROUPS:
        (hqx, hsx), (dqx, dsx) = host_q[src][:2], dev_q[src][:2]
        (Y,) = pf.puro_fp8_gemm_grouped("NT", [(dqx, dsx, qwG[G], swG[G])], out_dtype=torch.bfloat16)
        (dX,) = pf.puro_fp8_gemm_grouped("NT", [dev_q["dY_" + G][:2] + (qwtG[G], swtG[G])],
                                         out_dtype=torch.bfloat16)
        torch.cuda.synchronize()
        _check_sampled("NT", "128x128", (hqx, hsx, hq[G], hs[G]), Y, inputs[src], seed + 1, torch.bfloat16)
        # dX = dY W: the oracle's NN product of the untransposed codes
        _check_sampled("NN", "128x128", host_q["dY_" + G][:2] + (hq[G], hs[G]), dX, width[G], seed + 2,
                       torch.bfloat16)
        seed += 2
    probs, hprobs = [], []
    for g in gs:
        n, k, src = shape[g]
        G, r0 = rows[g]
        qt, st = dev_q["dY_" + G][2:]
        hqt, hst = host_q["dY_" + G][2:]
        probs.append((qt[r0:r0 + n], st[r0:r0 + n]) + dev_q[src][2:])
        hprobs.append((hqt[r0:r0 + n], hst[r0:r0 + n]) + host_q[src][2:])
    dWs = pf.puro_fp8_gemm_grouped("NT", probs, bgran="1x128", out_dtype=torch.float32)
    torch.cuda.synchronize()
    for g, dW, hp in zip(gs, dWs, hprobs):
        seed += 1
        _check_sampled("NT", "1x128", hp, dW, T, seed, torch.float32)


def _check_sampled_mc(layout, bgran, ops, C, K, seed, out):
    """_check_sampled with the matrix-core bound of the native and MX datapaths:
    2^-9 C_abs + (4 KB + 4) 2^-23 C_abs per entry (plus half a BF16 ulp), and a sampled
    relative Frobenius error of at most 1e-3 for FP32 outputs."""
    qa, sa, qb, sb = ops
    M, N = C.shape
    rng = np.random.default_rng(seed)
    ms = rng.integers(0, M, SAMPLES)
    ns = rng.integers(0, N, SAMPLES)
    ms[:4] = [0, 0, M - 1, M - 1]
    ns[:4] = [0, N - 1, 0, N - 1]
    ref = oracle.gemm_entries(layout, qa, sa, qb, sb, bgran, ms, ns)
    ref_abs = oracle.gemm_entries(layout, qa & 0x7F, np.abs(sa), qb & 0x7F, np.abs(sb), bgran, ms, ns)
    E = (2.0 ** -9 + (4 * ((K + 127) // 128) + 4) * 2.0 ** -23) * ref_abs
    h = host(C)
    got = bf16_to_f64(h[ms, ns]) if out == torch.bfloat16 else h[ms, ns].astype(np.float64)
    tol = E + 2.0 ** -8 * (np.abs(ref) + E) if out == torch.bfloat16 else E
    bad = np.flatnonzero(np.abs(got - ref) > tol)
    assert bad.size == 0, ("entry", int(ms[bad[0]]), int(ns[bad[0]]), got[bad[0]], ref[bad[0]])
    if out == torch.float32:
        assert np.linalg.norm(got - ref) / np.linalg.norm(ref) <= 1e-3


@pytest.mark.parametrize("dp", ["native", "mx"])
def test_layer_grouped_fp8_datapaths_full_size(dev, dp):
    """The benchmark's side steps at full size: the gate/up forward product and the layer's
    seven weight gradients (K = 8,192) as grouped launches on the native-FP8 and on the MX
    datapath (MX with the power-of-two quantisers), sampled against the oracle."""
    T = synth.TOKENS
    p2 = dp == "mx"
    rule = {"rule": "pow2"} if p2 else {}
    kw = {"mx": p2, "native": not p2}
    shape = {g: (n, k, src) for g, n, k, src in synth.LAYER_GEMMS}
    host_q, dev_q = {}, {}

    def dual(name, x):
        d = pf.puro_fp8_quant_dual(to_dev(x), True, pow2=p2)
        r = oracle.quant_act(x, **rule) + oracle.quant_transpose(x, True, **rule)
        torch.cuda.synchronize()
        for t, ref, what in zip(d, r, ("q_row", "s_row", "q_tok", "s_tok")):
            _same(t, ref, (name, what))
        host_q[name], dev_q[name] = r, d

    for i, (name, c) in enumerate(synth.LAYER_INPUTS):
        dual(name, synth.normal((T, c), 1.0, synth.seed_of(4, 0, i), "bf16"))
    for j, (g, n, k, src) in enumerate(synth.LAYER_GEMMS):
        dual("dY_" + g, synth.normal((T, n), 1e-3, synth.seed_of(4, 0, 20 + j), "bf16"))
    seed = 50
    # forward gate and up on x_mlp, 128x128 weight scales
    Ws = {g: synth.normal((shape[g][0], shape[g][1]), 0.02, synth.seed_of(4, 0, 15 + i))
          for i, g in enumerate(("gate", "up"))}
    for g in ("gate", "up"):
        qw = pf.puro_fp8_quant_weight(to_dev(Ws[g]), pow2=p2)
        rw = oracle.quant_weight(Ws[g], **rule)
        torch.cuda.synchronize()
        _same(qw[0], rw[0], ("qW", g))
        _same(qw[1], rw[1], ("sW", g))
        host_q["W_" + g], dev_q["W_" + g] = rw, qw
    (hqx, hsx), (dqx, dsx) = host_q["x_mlp"][:2], dev_q["x_mlp"][:2]
    Ys = pf.puro_fp8_gemm_grouped("NT", [(dqx, dsx) + dev_q["W_" + g] for g in ("gate", "up")],
                                  out_dtype=torch.bfloat16, **kw)
    torch.cuda.synchronize()
    for g, Y in zip(("gate", "up"), Ys):
        seed += 1
        _check_sampled_mc("NT", "128x128", (hqx, hsx) + host_q["W_" + g], Y, shape[g][1], seed, torch.bfloat16)
    gs = [g for g, _, _, _ in synth.LAYER_GEMMS]
    dWs = pf.puro_fp8_gemm_grouped("NT", [dev_q["dY_" + g][2:] + dev_q[shape[g][2]][2:] for g in gs],
                                   bgran="1x128", out_dtype=torch.float32, **kw)
    torch.cuda.synchronize()
    for g, dW in zip(gs, dWs):
        seed += 1
        _check_sampled_mc("NT", "1x128", host_q["dY_" + g][2:] + host_q[shape[g][2]][2:], dW, T, seed,
                          torch.float32)
