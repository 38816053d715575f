"""Benchmark: blockwise-FP8 linear-layer GEMMs of the Qwen3-1.7B stack on one MI355X.

One step = one micro-batch (2 x 4,096 = 8,192 tokens) through the linear
layers of all 28 Transformer layers: the seven unfused projections
(q, k, v, o, gate, up, down) in forward (Y = X W^T), data gradient
(dX = dY W) and weight gradient (dW = dY^T X), with every quantiser inside
the timed region: weights in 128x128 tiles (a layer's seven in one launch),
and each layer input X and each output gradient dY quantised both ways in one
read (1x128 along features for the forward / data-gradient GEMM, 128-token
blocks for the weight gradient).  The projections that read one input (q/k/v,
gate/up) keep their weight codes in adjacent rows and their outputs and output
gradients in adjacent columns, as fused QKV and gate/up projections do, so
their forward products are one GEMM and the data gradient of their input (the
sum of their products) is one GEMM over the concatenated K; a layer's seven
weight gradients share one grouped launch.  Shapes come from the
Puro-2B-Base model card (Qwen3-1.7B configuration: hidden 2,048, FFN 6,144,
16 / 8 heads, 28 layers; sequence length 4,096, micro-batch 2).

Inputs are seeded synthetic tensors already resident in HBM: activations
BF16 N(0,1), gradients BF16 N(0,1e-3), FP32 master weights N(0,0.02), fresh
per layer.  Output: one JSON line (see the end of main()).  Besides the step,
the gated activation fused into the dual quantiser (the down projection's
input formed from the gate/up product), other GEMM forms and the whole step on
the native-FP8 and scaled (MX) matrix-core variants are timed on their own and
reported under "side_kernels", as is the vendor library's plain BF16 GEMM on
the layer's shapes (the stock rate of the FP16-class datapath the FP32-exact
kernels run on); none is part of the step or of its FLOP rate.
After the timing, the oracle leg (skipped with --no-cpu-baseline) checks the
timed step's last layer -- every code and scale byte and sampled entries of
its 15 GEMM outputs -- against the CPU oracle ("parity"), times the oracle on a
sample of the workload ("cpu_baseline") and per configuration ("configs").

    python bench.py [--gpus 1] [--steps K] [--warmup W]
"""
import argparse
import ctypes
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "blockwise-FP8 GEMM TFLOP/s (fwd+dgrad+wgrad), Qwen3-1.7B shapes; % FP8 peak"
FP8_PEAK_TFLOPS = 5000.0       # MI355X dense FP8 MFMA (published)
F16_PEAK_TFLOPS = 2500.0       # MI355X dense FP16 MFMA (published): the rate of the FP32-exact datapath
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E (published)


def log(*a):
    print(*a, file=sys.stderr, flush=True)


class Plan:
    """Pre-marshalled C-ABI calls of one step (pointers fixed, buffers preallocated)."""

    def __init__(self):
        self.calls = []   # (fn, args, kind, name, flops, bytes)

    def add(self, fn, args, kind, name, flops=0.0, nbytes=0.0):
        self.calls.append((fn, args, kind, name, flops, nbytes))

    def run(self):
        for fn, args, _, _, _, _ in self.calls:
            st = fn(*args)
            if st:
                raise RuntimeError("C-ABI call failed with status %d" % st)


def build_stack_plan(pf, torch, dev, layers, tokens, stream_ptr, datapath="exact", resident=None):
    """Allocate the stack's inputs (seeded, on the GPU; or reuse `resident`, an earlier plan's) and
    outputs; return (plan, keepalive, buffers).

    datapath: "exact" -- the recipe on the FP32-exact GEMMs (the benchmarked step);
              "native" -- the same quantisers, GEMMs on the native FP8 matrix cores
                          (puro_fp8_gemm_grouped_native);
              "mx" -- power-of-two quantisers and the scaled matrix cores (puro_fp8_gemm_grouped_mx).
    Every datapath runs the same launches: per layer one grouped weight quantisation, 8 dual
    quantisations and 9 grouped GEMM calls.

    The projections that read one input (q/k/v; gate/up) keep their weights' codes in adjacent
    rows of one buffer and their outputs and output gradients in adjacent columns, as a fused
    QKV or gate/up projection stores them.  Their forward products are then one GEMM, their
    output gradients one dual-quantiser call, and the data gradient of their input, the sum of
    their products, one GEMM over the concatenated K.  The products, codes and scales are those
    of the separate projections: every 128-block boundary falls on a projection boundary."""
    import synth
    L = pf.lib()
    vp = ctypes.c_void_p
    keep = []
    plan = Plan()
    bf16, f32, u8 = torch.bfloat16, torch.float32, torch.uint8

    def P(t, off=0):
        return vp(t.data_ptr() + off)

    def nb(n):
        return (n + 127) // 128

    T = tokens
    shape = {g: (n, k, src) for g, n, k, src in synth.LAYER_GEMMS}
    inputs = dict(synth.LAYER_INPUTS)
    # per group: output width, input width, and each member's first row
    grp = {}
    for name, members, src in synth.PROJ_GROUPS:
        rows, r0 = {}, 0
        for g in members:
            rows[g] = r0
            r0 += shape[g][0]
        grp[name] = (r0, inputs[src], src, members, rows)

    # Per-layer work buffers, reused by every layer.
    qx = {x: torch.empty((T, c), dtype=u8, device=dev) for x, c in synth.LAYER_INPUTS}
    sx = {x: torch.empty((T, nb(c)), dtype=f32, device=dev) for x, c in synth.LAYER_INPUTS}
    qxt = {x: torch.empty((c, T), dtype=u8, device=dev) for x, c in synth.LAYER_INPUTS}
    sxt = {x: torch.empty((c, nb(T)), dtype=f32, device=dev) for x, c in synth.LAYER_INPUTS}
    qdy = {G: torch.empty((T, n), dtype=u8, device=dev) for G, (n, _, _, _, _) in grp.items()}
    sdy = {G: torch.empty((T, nb(n)), dtype=f32, device=dev) for G, (n, _, _, _, _) in grp.items()}
    qdyt = {G: torch.empty((n, T), dtype=u8, device=dev) for G, (n, _, _, _, _) in grp.items()}
    sdyt = {G: torch.empty((n, nb(T)), dtype=f32, device=dev) for G, (n, _, _, _, _) in grp.items()}
    qw = {G: torch.empty((n, k), dtype=u8, device=dev) for G, (n, k, _, _, _) in grp.items()}
    sw = {G: torch.empty((nb(n), nb(k)), dtype=f32, device=dev) for G, (n, k, _, _, _) in grp.items()}
    qwt = {G: torch.empty((k, n), dtype=u8, device=dev) for G, (n, k, _, _, _) in grp.items()}
    swt = {G: torch.empty((nb(k), nb(n)), dtype=f32, device=dev) for G, (n, k, _, _, _) in grp.items()}
    y = {G: torch.empty((T, n), dtype=bf16, device=dev) for G, (n, _, _, _, _) in grp.items()}
    dx = {x: torch.empty((T, c), dtype=bf16, device=dev) for x, c in synth.LAYER_INPUTS}
    dw = {g: torch.empty((n, k), dtype=f32, device=dev) for g, n, k, _ in synth.LAYER_GEMMS}
    keep += [qx, sx, qxt, sxt, qdy, sdy, qdyt, sdyt, qw, sw, qwt, swt, y, dx, dw]
    bufs = {"qx": qx, "sx": sx, "qxt": qxt, "sxt": sxt, "qdy": qdy, "sdy": sdy, "qdyt": qdyt, "sdyt": sdyt,
            "qw": qw, "sw": sw, "qwt": qwt, "swt": swt, "y": y, "dx": dx, "dw": dw, "rows": {}, "inputs": []}

    BF16, F32 = pf.PURO_BF16, pf.PURO_F32
    NT, NN = pf.LAYOUTS["NT"], pf.LAYOUTS["NN"]
    S1, S128 = pf.BGRAN["1x128"], pf.BGRAN["128x128"]

    grouped_fn = {"exact": L.puro_fp8_gemm_grouped, "native": L.puro_fp8_gemm_grouped_native,
                  "mx": L.puro_fp8_gemm_grouped_mx}[datapath]

    def grouped(layout, bgran, cdt, descs, name, flops):
        arr = (pf.GemmDesc * len(descs))(*descs)
        keep.append(arr)
        plan.add(grouped_fn, (layout, bgran, cdt, arr, len(descs), stream_ptr), "gemm", name, flops)

    quant_dual_fn = L.puro_fp8_quant_dual_pow2 if datapath == "mx" else L.puro_fp8_quant_dual
    quant_weight_fn = (L.puro_fp8_quant_weight_grouped_pow2 if datapath == "mx"
                       else L.puro_fp8_quant_weight_grouped)

    def dual(x, c, q, s, qt, st):
        plan.add(quant_dual_fn, (P(x), BF16, T, c, c, P(q), c, P(s), 1, P(qt), T, P(st), stream_ptr),
                 "quant_dual", "quant_dual", 0, T * c * (2 + 2 + 8 / 128))

    def fwd(G):
        n, k, src, _, _ = grp[G]
        return pf.gemm_desc(T, n, [(k, P(qx[src]), k, P(sx[src]), P(qw[G]), k, P(sw[G]))], P(y[G]), n)

    def dgrad(G):
        # dX of the group's input = sum over its projections of dY_g W_g: one K loop over
        # the adjacent output-gradient columns and weight rows, with the weights' codes
        # read from their transposed copy (NT: K-contiguous like the forward's operands)
        n, k, src, _, _ = grp[G]
        return pf.gemm_desc(T, k, [(n, P(qdy[G]), n, P(sdy[G]), P(qwt[G]), n, P(swt[G]))], P(dx[src]), k)

    def wgrad(g, G):
        n, k, src = shape[g]
        r0 = grp[G][4][g]
        return pf.gemm_desc(n, k, [(T, P(qdyt[G], r0 * T), T, P(sdyt[G], r0 * nb(T) * 4),
                                    P(qxt[src]), T, P(sxt[src]))], P(dw[g]), k)

    def fl(G):
        n, k = grp[G][0], grp[G][1]
        return 2.0 * T * n * k

    group_of = {g: G for G, (_, _, _, members, _) in grp.items() for g in members}
    for layer in range(layers):
        if resident is not None:
            xs, wts, dys = resident[layer]
        else:
            xs = {x: synth.device_normal((T, c), 1.0, synth.seed_of(4, layer, i), "bf16", dev)
                  for i, (x, c) in enumerate(synth.LAYER_INPUTS)}
            # FP32 master weights, those of one group in adjacent rows of one tensor
            wts = {G: torch.empty((n, k), dtype=f32, device=dev) for G, (n, k, _, _, _) in grp.items()}
            for j, (g, n, k, _) in enumerate(synth.LAYER_GEMMS):
                G = group_of[g]
                r0 = grp[G][4][g]
                wts[G][r0:r0 + n] = synth.device_normal((n, k), 0.02, synth.seed_of(4, layer, 10 + j), "f32", dev)
            dys = {G: synth.device_normal((T, grp[G][0]), 1e-3, synth.seed_of(4, layer, 30 + j), "bf16", dev)
                   for j, (G, _, _) in enumerate(synth.PROJ_GROUPS)}
        keep += [xs, wts, dys]
        bufs["inputs"].append((xs, wts, dys))
        # the layer's weights quantised in one grouped launch (128x128 tiles; the tiles of a
        # group's weights are those of each weight), each group's codes also transposed
        descs = [pf.QuantWeightDesc(P(wts[G]), n, k, k, P(qw[G]), k, P(sw[G]), P(qwt[G]), n, P(swt[G]))
                 for G, (n, k, _, _, _) in grp.items()]
        wd = (pf.QuantWeightDesc * len(descs))(*descs)
        keep.append(wd)
        plan.add(quant_weight_fn, (F32, wd, len(descs), stream_ptr),
                 "quant_weight", "quant_weight", 0,
                 sum(n * k * (4 + 2) + 2 * nb(n) * nb(k) * 4 for _, n, k, _ in synth.LAYER_GEMMS))
        # forward: each input quantised once both ways (the 128-token copy is kept for the
        # weight gradient), then its group's product
        for G, _, src in synth.PROJ_GROUPS:
            c = inputs[src]
            dual(xs[src], c, qx[src], sx[src], qxt[src], sxt[src])
            grouped(NT, S128, BF16, [fwd(G)], "gemm_fwd_NT_128x128_bf16", fl(G))
        # backward, from the last group to the first: the group's output gradient quantised
        # both ways in one read, then the data gradient of its input with the forward's
        # quantised weights; the seven weight gradients once all output gradients exist
        for G, _, _ in reversed(synth.PROJ_GROUPS):
            n = grp[G][0]
            dual(dys[G], n, qdy[G], sdy[G], qdyt[G], sdyt[G])
            grouped(NT, S128, BF16, [dgrad(G)], "gemm_dgrad_NT_128x128_bf16", fl(G))
        grouped(NT, S1, F32, [wgrad(g, group_of[g]) for g, _, _, _ in synth.LAYER_GEMMS],
                "gemm_wgrad_NT_1x128_f32", sum(2.0 * T * n * k for _, n, k, _ in synth.LAYER_GEMMS))
    bufs["rows"] = {g: grp[group_of[g]][4][g] for g, _, _, _ in synth.LAYER_GEMMS}
    return plan, keep, bufs


def oracle_check_of_timed_layer(torch, bufs, samples=3000):
    """Oracle leg, part one: the timed step's last layer, checked after the timing.

    The step reuses its work buffers from layer to layer, so after the timed steps they hold
    the last layer's codes, scales and products.  That layer's inputs (drawn on the GPU) are
    copied to the host; every code and scale byte of its quantisers is compared with the
    oracle's, and `samples` entries of each of its 15 GEMM outputs (4 forward products, 4
    data gradients, 7 weight gradients) with the oracle's FP64 products of the oracle's
    codes, within the per-element bound (KB + 4) 2^-23 C_abs (plus one BF16 rounding for
    BF16 outputs).  Returns the summary reported as "parity" in the JSON line."""
    import numpy as np
    import oracle
    import synth
    T = synth.TOKENS
    layer = len(bufs["inputs"]) - 1
    xs, wts, dys = bufs["inputs"][layer]

    def h(t):
        t = t.detach().cpu().contiguous()
        if t.dtype == torch.bfloat16:
            return t.view(torch.int16).numpy().view(np.uint16)
        return t.numpy()

    def same(got, ref):
        got, ref = np.asarray(got), np.asarray(ref)
        if got.dtype == np.float32:
            got, ref = got.view(np.uint32), ref.astype(np.float32).view(np.uint32)
        return int(got.size), int(np.count_nonzero(got != ref))

    nbytes = mism = 0

    def cmp(got, ref):
        nonlocal nbytes, mism
        n_, m_ = same(h(got), ref)
        nbytes += n_
        mism += m_

    ref = {}
    for src, _ in synth.LAYER_INPUTS:
        x = h(xs[src])
        qa, sa = oracle.quant_act(x)
        qt, st = oracle.quant_transpose(x, True)
        cmp(bufs["qx"][src], qa); cmp(bufs["sx"][src], sa)
        cmp(bufs["qxt"][src], qt); cmp(bufs["sxt"][src], st)
        ref["x", src] = (qa, sa, qt, st)
    for G, _, _ in synth.PROJ_GROUPS:
        dy = h(dys[G])
        qa, sa = oracle.quant_act(dy)
        qt, st = oracle.quant_transpose(dy, True)
        cmp(bufs["qdy"][G], qa); cmp(bufs["sdy"][G], sa)
        cmp(bufs["qdyt"][G], qt); cmp(bufs["sdyt"][G], st)
        qw, sw = oracle.quant_weight(h(wts[G]))
        cmp(bufs["qw"][G], qw); cmp(bufs["sw"][G], sw)
        cmp(bufs["qwt"][G], qw.T); cmp(bufs["swt"][G], sw.T)
        ref["dy", G] = (qa, sa, qt, st)
        ref["w", G] = (qw, sw)

    rng = np.random.default_rng(20261203)
    worst, checked, failed = 0.0, 0, 0
    worst_rel = {False: 0.0, True: 0.0}   # relative Frobenius error of the samples, FP32 / BF16 outputs

    def entries(layout, A, sA, B, sB, bgran, K, got_t, bf16_out):
        nonlocal worst, checked, failed
        M, N = got_t.shape
        ms, ns = rng.integers(0, M, samples), rng.integers(0, N, samples)
        ms[:4], ns[:4] = [0, 0, M - 1, M - 1], [0, N - 1, 0, N - 1]
        A, sA, B, sB = (np.ascontiguousarray(v) for v in (A, sA, B, sB))
        r = oracle.gemm_entries(layout, A, sA, B, sB, bgran, ms, ns)
        c_abs = oracle.gemm_entries(layout, A & 0x7F, np.abs(sA), B & 0x7F, np.abs(sB), bgran, ms, ns)
        E = (K // 128 + 4) * 2.0 ** -23 * c_abs
        g = h(got_t)[ms, ns]
        if bf16_out:
            g = (g.astype(np.uint32) << 16).view(np.float32)
            E = E + 2.0 ** -8 * (np.abs(r) + E)
        err = np.abs(g.astype(np.float64) - r)
        ratio = err / np.where(E > 0, E, np.inf)
        worst = max(worst, float(np.max(np.where(E > 0, ratio, np.where(err > 0, np.inf, 0.0)))))
        worst_rel[bf16_out] = max(worst_rel[bf16_out], float(np.linalg.norm(err) / max(np.linalg.norm(r), 1e-300)))
        checked += samples
        failed += int(np.count_nonzero(err > E))

    shape = {g: (n, k, src) for g, n, k, src in synth.LAYER_GEMMS}
    for G, members, src in synth.PROJ_GROUPS:
        qa, sa, _, _ = ref["x", src]
        qw, sw = ref["w", G]
        K_in = qa.shape[1]
        entries("NT", qa, sa, qw, sw, "128x128", K_in, bufs["y"][G], True)                 # forward
        qd, sd, _, _ = ref["dy", G]
        entries("NT", qd, sd, qw.T, sw.T, "128x128", qd.shape[1], bufs["dx"][src], True)    # data gradient
        for g in members:                                                                   # weight gradients
            n, k, _ = shape[g]
            r0 = bufs["rows"][g]
            _, _, qdt, sdt = ref["dy", G]
            _, _, qxt, sxt = ref["x", src]
            entries("NT", qdt[r0:r0 + n], sdt[r0:r0 + n], qxt, sxt, "1x128", T, bufs["dw"][g], False)
    ok = mism == 0 and failed == 0
    return {"layer": layer, "pass": bool(ok), "quantiser_bytes_compared": nbytes, "quantiser_mismatches": mism,
            "gemm_outputs": 15, "gemm_entries_checked": checked, "gemm_entries_over_bound": failed,
            "max_err_over_bound": round(worst, 4),
            "max_rel_frobenius_fp32_outputs": float("%.3g" % worst_rel[False]),
            "max_rel_frobenius_bf16_outputs": float("%.3g" % worst_rel[True])}


def step_side_figure(torch, plan, stream, steps, step_flops):
    """Time a variant of the step (2 warm-up steps, then `steps` steps, event-timed), then once
    more with an event between launches for its GEMM share."""
    for _ in range(2):
        plan.run()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    a.record(stream)
    for _ in range(steps):
        plan.run()
    b.record(stream)
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / steps
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(len(plan.calls) + 1)]
    evs[0].record(stream)
    for j, (fn, args, _, _, _, _) in enumerate(plan.calls):
        if fn(*args):
            raise RuntimeError("C-ABI call failed")
        evs[j + 1].record(stream)
    torch.cuda.synchronize()
    gemm_ms = sum(evs[j].elapsed_time(evs[j + 1]) for j, c in enumerate(plan.calls) if c[2] == "gemm")
    return {"ms_per_step": round(ms, 3), "TFLOP/s": round(step_flops / (ms * 1e-3) / 1e12, 1),
            "gemm_ms": round(gemm_ms, 3), "gemm_TFLOP/s": round(step_flops / (gemm_ms * 1e-3) / 1e12, 1),
            "launches": len(plan.calls)}


def swiglu_setup(pf, torch, dev, tokens, sp):
    """The gated activation fused into the dual quantiser at the down projection's input: h formed
    from the two halves of a resident BF16 [tokens][2 x 6144] gate/up product, not stored (a step
    needs only its codes).  Returns (fn, args, algorithmic bytes, buffers to keep alive).
    Algorithmic bytes per element: 2 x 2 read + 2 x 1 written + 2 scales per 128."""
    import synth
    F = 6144
    gu = synth.device_normal((tokens, 2 * F), 1.0, 9001, "bf16", dev)
    qr = torch.empty((tokens, F), dtype=torch.uint8, device=dev)
    sr = torch.empty((tokens, F // 128), dtype=torch.float32, device=dev)
    qt = torch.empty((F, tokens), dtype=torch.uint8, device=dev)
    st = torch.empty((F, tokens // 128), dtype=torch.float32, device=dev)
    fn = pf.lib().puro_fp8_swiglu_quant_dual
    args = (ctypes.c_void_p(gu.data_ptr()), 2 * F, ctypes.c_void_p(gu.data_ptr() + 2 * F), 2 * F, tokens, F,
            None, 0, ctypes.c_void_p(qr.data_ptr()), F, ctypes.c_void_p(sr.data_ptr()), 1,
            ctypes.c_void_p(qt.data_ptr()), tokens, ctypes.c_void_p(st.data_ptr()), sp)
    return fn, args, tokens * F * (4 + 2 + 8 / 128), (gu, qr, sr, qt, st)


def swiglu_side(pf, torch, dev, tokens, sp, reps):
    """swiglu_setup's launch timed on its own (it is not a quantiser of the step)."""
    fn, args, nbytes, keep = swiglu_setup(pf, torch, dev, tokens, sp)
    stream = torch.cuda.current_stream()
    for _ in range(3):
        if fn(*args):
            raise RuntimeError("puro_fp8_swiglu_quant_dual failed")
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    n = max(reps, 1) * 10
    torch.cuda.synchronize()
    a.record(stream)
    for _ in range(n):
        fn(*args)
    b.record(stream)
    torch.cuda.synchronize()
    us = a.elapsed_time(b) * 1e3 / n
    gbs = nbytes / (us * 1e-6) / 1e9
    log("  swiglu_quant_dual [%d x %d] (outside the step): %.1f us per call, %.0f GB/s"
        % (tokens, args[5], us, gbs))
    return {"shape": [tokens, args[5]], "avg_us": round(us, 2), "bytes": int(nbytes), "GB/s": round(gbs, 1),
            "hbm_frac": round(gbs / HBM_PEAK_GBS, 4)}


def config_runs(pf, torch, dev, sp):
    """The per-layer configurations of the workload table as lists of single C-ABI calls.

    1 single fwd   X [256,512], W [256,512] FP32 N(0,1): quant_act, quant_weight, gemm NT (FP32 out)
    2 layer fwd    the fused four-GEMM layer (qkv, o, gate_up, down) at 8,192 tokens: quant_act of
                   X_g (BF16 N(0,1)), quant_weight of W_g (FP32 N(0,0.02)), gemm NT (BF16 out)
    3 layer bwd    dY_g BF16 N(0,1e-3): dual quantiser of dY_g (1x128 copy + 128-token copy),
                   quant_transpose of X_g, gemm NN (dX, BF16) and gemm NT (dW, FP32, K = 8,192);
                   W_g as quantised by config 2
    5 outlier      X [16384,6144] BF16 with 1% of channels x100, dY [16384,2048] BF16 lognormal
                   (exp N(ln 1e-6, 2)), both with 1% zero row and column segments, W [2048,6144]:
                   dual quantisers of X and dY, quant_weight, fwd NT, dgrad NN, wgrad NT
    Returns [(name, [(fn, args)], flops, buffers to keep alive)]."""
    import synth
    L = pf.lib()
    vp = ctypes.c_void_p
    bf16, f32, u8 = torch.bfloat16, torch.float32, torch.uint8
    BF16, F32 = pf.PURO_BF16, pf.PURO_F32
    NT, NN = pf.LAYOUTS["NT"], pf.LAYOUTS["NN"]
    S1, S128 = pf.BGRAN["1x128"], pf.BGRAN["128x128"]

    def P(t):
        return vp(t.data_ptr())

    def nb(n):
        return (n + 127) // 128

    def E(shape, dt):
        return torch.empty(shape, dtype=dt, device=dev)

    def gemm(layout, M, N, K, A, lda, sA, B, ldb, sB, bg, C, cdt, ldc, keep):
        ws_n = L.puro_fp8_gemm_workspace_size(layout, M, N, K, bg)
        ws = E((max(ws_n, 1),), u8)
        keep.append(ws)
        return (L.puro_fp8_gemm, (layout, M, N, K, P(A), lda, P(sA), P(B), ldb, P(sB), bg, P(C), cdt, ldc,
                                  P(ws), ws_n, sp))

    def qweight(w, n, k, q, s):
        return (L.puro_fp8_quant_weight, (P(w), F32, n, k, k, P(q), k, P(s), sp))

    def qdual(x, t, c, q, s, qt, st):
        return (L.puro_fp8_quant_dual, (P(x), BF16, t, c, c, P(q), c, P(s), 1, P(qt), t, P(st), sp))

    runs = []
    # config 1
    keep = []
    X = synth.device_normal((256, 512), 1.0, synth.seed_of(1, 0, 0), "f32", dev)
    W = synth.device_normal((256, 512), 1.0, synth.seed_of(1, 0, 1), "f32", dev)
    qx, sx, qw, sw, C = E((256, 512), u8), E((256, 4), f32), E((256, 512), u8), E((2, 4), f32), E((256, 256), f32)
    keep += [X, W, qx, sx, qw, sw, C]
    calls = [(L.puro_fp8_quant_act, (P(X), F32, 256, 512, 512, P(qx), 512, P(sx), sp)),
             qweight(W, 256, 512, qw, sw),
             gemm(NT, 256, 256, 512, qx, 512, sx, qw, 512, sw, S128, C, F32, 256, keep)]
    runs.append(("1_single_fwd", calls, 2.0 * 256 * 256 * 512, keep))

    # configs 2 and 3
    T = synth.TOKENS
    keep2, keep3, c2, c3, fl = [], [], [], [], 0.0
    for i, (g, n, k) in enumerate(synth.FUSED_GEMMS):
        X = synth.device_normal((T, k), 1.0, synth.seed_of(2, 0, i), "bf16", dev)
        W = synth.device_normal((n, k), 0.02, synth.seed_of(2, 0, 10 + i), "f32", dev)
        dY = synth.device_normal((T, n), 1e-3, synth.seed_of(3, 0, 20 + i), "bf16", dev)
        qx, sx = E((T, k), u8), E((T, nb(k)), f32)
        qxt, sxt = E((k, T), u8), E((k, nb(T)), f32)
        qw, sw = E((n, k), u8), E((nb(n), nb(k)), f32)
        Y = E((T, n), bf16)
        qdy, sdy, qdyt, sdyt = E((T, n), u8), E((T, nb(n)), f32), E((n, T), u8), E((n, nb(T)), f32)
        dX, dW = E((T, k), bf16), E((n, k), f32)
        keep2 += [X, W, qx, sx, qw, sw, Y]
        keep3 += [X, dY, qxt, sxt, qdy, sdy, qdyt, sdyt, dX, dW]
        c2 += [(L.puro_fp8_quant_act, (P(X), BF16, T, k, k, P(qx), k, P(sx), sp)),
               qweight(W, n, k, qw, sw),
               gemm(NT, T, n, k, qx, k, sx, qw, k, sw, S128, Y, BF16, n, keep2)]
        c3 += [qdual(dY, T, n, qdy, sdy, qdyt, sdyt),
               (L.puro_fp8_quant_transpose, (P(X), BF16, T, k, k, 1, P(qxt), T, P(sxt), sp)),
               gemm(NN, T, k, n, qdy, n, sdy, qw, k, sw, S128, dX, BF16, k, keep3),
               gemm(NT, n, k, T, qdyt, T, sdyt, qxt, T, sxt, S1, dW, F32, k, keep3)]
        fl += 2.0 * T * n * k
    runs.append(("2_layer_fwd", c2, fl, keep2))
    runs.append(("3_layer_bwd", c3, 2 * fl, keep3 + keep2))

    # config 5
    T5, N5, K5 = 16384, 2048, 6144
    X = synth.device_outlier_activations(T5, K5, synth.seed_of(5, 0, 0), dev)
    dY = synth.device_lognormal_gradients(T5, N5, synth.seed_of(5, 0, 1), dev)
    W = synth.device_normal((N5, K5), 0.02, synth.seed_of(5, 0, 2), "f32", dev)
    qx, sx, qxt, sxt = E((T5, K5), u8), E((T5, nb(K5)), f32), E((K5, T5), u8), E((K5, nb(T5)), f32)
    qdy, sdy, qdyt, sdyt = E((T5, N5), u8), E((T5, nb(N5)), f32), E((N5, T5), u8), E((N5, nb(T5)), f32)
    qw, sw = E((N5, K5), u8), E((nb(N5), nb(K5)), f32)
    Y, dX, dW = E((T5, N5), bf16), E((T5, K5), bf16), E((N5, K5), f32)
    keep = [X, dY, W, qx, sx, qxt, sxt, qdy, sdy, qdyt, sdyt, qw, sw, Y, dX, dW]
    c5 = [qdual(X, T5, K5, qx, sx, qxt, sxt), qweight(W, N5, K5, qw, sw),
          gemm(NT, T5, N5, K5, qx, K5, sx, qw, K5, sw, S128, Y, BF16, N5, keep),
          qdual(dY, T5, N5, qdy, sdy, qdyt, sdyt),
          gemm(NN, T5, K5, N5, qdy, N5, sdy, qw, K5, sw, S128, dX, BF16, K5, keep),
          gemm(NT, N5, K5, T5, qdyt, T5, sdyt, qxt, T5, sxt, S1, dW, F32, K5, keep)]
    runs.append(("5_outlier_stress", c5, 3 * 2.0 * T5 * N5 * K5, keep))
    return runs


def measure_configs(pf, torch, dev, sp, reps=20, warmup=5):
    """Median time of each configuration's calls over `reps` repetitions, hot (back to back) and
    cold (a 512 MiB buffer written before each repetition, outside the timed interval, to evict
    the last-level cache).  Event-timed on the launch stream."""
    stream = torch.cuda.current_stream()
    flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    out = {}
    for name, calls, flops, keep in config_runs(pf, torch, dev, sp):
        def once():
            for fn, a in calls:
                st = fn(*a)
                if st:
                    raise RuntimeError("%s: status %d" % (name, st))
        for _ in range(warmup):
            once()
        res = {}
        for mode in ("hot", "cold"):
            ts = []
            for _ in range(reps):
                if mode == "cold":
                    flush.fill_(1)
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record(stream)
                once()
                b.record(stream)
                b.synchronize()
                ts.append(a.elapsed_time(b) * 1e3)
            ts.sort()
            med = ts[len(ts) // 2]
            res[mode + "_us"] = round(med, 2)
            res[mode + "_tflops"] = round(flops / (med * 1e-6) / 1e12, 1)
        res["gflop"] = round(flops / 1e9, 3)
        log("  config %-18s %10.3f GFLOP  hot %9.1f us (%6.1f TFLOP/s)  cold %9.1f us (%6.1f TFLOP/s)"
            % (name, flops / 1e9, res["hot_us"], res["hot_tflops"], res["cold_us"], res["cold_tflops"]))
        out[name] = res
        del keep
    return out


def _timed(torch, fn, args, reps):
    """Average event-timed microseconds of fn(*args) on the current stream (3 warm-up calls)."""
    stream = torch.cuda.current_stream()
    for _ in range(3):
        if fn(*args):
            raise RuntimeError("C-ABI call failed")
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    a.record(stream)
    for _ in range(reps):
        fn(*args)
    b.record(stream)
    torch.cuda.synchronize()
    return a.elapsed_time(b) * 1e3 / reps


def gemm_side(pf, torch, dev, tokens, sp, reps):
    """GEMM forms outside the step, on the gate/up projections of one layer:
    segment_sum_accumulate: the data gradient of x_mlp as the sum of two K segments held in
        separate tensors (dY_gate W_gate + dY_up W_up, NN on the forward's codes), added into an
        existing BF16 output (C += sum: gradient accumulation over micro-batches);
    tn_wgrad: the gate projection's weight gradient (6,144 x 2,048, K = 8,192 tokens) in TN form, on
        untransposed 128-token copies of dY and X;
    mx_forward: the forward gate/up product (N = 12,288) with power-of-two block scales on the
        scaled FP8 matrix cores."""
    import synth
    L = pf.lib()
    vp = ctypes.c_void_p
    T, F, H = tokens, 6144, 2048
    out = {}
    # K-segment sum with accumulate-into
    dys = [synth.device_normal((T, F), 1e-3, 9201 + i, "bf16", dev) for i in range(2)]
    ws = [synth.device_normal((F, H), 0.02, 9203 + i, "f32", dev) for i in range(2)]
    qd = [pf.puro_fp8_quant_act(d) for d in dys]
    qw = [pf.puro_fp8_quant_weight(w) for w in ws]
    C = torch.zeros((T, H), dtype=torch.bfloat16, device=dev)
    segs = [(F, vp(q.data_ptr()), F, vp(sq.data_ptr()), vp(w.data_ptr()), H, vp(sw_.data_ptr()))
            for (q, sq), (w, sw_) in zip(qd, qw)]
    desc = (pf.GemmDesc * 1)(pf.gemm_desc(T, H, segs, vp(C.data_ptr()), H, accumulate=True))
    args = (pf.LAYOUTS["NN"], pf.BGRAN["128x128"], pf.PURO_BF16, desc, 1, sp)
    us = _timed(torch, L.puro_fp8_gemm_grouped, args, max(reps, 1) * 5)
    fl = 2.0 * T * H * 2 * F
    out["segment_sum_accumulate"] = {"shape": [T, H, 2 * F], "segments": 2, "avg_us": round(us, 2),
                                     "TFLOP/s": round(fl / (us * 1e-6) / 1e12, 1)}
    log("  segment sum + accumulate [%d x %d, K = 2 x %d] (outside the step): %.1f us, %.0f TFLOP/s"
        % (T, H, F, us, fl / (us * 1e-6) / 1e12))
    # weight gradient in TN form, on untransposed 128-token copies (dW_gate = dY_gate^T X)
    qdt, sdt = pf.puro_fp8_quant_transpose(dys[0], transpose_out=False)
    Xg = synth.device_normal((T, H), 1.0, 9207, "bf16", dev)
    qxt, sxt = pf.puro_fp8_quant_transpose(Xg, transpose_out=False)
    dW = torch.empty((F, H), dtype=torch.float32, device=dev)
    need = L.puro_fp8_gemm_workspace_size(pf.LAYOUTS["TN"], F, H, T, pf.BGRAN["1x128"])
    wst = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    args = (pf.LAYOUTS["TN"], F, H, T, vp(qdt.data_ptr()), F, vp(sdt.data_ptr()), vp(qxt.data_ptr()), H,
            vp(sxt.data_ptr()), pf.BGRAN["1x128"], vp(dW.data_ptr()), pf.PURO_F32, H, vp(wst.data_ptr()), need, sp)
    us = _timed(torch, L.puro_fp8_gemm, args, max(reps, 1) * 5)
    fl = 2.0 * F * H * T
    out["tn_wgrad"] = {"shape": [F, H, T], "avg_us": round(us, 2), "TFLOP/s": round(fl / (us * 1e-6) / 1e12, 1)}
    log("  TN weight gradient [%d x %d, K = %d] (outside the step): %.1f us, %.0f TFLOP/s"
        % (F, H, T, us, fl / (us * 1e-6) / 1e12))
    # power-of-two scales on the scaled matrix cores
    X = synth.device_normal((T, H), 1.0, 9205, "bf16", dev)
    W = synth.device_normal((2 * F, H), 0.02, 9206, "f32", dev)
    qx, sx = pf.puro_fp8_quant_act(X, pow2=True)
    qw2, sw2 = pf.puro_fp8_quant_weight(W, pow2=True)
    Y = torch.empty((T, 2 * F), dtype=torch.bfloat16, device=dev)
    need = L.puro_fp8_gemm_mx_workspace_size(pf.LAYOUTS["NT"], T, 2 * F, H, pf.BGRAN["128x128"])
    wsb = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    args = (pf.LAYOUTS["NT"], T, 2 * F, H, vp(qx.data_ptr()), H, vp(sx.data_ptr()), vp(qw2.data_ptr()), H,
            vp(sw2.data_ptr()), pf.BGRAN["128x128"], vp(Y.data_ptr()), pf.PURO_BF16, 2 * F, vp(wsb.data_ptr()),
            need, sp)
    us = _timed(torch, L.puro_fp8_gemm_mx, args, max(reps, 1) * 5)
    fl = 2.0 * T * 2 * F * H
    out["mx_forward"] = {"shape": [T, 2 * F, H], "avg_us": round(us, 2), "TFLOP/s": round(fl / (us * 1e-6) / 1e12, 1),
                         "frac_fp8_peak": round(fl / (us * 1e-6) / 1e12 / FP8_PEAK_TFLOPS, 4)}
    log("  MX forward [%d x %d x %d] (outside the step): %.1f us, %.0f TFLOP/s"
        % (T, 2 * F, H, us, fl / (us * 1e-6) / 1e12))
    return out


def vendor_bf16_side(torch, dev, tokens, reps):
    """The same layer's 15 products (the forward and data-gradient GEMMs of the four fused
    projections, the seven weight gradients) as plain BF16 GEMMs through torch.mm (the vendor
    library), on E4M3-valued operands, BF16 out: no block scales, no widening, no promotion.
    It runs on the same FP16-class matrix-core datapath as the FP32-exact kernels and gives the
    rate a stock GEMM of that width reaches on these shapes on this GPU (context only)."""
    import synth
    T = tokens
    probs = {"fwd": [(T, n, k) for _, n, k in synth.FUSED_GEMMS],
             "dgrad": [(T, k, n) for _, n, k in synth.FUSED_GEMMS],
             "wgrad": [(n, k, T) for _, n, k, _ in synth.LAYER_GEMMS]}
    gen = torch.Generator(device=dev)
    gen.manual_seed(9301)

    def e4m3_valued(r, c):
        x = (torch.randn((r, c), device=dev, generator=gen) * 128.0).clamp_(-448.0, 448.0)
        return x.to(torch.float8_e4m3fn).to(torch.bfloat16).contiguous()

    out, tot_ms, tot_fl = {}, 0.0, 0.0
    for kind, lst in probs.items():
        k_ms, k_fl = 0.0, 0.0
        for M, N, K in lst:
            A, B = e4m3_valued(M, K), e4m3_valued(K, N)
            C = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
            for _ in range(3):
                torch.mm(A, B, out=C)
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            n = max(reps, 1) * 2
            torch.cuda.synchronize()
            a.record()
            for _ in range(n):
                torch.mm(A, B, out=C)
            b.record()
            torch.cuda.synchronize()
            k_ms += a.elapsed_time(b) / n
            k_fl += 2.0 * M * N * K
            del A, B, C
        out[kind] = round(k_fl / (k_ms * 1e-3) / 1e12, 1)
        tot_ms += k_ms
        tot_fl += k_fl
    torch.cuda.empty_cache()
    res = {"what": "torch.mm BF16 x BF16 -> BF16 on E4M3-valued operands, the layer's 15 products",
           "ms_per_layer": round(tot_ms, 3), "TFLOP/s": round(tot_fl / (tot_ms * 1e-3) / 1e12, 1),
           "TFLOP/s_by_kind": out}
    log("  vendor BF16 GEMM on the layer's shapes (context, outside the step): %.3f ms/layer, %.0f TFLOP/s "
        "(fwd %.0f, dgrad %.0f, wgrad %.0f)" % (tot_ms, res["TFLOP/s"], out["fwd"], out["dgrad"], out["wgrad"]))
    return res


def cpu_baseline(rows):
    """Time the oracle on a bounded sample of one layer of the same workload."""
    import numpy as np
    import oracle
    import synth
    T = synth.TOKENS
    rng_layer = 0
    t_total = 0.0
    flops = 0.0
    for j, (g, n, k, src) in enumerate(synth.LAYER_GEMMS):
        x = synth.normal((rows, k), 1.0, synth.seed_of(4, rng_layer, 100 + j), "bf16")
        w = synth.normal((n, k), 0.02, synth.seed_of(4, rng_layer, 110 + j))
        dy = synth.normal((rows, n), 1e-3, synth.seed_of(4, rng_layer, 120 + j), "bf16")
        xt = synth.normal((T, k), 1.0, synth.seed_of(4, rng_layer, 130 + j), "bf16")
        dyt = synth.normal((T, rows), 1e-3, synth.seed_of(4, rng_layer, 140 + j), "bf16")
        t0 = time.perf_counter()
        qa, sa = oracle.quant_act(x)
        qw, sw = oracle.quant_weight(w)
        oracle.gemm("NT", qa, sa, qw, sw, "128x128")                   # rows x n x k
        qd, sd = oracle.quant_act(dy)
        oracle.gemm("NN", qd, sd, qw, sw, "128x128")                   # rows x k x n
        qdt, sdt = oracle.quant_transpose(dyt, True)
        qxt, sxt = oracle.quant_transpose(xt, True)
        oracle.gemm("NT", qdt, sdt, qxt, sxt, "1x128")                 # rows x k x T
        t_total += time.perf_counter() - t0
        flops += 2.0 * rows * n * k * 2 + 2.0 * rows * k * T
    return {"value": flops / t_total / 1e12, "unit": "TFLOP/s", "cores": oracle.num_threads(),
            "kind": "oracle",
            "sample": "one layer, %d rows of each of its 21 GEMMs (fwd/dgrad: %d of 8192 tokens; "
                      "wgrad: %d output rows, K=8192) with their quantisers; %.1f GFLOP in %.1f s"
                      % (rows, rows, rows, flops / 1e9, t_total)}


def oracle_configs(rows=32):
    """Oracle leg, per configuration of the workload table: the oracle's quantisers (GB/s over
    their algorithmic bytes) and blockwise GEMMs (GFLOP/s, FP64) timed on a stated sample of
    that configuration's inputs, with the thread count used.  Config 1 runs whole; the others
    quantise and multiply `rows` rows of each operand that carries the tokens (and the whole
    weights), and for their weight gradients `rows` x 256 outputs over all tokens."""
    import numpy as np
    import oracle
    import synth
    T = synth.TOKENS
    out = {}

    def timed(fn):
        t0 = time.perf_counter()
        fn()
        return time.perf_counter() - t0

    def entry(q_bytes, q_s, flops, g_s, sample):
        return {"quant_GB/s": round(q_bytes / q_s / 1e9, 3), "gemm_GFLOP/s": round(flops / g_s / 1e9, 3),
                "threads": oracle.num_threads(), "sample": sample}

    # config 1, whole
    X = synth.normal((256, 512), 1.0, synth.seed_of(1, 0, 0))
    W = synth.normal((256, 512), 1.0, synth.seed_of(1, 0, 1))
    r = {}
    q_s = timed(lambda: r.update(a=oracle.quant_act(X), w=oracle.quant_weight(W)))
    g_s = timed(lambda: oracle.gemm("NT", *r["a"], *r["w"], "128x128"))
    out["1_single_fwd"] = entry(2 * 256 * 512 * (4 + 1) + 256 * 4 * 4 + 8 * 4, q_s, 2.0 * 256 * 256 * 512, g_s,
                                "whole configuration")
    # configs 2 and 3: the fused four-GEMM layer
    q2 = g2 = q3 = g3 = 0.0
    qb2 = fl2 = qb3 = fl3 = 0.0
    for i, (g, n, k) in enumerate(synth.FUSED_GEMMS):
        X = synth.normal((rows, k), 1.0, synth.seed_of(2, 0, i), "bf16")
        W = synth.normal((n, k), 0.02, synth.seed_of(2, 0, 10 + i))
        dY = synth.normal((128, n), 1e-3, synth.seed_of(3, 0, 20 + i), "bf16")
        Xt = synth.normal((T, 256), 1.0, synth.seed_of(3, 0, 30 + i), "bf16")
        dYt = synth.normal((T, rows), 1e-3, synth.seed_of(3, 0, 40 + i), "bf16")
        q2 += timed(lambda: r.update(a=oracle.quant_act(X), w=oracle.quant_weight(W)))
        qb2 += rows * k * (2 + 1 + 4 / 128) + n * k * 5
        g2 += timed(lambda: oracle.gemm("NT", *r["a"], *r["w"], "128x128"))
        fl2 += 2.0 * rows * n * k
        q3 += timed(lambda: r.update(d=oracle.quant_act(dY), dt=oracle.quant_transpose(dY, True),
                                     xt=oracle.quant_transpose(Xt, True), yt=oracle.quant_transpose(dYt, True)))
        qb3 += 128 * n * (2 + 2 + 8 / 128) + (T * 256 + T * rows) * (2 + 1 + 4 / 128)
        g3 += timed(lambda: oracle.gemm("NN", r["d"][0][:rows], r["d"][1][:rows], *r["w"], "128x128"))
        g3 += timed(lambda: oracle.gemm("NT", *r["yt"], *r["xt"], "1x128"))
        fl3 += 2.0 * rows * k * n + 2.0 * rows * 256 * T
    out["2_layer_fwd"] = entry(qb2, q2, fl2, g2, "%d of 8,192 token rows per GEMM, whole weights" % rows)
    out["3_layer_bwd"] = entry(qb3, q3, fl3, g3, "dgrad: %d token rows (a 128-token block quantised); wgrad: "
                                                 "%d x 256 outputs over all 8,192 tokens" % (rows, rows))
    # config 5
    T5, N5, K5 = 16384, 2048, 6144
    X, _ = synth.outlier_activations(128, K5, synth.seed_of(5, 0, 0))
    dY = synth.lognormal_gradients(128, N5, synth.seed_of(5, 0, 1))
    W = synth.normal((N5, K5), 0.02, synth.seed_of(5, 0, 2))
    Xt, _ = synth.outlier_activations(T5, 128, synth.seed_of(5, 0, 3))
    dYt = synth.lognormal_gradients(T5, 128, synth.seed_of(5, 0, 4))
    q5 = timed(lambda: r.update(a=oracle.quant_act(X), w=oracle.quant_weight(W), d=oracle.quant_act(dY),
                                xt=oracle.quant_transpose(Xt, True), yt=oracle.quant_transpose(dYt, True)))
    qb5 = 128 * (K5 + N5) * (2 + 1 + 4 / 128) + N5 * K5 * 5 + 2 * T5 * 128 * (2 + 1 + 4 / 128)
    g5 = timed(lambda: oracle.gemm("NT", r["a"][0][:rows], r["a"][1][:rows], *r["w"], "128x128"))
    g5 += timed(lambda: oracle.gemm("NN", r["d"][0][:rows], r["d"][1][:rows], *r["w"], "128x128"))
    g5 += timed(lambda: oracle.gemm("NT", r["yt"][0][:rows], r["yt"][1][:rows], *r["xt"], "1x128"))
    fl5 = 2.0 * rows * N5 * K5 * 2 + 2.0 * rows * 128 * T5
    out["5_outlier_stress"] = entry(qb5, q5, fl5, g5, "%d token rows (fwd, dgrad) and %d output rows x 128 "
                                                      "channels over all 16,384 tokens (wgrad); 128-row blocks "
                                                      "quantised" % (rows, rows))
    return out


# Measured HBM traffic per launch of each GEMM kind (rocprofv3 FETCH_SIZE and
# WRITE_SIZE, scaled by the same counters on a plain copy of known size).  It
# holds only for the kernel source it was measured on, identified by hash.
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gemm_hbm_traffic.md")
KERNEL_SOURCES = [os.path.join(ROOT, "blockwise_fp8_gemm_amd", "csrc", f) for f in ("gemm.hip", "common.h")]


def kernel_source_hash():
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic(name):
    """HBM bytes per launch of kind `name` from TRAFFIC_FILE, or None when the
    file is missing, has no row for it, or was measured on other kernel source."""
    import re
    try:
        text = open(TRAFFIC_FILE).read()
    except OSError:
        return None
    m = re.search(r"kernel source sha256: ([0-9a-f]{64})", text)
    if not m or m.group(1) != kernel_source_hash():
        return None
    m = re.search(r"^\| `%s` \|[^\n]*\| ([0-9.eE+]+) \|\s*$" % re.escape(name), text, flags=re.M)
    return float(m.group(1)) if m else None


def traffic_probe():
    """One layer of the step three times, then the same layer on the native-FP8 and on the
    scaled (MX) datapaths three times each, the fused activation + dual quantiser three times,
    then a plain 1 GiB copy three times (the calibration for the memory counters); run under
    rocprofv3 --pmc."""
    import torch
    import blockwise_fp8_gemm_amd as pf
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    sp = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    import synth
    plan, keep, bufs = build_stack_plan(pf, torch, dev, 1, synth.TOKENS, sp)
    for _ in range(3):
        plan.run()
    for dp in ("native", "mx"):
        plan_d, keep_d, _ = build_stack_plan(pf, torch, dev, 1, synth.TOKENS, sp, datapath=dp,
                                             resident=bufs["inputs"])
        for _ in range(3):
            plan_d.run()
        torch.cuda.synchronize()
        del plan_d, keep_d
    fn, args, _, keep_sw = swiglu_setup(pf, torch, dev, synth.TOKENS, sp)
    for _ in range(3):
        if fn(*args):
            raise RuntimeError("puro_fp8_swiglu_quant_dual failed")
    src = torch.empty(1 << 30, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print("traffic probe done: 1 layer x 3 on each of the exact, native and mx datapaths, the fused "
          "activation x 3, then copy of %d bytes x 3" % src.numel(), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--layers", type=int, default=28, help=argparse.SUPPRESS)
    ap.add_argument("--cpu-rows", type=int, default=16, help="rows per GEMM in the oracle sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the per-configuration timings (configs 1, 2, 3, 5 of the workload table)")
    ap.add_argument("--traffic-probe", action="store_true",
                    help="run one layer and a calibration copy for the memory counters, then exit")
    args = ap.parse_args()
    if args.traffic_probe:
        traffic_probe()
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch
    import blockwise_fp8_gemm_amd as pf
    import synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()
    sp = ctypes.c_void_p(stream.cuda_stream)
    tokens = synth.TOKENS

    t0 = time.time()
    plan, keep, bufs = build_stack_plan(pf, torch, dev, args.layers, tokens, sp)
    torch.cuda.synchronize()
    log("inputs resident: %d layers, %.1f GB allocated, %d launches per step (%.1fs)"
        % (args.layers, torch.cuda.memory_allocated() / 1e9, len(plan.calls), time.time() - t0))
    step_flops = sum(c[4] for c in plan.calls)

    for i in range(args.warmup):
        plan.run()
    torch.cuda.synchronize()
    log("warmup done")

    # Timed region: K whole steps, nothing else on the stream.
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record(stream)
    for i in range(args.steps):
        plan.run()
    stop.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = start.elapsed_time(stop) / args.steps
    log("timed: %.3f ms/step (event), %.3f ms/step (wall)" % (ms_per_step, wall * 1e3 / args.steps))

    # Per-kernel durations: the same K steps again with an event between consecutive launches.
    nlaunch = len(plan.calls)
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(nlaunch + 1)]
    per_kind = {}
    per_name = {}
    for i in range(args.steps):
        evs[0].record(stream)
        for j, (fn, a, kind, name, fl, nbyt) in enumerate(plan.calls):
            st = fn(*a)
            if st:
                raise RuntimeError("status %d" % st)
            evs[j + 1].record(stream)
        torch.cuda.synchronize()
        for j, (fn, a, kind, name, fl, nbyt) in enumerate(plan.calls):
            ms = evs[j].elapsed_time(evs[j + 1])
            k = per_kind.setdefault(kind, [0.0, 0.0, 0.0, 0])
            k[0] += ms; k[1] += fl; k[2] += nbyt; k[3] += 1
            n_ = per_name.setdefault(name, [0.0, 0.0, 0.0, 0])
            n_[0] += ms; n_[1] += fl; n_[2] += nbyt; n_[3] += 1
    for k, v in sorted(per_kind.items(), key=lambda kv: -kv[1][0]):
        log("  %-16s %8.3f ms/step  %s" % (k, v[0] / args.steps,
            ("%.0f TFLOP/s" % (v[1] / v[0] / 1e9)) if v[1] else ("%.0f GB/s" % (v[2] / v[0] / 1e6))))
    for k, v in sorted(per_name.items(), key=lambda kv: -kv[1][0]):
        log("  %-28s %8.3f ms/step  calls %d  avg %.1f us  %s" % (
            k, v[0] / args.steps, v[3] // args.steps, v[0] / v[3] * 1e3,
            ("%.0f TFLOP/s" % (v[1] / v[0] / 1e9)) if v[1] else ("%.0f GB/s" % (v[2] / v[0] / 1e6))))

    # Oracle leg, part one (skipped with --no-cpu-baseline): the timed run's own outputs
    parity = None
    if not args.no_cpu_baseline:
        torch.cuda.synchronize()
        log("checking the timed step's last layer against the oracle ...")
        t1 = time.time()
        parity = oracle_check_of_timed_layer(torch, bufs)
        log("  parity of layer %d: %s (%d quantiser bytes, %d mismatches; %d GEMM entries, %d over the bound, "
            "max err/bound %.3f) in %.1fs" % (parity["layer"], "pass" if parity["pass"] else "FAIL",
                                               parity["quantiser_bytes_compared"], parity["quantiser_mismatches"],
                                               parity["gemm_entries_checked"], parity["gemm_entries_over_bound"],
                                               parity["max_err_over_bound"], time.time() - t1))
    inputs = bufs["inputs"]
    del bufs
    del plan, keep
    torch.cuda.empty_cache()

    # The same step (same resident inputs) on the two FP8-matrix-core variants, as side
    # figures: the native FP8 partials with the recipe's scales, and the power-of-two
    # quantisers with the scaled (MX) matrix cores.  Neither is the benchmarked step.
    side_steps = {}
    for dp in ("native", "mx"):
        plan_d, keep_d, _ = build_stack_plan(pf, torch, dev, args.layers, tokens, sp, datapath=dp,
                                             resident=inputs)
        side_steps[dp] = step_side_figure(torch, plan_d, stream, max(3, args.steps // 2), step_flops)
        log("  %s step (outside the benchmarked step): %.3f ms/step, %.0f TFLOP/s (GEMMs %.3f ms, %.0f TFLOP/s)"
            % (dp, side_steps[dp]["ms_per_step"], side_steps[dp]["TFLOP/s"], side_steps[dp]["gemm_ms"],
               side_steps[dp]["gemm_TFLOP/s"]))
        del plan_d, keep_d
        torch.cuda.empty_cache()
    del inputs
    torch.cuda.empty_cache()

    side = {"swiglu_quant_dual": swiglu_side(pf, torch, dev, tokens, sp, args.steps)}
    side.update(gemm_side(pf, torch, dev, tokens, sp, args.steps))
    side["steps"] = side_steps
    side["vendor_bf16_gemm"] = vendor_bf16_side(torch, dev, tokens, args.steps)
    configs = measure_configs(pf, torch, dev, sp) if not args.no_configs else None

    dom_name, dom = max(per_name.items(), key=lambda kv: kv[1][0])
    gemm_ms = per_kind["gemm"][0] / args.steps
    if dom[1] > 0:
        achieved = dom[1] / dom[0] / 1e9            # TFLOP/s
        roofline = {"bound": "mfma", "achieved": round(achieved, 1), "peak": FP8_PEAK_TFLOPS,
                    "unit": "TFLOP/s", "frac": round(achieved / FP8_PEAK_TFLOPS, 4),
                    "traffic": measured_traffic(dom_name),
                    "kernel": dom_name, "avg_launch_us": round(dom[0] / dom[3] * 1e3, 2),
                    # the E4M3 codes are widened exactly to FP16 for the matrix cores (the
                    # FP8 matrix cores' in-run fixed-point sums miss the precision bound),
                    # so the datapath's own ceiling is the FP16 rate
                    "datapath": "e4m3 widened to f16 MFMA, fp32 accumulate",
                    "frac_of_datapath_peak": round(achieved / F16_PEAK_TFLOPS, 4)}
    else:
        achieved = dom[2] / dom[0] / 1e6            # GB/s
        roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                    "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None,
                    "kernel": dom_name, "avg_launch_us": round(dom[0] / dom[3] * 1e3, 2)}

    value = step_flops / (ms_per_step * 1e-3) / 1e12
    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8_e4m3",
        "data": "synthetic",
        "config": {"workload": "Qwen3-1.7B linear stack, %d layers x 7 projections, fwd+dgrad+wgrad, "
                               "%d tokens (2x4096), quantisers included" % (args.layers, tokens),
                   "layers": args.layers, "tokens": tokens, "gemms_per_step": 21 * args.layers,
                   "tflop_per_step": round(step_flops / 1e12, 3)},
        "pct_fp8_peak": round(100.0 * value / FP8_PEAK_TFLOPS, 2),
        "gemm_only_tflops": round(step_flops / (gemm_ms * 1e-3) / 1e12, 1),
        "breakdown_ms": {k: round(v[0] / args.steps, 3) for k, v in per_kind.items()},
        "roofline": roofline,
        "side_kernels": side,
        "configs": configs,
        "parity": parity,
    }
    if configs:
        for name, res in configs.items():
            res["pct_fp8_peak"] = round(100.0 * res["hot_tflops"] / FP8_PEAK_TFLOPS, 2)
    if not args.no_cpu_baseline:
        log("timing the oracle on a CPU sample ...")
        out["cpu_baseline"] = cpu_baseline(args.cpu_rows)
        if configs:
            log("timing the oracle per configuration on samples ...")
            for name, res in oracle_configs().items():
                configs[name]["oracle"] = res
                log("  config %-18s oracle: quantisers %.3f GB/s, GEMM %.3f GFLOP/s (%d threads; %s)"
                    % (name, res["quant_GB/s"], res["gemm_GFLOP/s"], res["threads"], res["sample"]))
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
