"""The library's launches recorded in a HIP graph and replayed.

A sequence like one layer's (dual quantiser, grouped weight quantiser with the
transposed copies, forward GEMM, a split-K GEMM through the caller's workspace,
a grouped GEMM of two K segments adding into an existing output, the fused
activation and the power-of-two GEMM on the scaled matrix cores) is run once
eagerly, then captured on a side stream into a graph.  The library records no
memset and allocates nothing, so every node is a kernel.  The graph is replayed
three times; before each replay the outputs are cleared and the accumulated
output is reset by eager work on the default stream, with synchronisations
between.  Every replay's outputs must equal the eager ones byte for byte (the
kernels are deterministic: fixed K order, fixed split-K reduction order).
"""
import pytest
import torch

import blockwise_fp8_gemm_amd as pf
import synth

pytestmark = pytest.mark.gpu

T, C, N1, N2, F = 1024, 768, 640, 256, 384


def _bytes(t):
    return t.contiguous().view(torch.uint8) if t.dtype != torch.uint8 else t.contiguous()


def test_graph_replay_matches_eager(dev):
    x = synth.device_normal((T, C), 1.0, 9301, "bf16", dev)
    w1 = synth.device_normal((N1, C), 0.02, 9302, "f32", dev)
    w2 = synth.device_normal((N2, C), 0.02, 9303, "f32", dev)
    gu = synth.device_normal((T, 2 * F), 1.0, 9304, "bf16", dev)
    gate, up = gu[:, :F], gu[:, F:]
    a_long = synth.device_normal((128, 4096), 1.0, 9305, "bf16", dev)
    b_long = synth.device_normal((128, 4096), 1.0, 9306, "bf16", dev)
    c0 = synth.device_normal((T, N1), 1.0, 9307, "f32", dev)
    x2 = synth.device_normal((T, 256), 1.0, 9308, "bf16", dev)
    w3 = synth.device_normal((N1, 256), 0.02, 9309, "f32", dev)

    # outputs, allocated once (eager first call)
    dx = pf.puro_fp8_quant_dual(x)
    wq = pf.puro_fp8_quant_weight_grouped([w1, w2], transposed=True)
    qa, sa = pf.puro_fp8_quant_act(a_long)
    qb, sb = pf.puro_fp8_quant_act(b_long)
    qx2, sx2 = pf.puro_fp8_quant_act(x2)
    qw3, sw3 = pf.puro_fp8_quant_weight(w3)
    px, psx = pf.puro_fp8_quant_act(x, pow2=True)
    pw, psw = pf.puro_fp8_quant_weight(w1, pow2=True)
    y = torch.empty((T, N1), dtype=torch.bfloat16, device=dev)
    ws_y = torch.empty(max(pf.puro_fp8_gemm_workspace_size("NT", T, N1, C, "128x128"), 256),
                       dtype=torch.uint8, device=dev)
    ys = torch.empty((128, 128), dtype=torch.float32, device=dev)
    ws = torch.empty(max(pf.puro_fp8_gemm_workspace_size("NT", 128, 128, 4096, "1x128"), 256),
                     dtype=torch.uint8, device=dev)
    acc = torch.empty((T, N1), dtype=torch.float32, device=dev)
    h = torch.empty((T, F), dtype=torch.bfloat16, device=dev)
    sw = pf.puro_fp8_swiglu_quant_dual(gate, up, h=h)[1:]
    ymx = torch.empty((T, N1), dtype=torch.bfloat16, device=dev)
    ws_mx = torch.empty(max(pf.puro_fp8_gemm_mx_workspace_size("NT", T, N1, C, "128x128"), 256),
                        dtype=torch.uint8, device=dev)

    def sequence():
        pf.puro_fp8_quant_dual(x, True, *dx)
        pf.puro_fp8_quant_weight_grouped([w1, w2], outs=wq, transposed=True)
        (q1, s1, _, _), (q2, s2, _, _) = wq
        pf.puro_fp8_gemm("NT", dx[0], dx[1], q1, s1, bgran="128x128", out_dtype=torch.bfloat16, C=y,
                         workspace=ws_y)
        pf.puro_fp8_gemm("NT", qa, sa, qb, sb, bgran="1x128", out_dtype=torch.float32, C=ys, workspace=ws)
        pf.puro_fp8_gemm_grouped("NT", [{"segments": [(dx[0], dx[1], q1, s1), (qx2, sx2, qw3, sw3)],
                                          "C": acc, "accumulate": True}],
                                 bgran="128x128", out_dtype=torch.float32)
        pf.puro_fp8_swiglu_quant_dual(gate, up, h=h, q_row=sw[0], s_row=sw[1], q_tok=sw[2], s_tok=sw[3])
        pf.puro_fp8_gemm("NT", px, psx, pw, psw, bgran="128x128", out_dtype=torch.bfloat16, C=ymx,
                         workspace=ws_mx, mx=True)

    outs = list(dx) + [t for o in wq for t in o] + [y, ys, acc, h] + list(sw) + [ymx]
    acc.copy_(c0)
    sequence()
    torch.cuda.synchronize()
    eager = [o.clone() for o in outs]
    assert torch.isfinite(eager[-1].float()).all() and torch.isfinite(acc).all()

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        sequence()
    torch.cuda.synchronize()

    for rep in range(3):
        for o in outs:
            o.zero_()
        acc.copy_(c0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, (o, e) in enumerate(zip(outs, eager)):
            assert torch.equal(_bytes(o), _bytes(e)), ("replay", rep, "output", i)
        # unrelated eager work between replays
        (torch.randn(256, 256, device=dev) @ torch.randn(256, 256, device=dev)).sum().item()
