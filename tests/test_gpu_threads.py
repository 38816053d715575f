"""Calls from several host threads at once, each on its own stream.

The library keeps no mutable host state (validation and launch planning work
on the call's arguments only), and the binding's foreign calls release the
interpreter lock, so four threads run quantise-and-GEMM sequences concurrently
on four streams.  Each thread's outputs must equal, byte for byte, those of the
same sequence run alone on the default stream.
"""
import threading

import pytest
import torch

import blockwise_fp8_gemm_amd as pf
import synth

pytestmark = pytest.mark.gpu

T, C, N = 1024, 512, 768


def _sequence(x, w, a_long, b_long):
    qx, sx, qxt, sxt = pf.puro_fp8_quant_dual(x)
    (qw, sw, qwt, swt), = pf.puro_fp8_quant_weight_grouped([w], transposed=True)
    y = pf.puro_fp8_gemm("NT", qx, sx, qw, sw, bgran="128x128", out_dtype=torch.bfloat16)
    # weight-gradient form: NT on the token-blocked copies, 1x128 B scales, split K
    qa, sa = pf.puro_fp8_quant_act(a_long)
    qb, sb = pf.puro_fp8_quant_act(b_long)
    ys = pf.puro_fp8_gemm("NT", qa, sa, qb, sb, bgran="1x128", out_dtype=torch.float32)
    return [qx, sx, qxt, sxt, qw, sw, qwt, swt, y, ys]


def _bytes(t):
    return t.contiguous().view(torch.uint8) if t.dtype != torch.uint8 else t.contiguous()


def test_concurrent_threads_match_serial(dev):
    nthreads, reps = 4, 5
    inputs = []
    for i in range(nthreads):
        inputs.append((synth.device_normal((T, C), 1.0, 9400 + 10 * i, "bf16", dev),
                       synth.device_normal((N, C), 0.02, 9401 + 10 * i, "f32", dev),
                       synth.device_normal((128, 4096), 1.0, 9402 + 10 * i, "bf16", dev),
                       synth.device_normal((256, 4096), 1.0, 9403 + 10 * i, "bf16", dev)))
    serial = []
    for args in inputs:
        serial.append([o.clone() for o in _sequence(*args)])
    torch.cuda.synchronize()

    results = [[None] * reps for _ in range(nthreads)]
    errors = []
    start = threading.Barrier(nthreads)

    def worker(i):
        try:
            s = torch.cuda.Stream()
            start.wait()
            with torch.cuda.stream(s):
                for r in range(reps):
                    results[i][r] = _sequence(*inputs[i])
            s.synchronize()
        except Exception as e:      # reported after the join
            errors.append((i, repr(e)))

    threads = [threading.Thread(target=worker, args=(i,)) for i in range(nthreads)]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    torch.cuda.synchronize()
    assert not errors, errors
    for i in range(nthreads):
        for r in range(reps):
            for k, (o, e) in enumerate(zip(results[i][r], serial[i])):
                assert torch.equal(_bytes(o), _bytes(e)), ("thread", i, "rep", r, "output", k)
