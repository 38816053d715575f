"""Explicit launch streams in the Python binding.

When a call is given a stream other than the current one, the tensors the
binding allocates (outputs and the split-K workspace) must belong to that
stream: PyTorch's caching allocator then reuses their memory only for later
work on that stream, after the kernels.  Allocated on the current stream, the
workspace could be handed to other work while the split-K kernels still write
it.
"""
import numpy as np
import pytest
import torch

import blockwise_fp8_gemm_amd as pf
import synth
from helpers import host, to_dev

pytestmark = pytest.mark.gpu


def _operands(dev, M, N, K, seed):
    X = to_dev(synth.normal((M, K), 1.0, seed, "bf16"), dev)
    W = to_dev(synth.normal((N, K), 0.02, seed + 1), dev)
    qx, sx = pf.puro_fp8_quant_act(X)
    qw, sw = pf.puro_fp8_quant_weight(W)
    return qx, sx, qw, sw


def test_outputs_belong_to_the_launch_stream(dev):
    # a product the plan splits over K, so that a workspace is allocated too
    M, N, K = 256, 256, 8192
    assert pf.puro_fp8_gemm_workspace_size("NT", M, N, K, "128x128") > 0
    qx, sx, qw, sw = _operands(dev, M, N, K, 501)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    C = pf.puro_fp8_gemm("NT", qx, sx, qw, sw, bgran="128x128", out_dtype=torch.float32, stream=side)
    ptr, nbytes = C.data_ptr(), C.numel() * C.element_size()
    side.synchronize()
    del C
    # a block freed on the side stream is not handed to the current stream ...
    other = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    assert other.data_ptr() != ptr
    # ... but is to the side stream
    with torch.cuda.stream(side):
        again = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    assert again.data_ptr() == ptr
    # a raw stream handle behaves the same
    q, s = pf.puro_fp8_quant_act(to_dev(synth.normal((128, 256), 1.0, 502, "bf16"), dev),
                                 stream=side.cuda_stream)
    qptr = q.data_ptr()
    side.synchronize()
    del q, s
    with torch.cuda.stream(side):
        assert torch.empty(128 * 256, dtype=torch.uint8, device=dev).data_ptr() == qptr
    torch.cuda.synchronize()


def test_split_k_results_on_a_side_stream_while_the_current_stream_allocates(dev):
    M, N, K = 256, 256, 8192
    qx, sx, qw, sw = _operands(dev, M, N, K, 503)
    want = host(pf.puro_fp8_gemm("NT", qx, sx, qw, sw, bgran="128x128", out_dtype=torch.float32))
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    need = pf.puro_fp8_gemm_workspace_size("NT", M, N, K, "128x128")
    outs = []
    for _ in range(20):
        outs.append(pf.puro_fp8_gemm("NT", qx, sx, qw, sw, bgran="128x128", out_dtype=torch.float32,
                                     stream=side))
        # the current stream takes and scribbles over blocks of the workspace's size meanwhile
        junk = torch.empty(need, dtype=torch.uint8, device=dev)
        junk.fill_(0xFF)
        del junk
    side.synchronize()
    torch.cuda.synchronize()
    for C in outs:
        assert np.array_equal(host(C).view(np.uint32), want.view(np.uint32))
