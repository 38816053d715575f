"""Host <-> device marshalling and comparison helpers for the GPU parity tests."""
import numpy as np
import torch


def to_dev(a, device="cuda:0", ld=None):
    """numpy float32 / uint16 (BF16 bits) / uint8 array -> 2-D device tensor.

    With ld, the tensor is a view with that row stride (padded rows)."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        t = torch.from_numpy(a.view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(a)
    if ld is None or ld == a.shape[1]:
        return t.to(device)
    rows, cols = a.shape
    buf = torch.full((rows, ld), 0, dtype=t.dtype, device=device)
    if t.dtype == torch.bfloat16:
        buf.view(torch.int16).fill_(0x7FC0)   # NaN padding: must never be read
    elif t.dtype == torch.float32:
        buf.fill_(float("nan"))
    else:
        buf.fill_(0x7F)                        # E4M3 NaN code
    view = buf[:, :cols]
    view.copy_(t.to(device))
    return view


def host(t):
    """Device tensor -> numpy (uint8, float32, or uint16 BF16 bits)."""
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return t.contiguous().view(torch.int16).numpy().view(np.uint16)
    return t.contiguous().numpy()


def bf16_to_f64(u16):
    return (np.asarray(u16, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def rel_frobenius(c_gpu, c_ref):
    c_gpu = np.asarray(c_gpu, np.float64)
    den = np.linalg.norm(c_ref)
    num = np.linalg.norm(c_gpu - c_ref)
    if den == 0:
        return 0.0 if num == 0 else np.inf
    return num / den


def bf16_ulp_diff(got_bits, ref_bits):
    """Per-element distance in BF16 ulps between two BF16 bit arrays (finite values)."""
    def ordered(u):
        u = np.asarray(u, np.uint16).astype(np.int64)
        return np.where(u & 0x8000, -(u & 0x7FFF), u)
    return np.abs(ordered(got_bits) - ordered(ref_bits))


def first_mismatch(a, b):
    idx = np.argwhere(np.asarray(a) != np.asarray(b))
    return None if idx.size == 0 else tuple(int(v) for v in idx[0])
