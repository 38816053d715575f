"""Seeded synthetic inputs for the blockwise-FP8 linear-layer workloads.

This module draws random tensors and nothing else: it holds no quantisation,
scaling or GEMM arithmetic.  Both the CPU oracle's tests and the GPU path's
tests, the smoke check and the benchmark take their inputs from here.

Two generators, one recipe:

* host (numpy): a counter-based stream.  Element i of a tensor with seed S is
  built from splitmix64 outputs z(S, 2j) and z(S, 2j+1), j = i // 2, mapped to
  53-bit uniforms u1, u2 in [0, 1); Box-Muller in FP64 gives
  r = sqrt(-2 ln(1 - u1)), normals r cos(2 pi u2) (even i) and r sin(2 pi u2)
  (odd i); then multiply by sigma, round to FP32 (round-to-nearest-even) and,
  for BF16 tensors, round once more to BF16 (round-to-nearest-even).
  splitmix64 (Steele, Lea and Flood, 2014): state_i = S + (i + 1) * 0x9E3779B97F4A7C15;
  z = (x ^ (x >> 30)) * 0xBF58476D1CE4E5B9; z = (z ^ (z >> 27)) * 0x94D049BB133111EB;
  out = z ^ (z >> 31) (all mod 2^64).
* device (torch, for the full-size benchmark stack whose inputs are tens of
  GB): torch's seeded Philox generator on the GPU, same distributions, same
  FP32 -> BF16 rounding.  Values differ from the host stream for equal seeds.

Seeds: seed = 1_000_003 * config + 1_009 * layer + tensor_id.

BF16 tensors on the host are numpy uint16 arrays of raw BF16 bit patterns.

Workload shapes are those of the Puro-2B-Base model card's property table
(Qwen3-1.7B configuration: hidden 2,048, 28 layers, 16 attention / 8 KV heads,
FFN 6,144) and its training-setup paragraph (sequence length 4,096 and
micro-batch 2, so 8,192 tokens per micro-batch).
"""
import math

import numpy as np

_GAMMA = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)
_CHUNK = 1 << 22

HIDDEN = 2048
FFN = 6144
LAYERS = 28
Q_HEADS, KV_HEADS = 16, 8
HEAD_DIM = HIDDEN // Q_HEADS          # 128 (derived)
TOKENS = 2 * 4096                     # micro-batch 2 x sequence 4,096

# The seven unfused projections of one layer: name -> (N_out, K_in, input name)
LAYER_GEMMS = [
    ("q", Q_HEADS * HEAD_DIM, HIDDEN, "x_attn"),
    ("k", KV_HEADS * HEAD_DIM, HIDDEN, "x_attn"),
    ("v", KV_HEADS * HEAD_DIM, HIDDEN, "x_attn"),
    ("o", HIDDEN, Q_HEADS * HEAD_DIM, "x_o"),
    ("gate", FFN, HIDDEN, "x_mlp"),
    ("up", FFN, HIDDEN, "x_mlp"),
    ("down", HIDDEN, FFN, "h"),
]
LAYER_INPUTS = [("x_attn", HIDDEN), ("x_o", Q_HEADS * HEAD_DIM), ("x_mlp", HIDDEN), ("h", FFN)]

# The fused four-GEMM view of the same layer (QKV, O, gate_up, down): (N_out, K_in)
FUSED_GEMMS = [("qkv", 4096, 2048), ("o", 2048, 2048), ("gate_up", 12288, 2048), ("down", 2048, 6144)]

# Projections that read the same input, in the order in which their weights' rows (and their
# outputs' and output gradients' columns) are stored side by side: (group, members, input)
PROJ_GROUPS = [("qkv", ("q", "k", "v"), "x_attn"), ("o", ("o",), "x_o"),
               ("gate_up", ("gate", "up"), "x_mlp"), ("down", ("down",), "h")]


def seed_of(config, layer=0, tensor_id=0):
    return 1_000_003 * config + 1_009 * layer + tensor_id


def _splitmix64(seed, start, count):
    with np.errstate(over="ignore"):
        idx = np.arange(start + 1, start + count + 1, dtype=np.uint64)
        x = np.uint64(seed & 0xFFFFFFFFFFFFFFFF) + idx * _GAMMA
        z = (x ^ (x >> np.uint64(30))) * _M1
        z = (z ^ (z >> np.uint64(27))) * _M2
        return z ^ (z >> np.uint64(31))


def normal_f64(n, seed):
    """n standard normals (float64) from the counter-based host stream."""
    out = np.empty(n, dtype=np.float64)
    pairs = (n + 1) // 2
    done = 0
    while done < pairs:
        cnt = min(_CHUNK, pairs - done)
        z = _splitmix64(seed, 2 * done, 2 * cnt)
        u1 = (z[0::2] >> np.uint64(11)).astype(np.float64) * 2.0 ** -53
        u2 = (z[1::2] >> np.uint64(11)).astype(np.float64) * 2.0 ** -53
        r = np.sqrt(-2.0 * np.log1p(-u1))
        t = 2.0 * math.pi * u2
        blk = np.empty(2 * cnt, dtype=np.float64)
        blk[0::2] = r * np.cos(t)
        blk[1::2] = r * np.sin(t)
        lo = 2 * done
        hi = min(n, lo + 2 * cnt)
        out[lo:hi] = blk[: hi - lo]
        done += cnt
    return out


def uniform_f64(n, seed):
    """n uniforms in [0, 1) (float64, 53-bit) from the host stream."""
    out = np.empty(n, dtype=np.float64)
    for lo in range(0, n, _CHUNK):
        cnt = min(_CHUNK, n - lo)
        out[lo:lo + cnt] = (_splitmix64(seed, lo, cnt) >> np.uint64(11)).astype(np.float64) * 2.0 ** -53
    return out


def f32_to_bf16_bits(x):
    """Round float32 values to BF16 (round-to-nearest-even); returns uint16 bit patterns."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def bf16_bits_to_f32(u):
    """Widen BF16 bit patterns (uint16) to float32 exactly."""
    return (np.asarray(u, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def normal(shape, std, seed, dtype="f32"):
    """Seeded N(0, std^2) tensor on the host: float32, or BF16 bits (uint16) for dtype='bf16'."""
    n = int(np.prod(shape))
    x = (normal_f64(n, seed) * std).astype(np.float32).reshape(shape)
    return f32_to_bf16_bits(x) if dtype == "bf16" else x


# --------------------------------------------------------------------------- outlier-stress recipe

def outlier_activations(tokens, channels, seed, frac_channels=0.01, factor=100.0, zero_frac=0.01):
    """BF16 N(0,1) activations with round(frac*channels) seeded channels scaled by `factor`,
    plus all-zero blocks: zero_frac of the 1x128 row segments and zero_frac of the
    128-token column segments."""
    x = (normal_f64(tokens * channels, seed) * 1.0).astype(np.float32).reshape(tokens, channels)
    n_out = int(round(frac_channels * channels))
    pick = np.argsort(uniform_f64(channels, seed + 7))[:n_out]
    x[:, pick] *= np.float32(factor)
    zero_blocks(x, seed + 11, zero_frac)
    return f32_to_bf16_bits(x), np.sort(pick)


def lognormal_gradients(tokens, channels, seed, mu=math.log(1e-6), sigma=2.0, zero_frac=0.01,
                        random_sign=False):
    """BF16 exp(N(mu, sigma^2)) gradients (positive unless random_sign), with zero blocks as above."""
    g = np.exp(mu + sigma * normal_f64(tokens * channels, seed)).astype(np.float32)
    g = g.reshape(tokens, channels)
    if random_sign:
        flip = uniform_f64(tokens * channels, seed + 3).reshape(tokens, channels) < 0.5
        g[flip] = -g[flip]
    zero_blocks(g, seed + 11, zero_frac)
    return f32_to_bf16_bits(g)


def zero_blocks(x, seed, frac):
    """Zero a seeded fraction of the 1x128 row segments and of the 128-row column segments (in place)."""
    rows, cols = x.shape
    rb, cb = rows // 128, cols // 128
    n_row_seg = rows * cb
    k = int(round(frac * n_row_seg))
    if k:
        sel = np.argsort(uniform_f64(n_row_seg, seed))[:k]
        for idx in sel:
            r, b = divmod(int(idx), cb)
            x[r, b * 128:(b + 1) * 128] = 0
    n_col_seg = rb * cols
    k = int(round(frac * n_col_seg))
    if k:
        sel = np.argsort(uniform_f64(n_col_seg, seed + 1))[:k]
        for idx in sel:
            b, c = divmod(int(idx), cols)
            x[b * 128:(b + 1) * 128, c] = 0
    return x


# --------------------------------------------------------------------------- device generator

def device_normal(shape, std, seed, dtype, device):
    """Seeded N(0, std^2) tensor generated on `device` with torch's Philox stream."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    x = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    if std != 1.0:
        x.mul_(std)
    return x.to(torch.bfloat16) if dtype == "bf16" else x


def _device_zero_blocks(x, gen, frac):
    """Device form of zero_blocks (seeded by `gen`): zero a fraction of the 1x128 row segments and
    of the 128-row column segments of x, in place."""
    import torch
    rows, cols = x.shape
    rb, cb = rows // 128, cols // 128
    lane = torch.arange(128, device=x.device)
    k = int(round(frac * rows * cb))
    if k:
        sel = torch.randperm(rows * cb, generator=gen, device=x.device)[:k]
        r, b = sel // cb, sel % cb
        x[r[:, None].expand(-1, 128).reshape(-1), (b[:, None] * 128 + lane).reshape(-1)] = 0
    k = int(round(frac * rb * cols))
    if k:
        sel = torch.randperm(rb * cols, generator=gen, device=x.device)[:k]
        b, c = sel // cols, sel % cols
        x[(b[:, None] * 128 + lane).reshape(-1), c[:, None].expand(-1, 128).reshape(-1)] = 0
    return x


def device_outlier_activations(tokens, channels, seed, device, frac_channels=0.01, factor=100.0,
                               zero_frac=0.01):
    """Device form of outlier_activations (torch's Philox stream; values differ from the host's)."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    x = torch.randn((tokens, channels), generator=g, device=device, dtype=torch.float32)
    pick = torch.randperm(channels, generator=g, device=device)[:int(round(frac_channels * channels))]
    x[:, pick] *= factor
    _device_zero_blocks(x, g, zero_frac)
    return x.to(torch.bfloat16)


def device_lognormal_gradients(tokens, channels, seed, device, mu=math.log(1e-6), sigma=2.0, zero_frac=0.01):
    """Device form of lognormal_gradients (positive; torch's Philox stream)."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    x = torch.randn((tokens, channels), generator=g, device=device, dtype=torch.float32)
    x.mul_(sigma).add_(mu).exp_()
    _device_zero_blocks(x, g, zero_frac)
    return x.to(torch.bfloat16)
