"""CPU oracle for blockwise E4M3 FP8 quantise-and-GEMM (numpy front end).

TEST INFRASTRUCTURE ONLY.  Only tests/, the smoke check in __graft_entry__ and
the CPU-baseline leg of bench.py may import this package.  It shares no code
with the HIP library and never calls it.

The arithmetic lives in puro_ref.c; this module only marshals numpy arrays.
BF16 tensors are passed as numpy uint16 arrays holding the raw BF16 bit
patterns; FP32 tensors as float32 arrays.

What is computed (each function below restates it):
  * E4M3 codec -- the E4M3 format of the FP8-formats paper (Micikevicius et
    al., 2022) that the Puro-2B report's related-work paragraph cites.
  * Blockwise quantisation -- per block: s = fl32(amax / 448), codes
    q = E4M3_RNE_sat(fl32(x / s)); zero blocks give s = 0 and signed zeros.
  * Blockwise GEMM -- C = sum over 128-wide K blocks of sA*sB*(exact block dot
    product), in FP64.
The model card's setup paragraph (Puro-2B-Base, under the Phase 1 / Phase 2
table) is the source for "blockwise E4M3 for the main linear-layer GEMMs,
BF16/FP32 elsewhere"; block shapes and the scale rule are readings, not
statements of the pages.
"""
import ctypes
import os

import numpy as np

from . import build as _build

_LIB = None

LAYOUTS = {"NT": 0, "NN": 1, "TN": 2}
BGRAN = {"1x128": 0, "128x128": 1}

_i64 = ctypes.c_int64
_p = ctypes.c_void_p


def _lib():
    global _LIB
    if _LIB is None:
        if not os.path.exists(_build.LIB):
            _build.build()
        lib = ctypes.CDLL(_build.LIB)
        lib.ref_e4m3_decode.restype = ctypes.c_double
        lib.ref_e4m3_decode.argtypes = [ctypes.c_uint8]
        lib.ref_e4m3_encode.restype = ctypes.c_uint8
        lib.ref_e4m3_encode.argtypes = [ctypes.c_float]
        lib.ref_e4m3_encode_array.argtypes = [_p, _i64, _p]
        lib.ref_e4m3_decode_array.argtypes = [_p, _i64, _p]
        for name in ("ref_quant_act_rule", "ref_quant_weight_rule"):
            f = getattr(lib, name)
            f.restype = ctypes.c_int
            f.argtypes = [_p, ctypes.c_int, _i64, _i64, _i64, _p, _i64, _p, ctypes.c_int]
        lib.ref_quant_transpose_rule.restype = ctypes.c_int
        lib.ref_quant_transpose_rule.argtypes = [_p, ctypes.c_int, _i64, _i64, _i64, ctypes.c_int,
                                                 _p, _i64, _p, ctypes.c_int]
        for name in ("ref_gemm", "ref_gemm_brute"):
            f = getattr(lib, name)
            f.restype = ctypes.c_int
            f.argtypes = [ctypes.c_int, _i64, _i64, _i64, _p, _i64, _p, _p, _i64, _p,
                          ctypes.c_int, _p, _i64]
        lib.ref_gemm_entries.restype = ctypes.c_int
        lib.ref_gemm_entries.argtypes = [ctypes.c_int, _i64, _i64, _i64, _p, _i64, _p, _p, _i64,
                                         _p, ctypes.c_int, _p, _p, _i64, _p]
        lib.ref_bf16_rne.restype = ctypes.c_uint16
        lib.ref_bf16_rne.argtypes = [ctypes.c_double]
        lib.ref_bf16_rne_array.argtypes = [_p, _i64, _p]
        lib.ref_swiglu.restype = ctypes.c_double
        lib.ref_swiglu.argtypes = [ctypes.c_double, ctypes.c_double]
        lib.ref_swiglu_array.argtypes = [_p, _p, _i64, _p]
        lib.ref_num_threads.restype = ctypes.c_int
        _LIB = lib
    return _LIB


def _ptr(a):
    return a.ctypes.data_as(ctypes.c_void_p)


def _nblk(n):
    return (n + 127) // 128


def _dtype_code(x):
    if x.dtype == np.float32:
        return 0
    if x.dtype == np.uint16:
        return 1
    raise TypeError("oracle inputs are float32 or uint16 (BF16 bit patterns), got %s" % x.dtype)


def _check(st, what):
    if st != 0:
        raise ValueError("%s: oracle rejected the arguments (status %d)" % (what, st))


def num_threads():
    """Threads the oracle's OpenMP loops use."""
    return int(_lib().ref_num_threads())


# --------------------------------------------------------------------------- E4M3 codec

def e4m3_decode(codes):
    """Exact value of each E4M3 code (NaN for 0x7F / 0xFF), as float64."""
    c = np.ascontiguousarray(codes, dtype=np.uint8)
    out = np.empty(c.shape, dtype=np.float64)
    _lib().ref_e4m3_decode_array(_ptr(c), c.size, _ptr(out))
    return out


def e4m3_encode(values):
    """Nearest E4M3 code to each float32 value, ties to even, saturating at 448."""
    y = np.ascontiguousarray(values, dtype=np.float32)
    out = np.empty(y.shape, dtype=np.uint8)
    _lib().ref_e4m3_encode_array(_ptr(y), y.size, _ptr(out))
    return out


# --------------------------------------------------------------------------- quantisers

RULES = {"amax": 0, "pow2": 1}


def quant_act(x, rule="amax"):
    """1x128 blocks along each row of x[rows][cols] -> (q uint8 [rows][cols], s f32 [rows][ceil(cols/128)]).

    rule "amax": s = fl32(amax / 448) (the recipe); "pow2": s = the smallest power of two
    with 448 s >= amax, in [2^-127, 2^127] (the scaled matrix cores' E8M0 scales)."""
    x = np.ascontiguousarray(x)
    rows, cols = x.shape
    q = np.empty((rows, cols), dtype=np.uint8)
    s = np.empty((rows, _nblk(cols)), dtype=np.float32)
    _check(_lib().ref_quant_act_rule(_ptr(x), _dtype_code(x), rows, cols, cols, _ptr(q), cols, _ptr(s),
                                     RULES[rule]), "quant_act")
    return q, s


def quant_weight(w, rule="amax"):
    """128x128 tiles of w[rows][cols] -> (q uint8 [rows][cols], s f32 [ceil(rows/128)][ceil(cols/128)])."""
    w = np.ascontiguousarray(w)
    rows, cols = w.shape
    q = np.empty((rows, cols), dtype=np.uint8)
    s = np.empty((_nblk(rows), _nblk(cols)), dtype=np.float32)
    _check(_lib().ref_quant_weight_rule(_ptr(w), _dtype_code(w), rows, cols, cols, _ptr(q), cols, _ptr(s),
                                        RULES[rule]), "quant_weight")
    return q, s


def quant_transpose(x, transpose_out=True, rule="amax"):
    """Blocks of 128 consecutive tokens per column of x[tokens][cols].

    transpose_out=True : q [cols][tokens], s [cols][ceil(tokens/128)]
    transpose_out=False: q [tokens][cols], s [ceil(tokens/128)][cols]
    """
    x = np.ascontiguousarray(x)
    tokens, cols = x.shape
    if transpose_out:
        q = np.empty((cols, tokens), dtype=np.uint8)
        s = np.empty((cols, _nblk(tokens)), dtype=np.float32)
        ldq = tokens
    else:
        q = np.empty((tokens, cols), dtype=np.uint8)
        s = np.empty((_nblk(tokens), cols), dtype=np.float32)
        ldq = cols
    _check(_lib().ref_quant_transpose_rule(_ptr(x), _dtype_code(x), tokens, cols, cols,
                                           1 if transpose_out else 0, _ptr(q), ldq, _ptr(s), RULES[rule]),
           "quant_transpose")
    return q, s


# --------------------------------------------------------------------------- GEMM

def _gemm_dims(layout, A, B):
    if layout == "NT":
        (M, K), (N, K2) = A.shape, B.shape
    elif layout == "NN":
        (M, K), (K2, N) = A.shape, B.shape
    elif layout == "TN":
        (K, M), (K2, N) = A.shape, B.shape
    else:
        raise ValueError(layout)
    if K != K2:
        raise ValueError("contraction extents differ: %d vs %d" % (K, K2))
    return M, N, K


def _gemm_args(layout, A, sA, B, sB, bgran):
    A = np.ascontiguousarray(A, dtype=np.uint8)
    B = np.ascontiguousarray(B, dtype=np.uint8)
    sA = np.ascontiguousarray(sA, dtype=np.float32)
    sB = np.ascontiguousarray(sB, dtype=np.float32)
    M, N, K = _gemm_dims(layout, A, B)
    return A, sA, B, sB, M, N, K, LAYOUTS[layout], BGRAN[bgran]


def gemm(layout, A, sA, B, sB, bgran="128x128"):
    """Blockwise-scaled product C [M][N] in FP64 (see puro_ref.c for layouts)."""
    A, sA, B, sB, M, N, K, lay, bg = _gemm_args(layout, A, sA, B, sB, bgran)
    C = np.empty((M, N), dtype=np.float64)
    _check(_lib().ref_gemm(lay, M, N, K, _ptr(A), A.shape[1], _ptr(sA), _ptr(B), B.shape[1],
                           _ptr(sB), bg, _ptr(C), N), "gemm")
    return C


def gemm_entries(layout, A, sA, B, sB, bgran, ms, ns):
    """C[ms[i]][ns[i]] only, in FP64."""
    A, sA, B, sB, M, N, K, lay, bg = _gemm_args(layout, A, sA, B, sB, bgran)
    ms = np.ascontiguousarray(ms, dtype=np.int64)
    ns = np.ascontiguousarray(ns, dtype=np.int64)
    out = np.empty(ms.shape, dtype=np.float64)
    _check(_lib().ref_gemm_entries(lay, M, N, K, _ptr(A), A.shape[1], _ptr(sA), _ptr(B),
                                   B.shape[1], _ptr(sB), bg, _ptr(ms), _ptr(ns), ms.size,
                                   _ptr(out)), "gemm_entries")
    return out


def gemm_brute(layout, A, sA, B, sB, bgran="128x128"):
    """Dequantise-then-matmul in FP64 with a textbook triple loop (tiny shapes only)."""
    A, sA, B, sB, M, N, K, lay, bg = _gemm_args(layout, A, sA, B, sB, bgran)
    C = np.empty((M, N), dtype=np.float64)
    _check(_lib().ref_gemm_brute(lay, M, N, K, _ptr(A), A.shape[1], _ptr(sA), _ptr(B),
                                 B.shape[1], _ptr(sB), bg, _ptr(C), N), "gemm_brute")
    return C


def gemm_segments(layout, segments, bgran="128x128", c_init=None):
    """C = c_init + sum over K segments of the blockwise product, in FP64.

    Each segment is (A, sA, B, sB) with its own K, blocked along its own K
    from its first index (the segments of one output share M and N).  This is
    the plain sum of the partial products that a linear layer's inputs
    receive from several projections (the data gradient of an input read by
    the q, k and v projections is dY_q W_q + dY_k W_k + dY_v W_v), and the
    accumulate-into output used to sum weight gradients over micro-batches."""
    out = None if c_init is None else np.array(c_init, dtype=np.float64)
    for A, sA, B, sB in segments:
        g = gemm(layout, A, sA, B, sB, bgran)
        out = g if out is None else out + g
    return out


def bf16_rne(values):
    """FP64 -> nearest BF16 bit pattern (uint16), ties to even."""
    v = np.ascontiguousarray(values, dtype=np.float64)
    out = np.empty(v.shape, dtype=np.uint16)
    _lib().ref_bf16_rne_array(_ptr(v), v.size, _ptr(out))
    return out


# --------------------------------------------------------------------------- gated activation

def _as_f64(x):
    x = np.asarray(x)
    if x.dtype == np.uint16:   # BF16 bit patterns
        return (x.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return x.astype(np.float64)


def swiglu(gate, up):
    """h = silu(gate) * up = gate * up / (1 + exp(-gate)) in FP64, elementwise.

    The gated feed-forward unit of the Qwen3-1.7B configuration that the model card's
    configuration table names (SwiGLU with Swish parameter 1; a reading, the pages do not
    state the activation).  gate and up are float arrays or BF16 bit patterns (uint16)."""
    g = np.ascontiguousarray(_as_f64(gate))
    u = np.ascontiguousarray(_as_f64(up))
    if g.shape != u.shape:
        raise ValueError("gate and up shapes differ: %s vs %s" % (g.shape, u.shape))
    out = np.empty(g.shape, dtype=np.float64)
    _lib().ref_swiglu_array(_ptr(g), _ptr(u), g.size, _ptr(out))
    return out


def swiglu_bf16(gate, up):
    """The BF16 activation tensor: swiglu() rounded once to the nearest BF16 (ties to even)."""
    return bf16_rne(swiglu(gate, up))
