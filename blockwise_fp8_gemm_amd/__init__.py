"""Python binding of libpuro_fp8 (blockwise E4M3 FP8 quantise-and-GEMM on gfx950).

Argument marshalling only: every step runs in the HIP kernels behind the
C-ABI declared in include/puro_fp8.h.  PyTorch supplies device memory and
the current stream.  There is no CPU fallback: without the built library
every call raises.

Names mirror the C entry points:
    puro_fp8_quant_act(x)                 -> (q, s)   1x128 blocks along rows
    puro_fp8_quant_weight(w)              -> (q, s)   128x128 tiles
    puro_fp8_quant_weight_grouped([w..])  -> [(q, s)..] several weights, one launch
    puro_fp8_quant_transpose(x, t_out)    -> (q, s)   128-token blocks per column
    puro_fp8_quant_dual(x, t_out)         -> both of the above from one read of x
    puro_fp8_swiglu_quant_dual(gate, up)  -> h = bf16(silu(gate) * up) and its dual quantisation
    puro_fp8_gemm(layout, A, sA, B, sB, bgran, out_dtype) -> C
    puro_fp8_gemm_workspace_size(layout, M, N, K, bgran)
    puro_fp8_gemm(..., mx=True)           -> puro_fp8_gemm_mx (power-of-two scales, scaled matrix cores)
    puro_fp8_gemm(..., native=True)       -> puro_fp8_gemm_native (partials on the FP8 matrix cores)
    puro_fp8_gemm_grouped(..., mx=True / native=True) -> the grouped forms of those two
    puro_status_string(status)
Tensors are 2-D, row-major (stride(1) == 1), with a row stride that is a
multiple of 16 elements and 16-byte aligned storage.
"""
import contextlib
import ctypes
import functools
import inspect
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libpuro_fp8.so")

PURO_OK = 0
PURO_F32, PURO_BF16 = 0, 1
LAYOUTS = {"NT": 0, "NN": 1, "TN": 2}
BGRAN = {"1x128": 0, "128x128": 1}

_lib = None


class PuroError(RuntimeError):
    def __init__(self, status, what):
        self.status = status
        super().__init__("%s failed: %s (status %d)" % (what, puro_status_string(status), status))


class GemmSegment(ctypes.Structure):
    """puro_gemm_segment_t: one K segment of a grouped-GEMM problem."""
    _fields_ = [("K", ctypes.c_int64), ("A", ctypes.c_void_p), ("lda", ctypes.c_int64), ("sA", ctypes.c_void_p),
                ("B", ctypes.c_void_p), ("ldb", ctypes.c_int64), ("sB", ctypes.c_void_p)]


MAX_SEGMENTS = 4


class GemmDesc(ctypes.Structure):
    """puro_gemm_desc_t: one problem of puro_fp8_gemm_grouped."""
    _fields_ = [("M", ctypes.c_int64), ("N", ctypes.c_int64), ("nseg", ctypes.c_int), ("accumulate", ctypes.c_int),
                ("seg", GemmSegment * MAX_SEGMENTS), ("C", ctypes.c_void_p), ("ldc", ctypes.c_int64)]


class QuantWeightDesc(ctypes.Structure):
    """puro_quant_weight_desc_t: one weight of puro_fp8_quant_weight_grouped."""
    _fields_ = [("w", ctypes.c_void_p), ("rows", ctypes.c_int64), ("cols", ctypes.c_int64), ("ldw", ctypes.c_int64),
                ("q", ctypes.c_void_p), ("ldq", ctypes.c_int64), ("s", ctypes.c_void_p),
                ("qt", ctypes.c_void_p), ("ldqt", ctypes.c_int64), ("st", ctypes.c_void_p)]


def gemm_desc(M, N, segments, C, ldc, accumulate=False):
    """GemmDesc from (K, A, lda, sA, B, ldb, sB) tuples of pointers and strides."""
    if not 1 <= len(segments) <= MAX_SEGMENTS:
        raise ValueError("1 to %d segments" % MAX_SEGMENTS)
    d = GemmDesc()
    d.M, d.N, d.nseg, d.accumulate, d.C, d.ldc = M, N, len(segments), int(bool(accumulate)), C, ldc
    for i, g in enumerate(segments):
        d.seg[i] = GemmSegment(*g)
    return d


def lib():
    """Load libpuro_fp8.so; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError("libpuro_fp8.so is not built (run blockwise_fp8_gemm_amd/build.py "
                              "or __graft_entry__.build())")
        L = ctypes.CDLL(LIB_PATH)
        i64, vp, i32 = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int
        for name in ("puro_fp8_quant_act", "puro_fp8_quant_weight", "puro_fp8_quant_act_pow2",
                     "puro_fp8_quant_weight_pow2"):
            f = getattr(L, name)
            f.restype = i32
            f.argtypes = [vp, i32, i64, i64, i64, vp, i64, vp, vp]
        for name in ("puro_fp8_quant_transpose", "puro_fp8_quant_transpose_pow2"):
            f = getattr(L, name)
            f.restype = i32
            f.argtypes = [vp, i32, i64, i64, i64, i32, vp, i64, vp, vp]
        for name in ("puro_fp8_quant_dual", "puro_fp8_quant_dual_pow2"):
            f = getattr(L, name)
            f.restype = i32
            f.argtypes = [vp, i32, i64, i64, i64, vp, i64, vp, i32, vp, i64, vp, vp]
        for name in ("puro_fp8_swiglu_quant_dual", "puro_fp8_swiglu_quant_dual_pow2"):
            f = getattr(L, name)
            f.restype = i32
            f.argtypes = [vp, i64, vp, i64, i64, i64, vp, i64, vp, i64, vp, i32, vp, i64, vp, vp]
        L.puro_fp8_gemm_workspace_size.restype = ctypes.c_size_t
        L.puro_fp8_gemm_workspace_size.argtypes = [i32, i64, i64, i64, i32]
        for name in ("puro_fp8_gemm", "puro_fp8_gemm_mx", "puro_fp8_gemm_native"):
            f = getattr(L, name)
            f.restype = i32
            f.argtypes = [i32, i64, i64, i64, vp, i64, vp, vp, i64, vp, i32, vp, i32, i64, vp, ctypes.c_size_t, vp]
        L.puro_fp8_gemm_noalloc.restype = i32
        L.puro_fp8_gemm_noalloc.argtypes = [i32, i64, i64, i64, vp, i64, vp, vp, i64, vp, i32, vp, i32, i64, vp]
        for name in ("puro_fp8_gemm_mx_workspace_size", "puro_fp8_gemm_native_workspace_size"):
            f = getattr(L, name)
            f.restype = ctypes.c_size_t
            f.argtypes = [i32, i64, i64, i64, i32]
        for name in ("puro_fp8_quant_weight_grouped", "puro_fp8_quant_weight_grouped_pow2"):
            f = getattr(L, name)
            f.restype = i32
            f.argtypes = [i32, ctypes.POINTER(QuantWeightDesc), i32, vp]
        for name in ("puro_fp8_gemm_grouped", "puro_fp8_gemm_grouped_mx", "puro_fp8_gemm_grouped_native"):
            f = getattr(L, name)
            f.restype = i32
            f.argtypes = [i32, i32, i32, ctypes.POINTER(GemmDesc), i32, vp]
        L.puro_status_string.restype = ctypes.c_char_p
        L.puro_status_string.argtypes = [i32]
        L.puro_fp8_version.restype = i32
        L.puro_fp8_version.argtypes = []
        _lib = L
    return _lib


def puro_status_string(status):
    return lib().puro_status_string(int(status)).decode()


def puro_fp8_version():
    return int(lib().puro_fp8_version())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _on(stream):
    """Context in which the wrappers allocate: the launch stream.

    Outputs and the split-K workspace allocated here belong to the stream the
    kernels run on, so PyTorch's caching allocator hands their memory to later
    work on that stream only after the kernels (stream order).  Allocating on
    another current stream would let that stream reuse the workspace while the
    kernels still write it."""
    if stream is None:
        return contextlib.nullcontext()
    if not isinstance(stream, torch.cuda.Stream):
        stream = torch.cuda.ExternalStream(int(stream))
    return torch.cuda.stream(stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr() if t is not None and t.numel() > 0 else 0)


def _ld(t):
    if t.dim() != 2:
        raise ValueError("expected a 2-D tensor, got shape %s" % (tuple(t.shape),))
    if t.shape[0] > 0 and t.shape[1] > 1 and t.stride(1) != 1:
        raise ValueError("expected unit stride along the last dimension")
    # with at most one row, or no elements, the stride never addresses memory
    if t.numel() == 0 or t.shape[0] <= 1:
        return _pad16(t.shape[1])
    return t.stride(0)


def _pad16(n):
    return (n + 15) // 16 * 16


def _dtype_code(t):
    if t.dtype == torch.float32:
        return PURO_F32
    if t.dtype == torch.bfloat16:
        return PURO_BF16
    raise TypeError("inputs are float32 or bfloat16, got %s" % t.dtype)


def _nblk(n):
    return (n + 127) // 128


def empty_2d(rows, cols, dtype, device):
    """Uninitialised [rows][cols] tensor whose row stride is a multiple of 16 elements."""
    ld = _pad16(cols)
    if ld == cols:
        return torch.empty((rows, cols), dtype=dtype, device=device)
    return torch.empty((rows, ld), dtype=dtype, device=device)[:, :cols]


def _check(status, what):
    if status != PURO_OK:
        raise PuroError(status, what)


def _need(t, shape, dtype, name):
    if tuple(t.shape) != tuple(shape) or t.dtype != dtype or not t.is_cuda:
        raise ValueError("%s: expected %s %s on the GPU, got %s %s" % (
            name, tuple(shape), dtype, tuple(t.shape), t.dtype))


def _stream_allocs(fn):
    """Runs the wrapper with its allocations on the launch stream (see _on)."""
    pos = list(inspect.signature(fn).parameters).index("stream")

    @functools.wraps(fn)
    def run(*args, **kw):
        stream = args[pos] if len(args) > pos else kw.get("stream")
        with _on(stream):
            return fn(*args, **kw)
    return run


def _need_dense(t, shape, name):
    _need(t, shape, torch.float32, name)
    if not t.is_contiguous():
        raise ValueError("%s: scale arrays must be dense (contiguous)" % name)


@_stream_allocs
def puro_fp8_quant_act(x, q=None, s=None, stream=None, pow2=False):
    """1x128 blocks along each row of x [rows][cols] (float32 / bfloat16).
    pow2: power-of-two block scales (puro_fp8_quant_act_pow2)."""
    rows, cols = x.shape
    if q is None:
        q = empty_2d(rows, cols, torch.uint8, x.device)
    if s is None:
        s = torch.empty((rows, _nblk(cols)), dtype=torch.float32, device=x.device)
    _need(q, (rows, cols), torch.uint8, "q")
    _need_dense(s, (rows, _nblk(cols)), "s")
    fn = lib().puro_fp8_quant_act_pow2 if pow2 else lib().puro_fp8_quant_act
    _check(fn(_ptr(x), _dtype_code(x), rows, cols, _ld(x), _ptr(q), _ld(q), _ptr(s), _stream(stream)),
           "puro_fp8_quant_act")
    return q, s


@_stream_allocs
def puro_fp8_quant_weight(w, q=None, s=None, stream=None, pow2=False):
    """128x128 tiles of w [rows][cols] (float32 / bfloat16); pow2: power-of-two scales."""
    rows, cols = w.shape
    if q is None:
        q = empty_2d(rows, cols, torch.uint8, w.device)
    if s is None:
        s = torch.empty((_nblk(rows), _nblk(cols)), dtype=torch.float32, device=w.device)
    _need(q, (rows, cols), torch.uint8, "q")
    _need_dense(s, (_nblk(rows), _nblk(cols)), "s")
    fn = lib().puro_fp8_quant_weight_pow2 if pow2 else lib().puro_fp8_quant_weight
    _check(fn(_ptr(w), _dtype_code(w), rows, cols, _ld(w), _ptr(q), _ld(q), _ptr(s), _stream(stream)),
           "puro_fp8_quant_weight")
    return q, s


@_stream_allocs
def puro_fp8_quant_weight_grouped(weights, outs=None, stream=None, pow2=False, transposed=False):
    """128x128 tiles of several weights (one dtype) in as few launches as possible.

    weights: list of 2-D tensors; outs: optional list of (q, s), or (q, s, qt, st) with
    transposed, to write into.  transposed: also write each weight's codes and scales
    transposed (qt [cols][rows], st [ceil(cols/128)][ceil(rows/128)]).
    Returns the list of (q, s), or of (q, s, qt, st) with transposed.
    """
    if outs is None:
        outs = [(None,) * (4 if transposed else 2)] * len(weights)
    if len(outs) != len(weights):
        raise ValueError("outs must have one entry per weight")
    if any(w.dtype != weights[0].dtype for w in weights):
        raise ValueError("all weights must share one dtype")
    res, descs = [], []
    for w, o in zip(weights, outs):
        rows, cols = w.shape
        q, s = o[0], o[1]
        if q is None:
            q = empty_2d(rows, cols, torch.uint8, w.device)
        if s is None:
            s = torch.empty((_nblk(rows), _nblk(cols)), dtype=torch.float32, device=w.device)
        _need(q, (rows, cols), torch.uint8, "q")
        _need_dense(s, (_nblk(rows), _nblk(cols)), "s")
        if transposed:
            qt, st = (o[2], o[3]) if len(o) == 4 else (None, None)
            if qt is None:
                qt = empty_2d(cols, rows, torch.uint8, w.device)
            if st is None:
                st = torch.empty((_nblk(cols), _nblk(rows)), dtype=torch.float32, device=w.device)
            _need(qt, (cols, rows), torch.uint8, "qt")
            _need_dense(st, (_nblk(cols), _nblk(rows)), "st")
            descs.append(QuantWeightDesc(_ptr(w), rows, cols, _ld(w), _ptr(q), _ld(q), _ptr(s),
                                         _ptr(qt), _ld(qt), _ptr(st)))
            res.append((q, s, qt, st))
        else:
            descs.append(QuantWeightDesc(_ptr(w), rows, cols, _ld(w), _ptr(q), _ld(q), _ptr(s), None, 0, None))
            res.append((q, s))
    if not descs:
        return res
    arr = (QuantWeightDesc * len(descs))(*descs)
    fn = lib().puro_fp8_quant_weight_grouped_pow2 if pow2 else lib().puro_fp8_quant_weight_grouped
    _check(fn(_dtype_code(weights[0]), arr, len(descs), _stream(stream)), "puro_fp8_quant_weight_grouped")
    return res


@_stream_allocs
def puro_fp8_quant_transpose(x, transpose_out=True, q=None, s=None, stream=None, pow2=False):
    """128-token blocks per column of x [tokens][cols].

    transpose_out=True : q [cols][tokens], s [cols][ceil(tokens/128)]
    transpose_out=False: q [tokens][cols], s [ceil(tokens/128)][cols]
    """
    tokens, cols = x.shape
    qshape = (cols, tokens) if transpose_out else (tokens, cols)
    sshape = (cols, _nblk(tokens)) if transpose_out else (_nblk(tokens), cols)
    if q is None:
        q = empty_2d(qshape[0], qshape[1], torch.uint8, x.device)
    if s is None:
        s = torch.empty(sshape, dtype=torch.float32, device=x.device)
    _need(q, qshape, torch.uint8, "q")
    _need_dense(s, sshape, "s")
    fn = lib().puro_fp8_quant_transpose_pow2 if pow2 else lib().puro_fp8_quant_transpose
    _check(fn(_ptr(x), _dtype_code(x), tokens, cols, _ld(x), 1 if transpose_out else 0, _ptr(q), _ld(q),
              _ptr(s), _stream(stream)), "puro_fp8_quant_transpose")
    return q, s


def _dual_outs(tokens, cols, transpose_out, device, q_row, s_row, q_tok, s_tok):
    if q_row is None:
        q_row = empty_2d(tokens, cols, torch.uint8, device)
    if s_row is None:
        s_row = torch.empty((tokens, _nblk(cols)), dtype=torch.float32, device=device)
    qshape = (cols, tokens) if transpose_out else (tokens, cols)
    sshape = (cols, _nblk(tokens)) if transpose_out else (_nblk(tokens), cols)
    if q_tok is None:
        q_tok = empty_2d(qshape[0], qshape[1], torch.uint8, device)
    if s_tok is None:
        s_tok = torch.empty(sshape, dtype=torch.float32, device=device)
    _need(q_row, (tokens, cols), torch.uint8, "q_row")
    _need_dense(s_row, (tokens, _nblk(cols)), "s_row")
    _need(q_tok, qshape, torch.uint8, "q_tok")
    _need_dense(s_tok, sshape, "s_tok")
    return q_row, s_row, q_tok, s_tok


@_stream_allocs
def puro_fp8_quant_dual(x, transpose_out=True, q_row=None, s_row=None, q_tok=None, s_tok=None,
                        stream=None, pow2=False):
    """One read of x [tokens][cols]: the outputs of puro_fp8_quant_act(x) and of
    puro_fp8_quant_transpose(x, transpose_out).  Returns (q_row, s_row, q_tok, s_tok)."""
    tokens, cols = x.shape
    q_row, s_row, q_tok, s_tok = _dual_outs(tokens, cols, transpose_out, x.device, q_row, s_row, q_tok, s_tok)
    fn = lib().puro_fp8_quant_dual_pow2 if pow2 else lib().puro_fp8_quant_dual
    _check(fn(_ptr(x), _dtype_code(x), tokens, cols, _ld(x), _ptr(q_row), _ld(q_row), _ptr(s_row),
              1 if transpose_out else 0, _ptr(q_tok), _ld(q_tok), _ptr(s_tok), _stream(stream)),
           "puro_fp8_quant_dual")
    return q_row, s_row, q_tok, s_tok


@_stream_allocs
def puro_fp8_swiglu_quant_dual(gate, up, transpose_out=True, h=None, store_h=True, q_row=None, s_row=None,
                               q_tok=None, s_tok=None, stream=None, pow2=False):
    """h = bf16(silu(gate) * up) for bfloat16 gate, up [tokens][cols], quantised as
    puro_fp8_quant_dual(h, transpose_out) would.  h is written to `h` (allocated when None)
    unless store_h is False.  Returns (h or None, q_row, s_row, q_tok, s_tok)."""
    if gate.shape != up.shape:
        raise ValueError("gate and up shapes differ: %s vs %s" % (tuple(gate.shape), tuple(up.shape)))
    if gate.dtype != torch.bfloat16 or up.dtype != torch.bfloat16:
        raise TypeError("gate and up must be bfloat16")
    tokens, cols = gate.shape
    if store_h:
        if h is None:
            h = empty_2d(tokens, cols, torch.bfloat16, gate.device)
        _need(h, (tokens, cols), torch.bfloat16, "h")
    else:
        h = None
    q_row, s_row, q_tok, s_tok = _dual_outs(tokens, cols, transpose_out, gate.device, q_row, s_row, q_tok,
                                            s_tok)
    fn = lib().puro_fp8_swiglu_quant_dual_pow2 if pow2 else lib().puro_fp8_swiglu_quant_dual
    _check(fn(_ptr(gate), _ld(gate), _ptr(up), _ld(up), tokens, cols,
              _ptr(h) if h is not None else ctypes.c_void_p(0), _ld(h) if h is not None else 0,
              _ptr(q_row), _ld(q_row), _ptr(s_row), 1 if transpose_out else 0, _ptr(q_tok), _ld(q_tok),
              _ptr(s_tok), _stream(stream)), "puro_fp8_swiglu_quant_dual")
    return h, q_row, s_row, q_tok, s_tok


def gemm_dims(layout, A, B):
    """(M, N, K) of a product in the given layout."""
    if layout == "NT":
        (M, K), (N, K2) = A.shape, B.shape
    elif layout == "NN":
        (M, K), (K2, N) = A.shape, B.shape
    elif layout == "TN":
        (K, M), (K2, N) = A.shape, B.shape
    else:
        raise ValueError("layout must be NT, NN or TN, got %r" % (layout,))
    if K != K2:
        raise ValueError("contraction extents differ: %d vs %d" % (K, K2))
    return M, N, K


def scale_shapes(layout, bgran, M, N, K):
    """Dense shapes of (sA, sB) for a product."""
    KB, NB = _nblk(K), _nblk(N)
    sa = (KB, M) if layout == "TN" else (M, KB)
    if layout == "NT":
        sb = (NB, KB) if bgran == "128x128" else (N, KB)
    else:
        sb = (KB, NB) if bgran == "128x128" else (KB, N)
    return sa, sb


def puro_fp8_gemm_workspace_size(layout, M, N, K, bgran):
    return int(lib().puro_fp8_gemm_workspace_size(LAYOUTS[layout], M, N, K, BGRAN[bgran]))


def puro_fp8_gemm_mx_workspace_size(layout, M, N, K, bgran):
    return int(lib().puro_fp8_gemm_mx_workspace_size(LAYOUTS[layout], M, N, K, BGRAN[bgran]))


def puro_fp8_gemm_native_workspace_size(layout, M, N, K, bgran):
    return int(lib().puro_fp8_gemm_native_workspace_size(LAYOUTS[layout], M, N, K, BGRAN[bgran]))


@_stream_allocs
def puro_fp8_gemm(layout, A, sA, B, sB, bgran="128x128", out_dtype=torch.bfloat16, C=None,
                  workspace=None, stream=None, mx=False, native=False):
    """Blockwise-scaled E4M3 GEMM; returns C [M][N] (float32 or bfloat16).
    mx: the scaled-FP8-matrix-core variant (puro_fp8_gemm_mx: power-of-two scales,
    extents multiples of 128).  native: block partials on the native FP8 matrix
    cores (puro_fp8_gemm_native: amax/448 scales, extents multiples of 128, not
    FP32-exact per block)."""
    if mx and native:
        raise ValueError("mx and native are different entry points")
    M, N, K = gemm_dims(layout, A, B)
    if A.dtype != torch.uint8 or B.dtype != torch.uint8:
        raise TypeError("A and B hold E4M3 codes (torch.uint8)")
    sa_shape, sb_shape = scale_shapes(layout, bgran, M, N, K)
    _need_dense(sA, sa_shape, "sA")
    _need_dense(sB, sb_shape, "sB")
    if out_dtype not in (torch.float32, torch.bfloat16):
        raise TypeError("out_dtype is float32 or bfloat16")
    if C is None:
        C = empty_2d(M, N, out_dtype, A.device)
    _need(C, (M, N), out_dtype, "C")
    size_fn = (puro_fp8_gemm_mx_workspace_size if mx else
               puro_fp8_gemm_native_workspace_size if native else puro_fp8_gemm_workspace_size)
    need = size_fn(layout, M, N, K, bgran)
    if need and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=A.device)
    ws_bytes = workspace.numel() if workspace is not None else 0
    name = "puro_fp8_gemm_mx" if mx else "puro_fp8_gemm_native" if native else "puro_fp8_gemm"
    _check(getattr(lib(), name)(LAYOUTS[layout], M, N, K, _ptr(A), _ld(A), _ptr(sA), _ptr(B), _ld(B), _ptr(sB),
                                BGRAN[bgran], _ptr(C), PURO_BF16 if out_dtype == torch.bfloat16 else PURO_F32,
                                _ld(C), _ptr(workspace), ws_bytes, _stream(stream)), name)
    return C


NOALLOC_SCRATCH_BYTES = 64 << 20   # PURO_NOALLOC_SCRATCH_BYTES


@_stream_allocs
def puro_fp8_gemm_noalloc(layout, A, sA, B, sB, C, bgran="128x128", stream=None):
    """puro_fp8_gemm into a caller-given C (float32 or bfloat16) with no workspace
    and no allocation: split-K partials go to the library's fixed device array."""
    M, N, K = gemm_dims(layout, A, B)
    if A.dtype != torch.uint8 or B.dtype != torch.uint8:
        raise TypeError("A and B hold E4M3 codes (torch.uint8)")
    sa_shape, sb_shape = scale_shapes(layout, bgran, M, N, K)
    _need_dense(sA, sa_shape, "sA")
    _need_dense(sB, sb_shape, "sB")
    if C.dtype not in (torch.float32, torch.bfloat16):
        raise TypeError("C is float32 or bfloat16")
    _need(C, (M, N), C.dtype, "C")
    _check(lib().puro_fp8_gemm_noalloc(LAYOUTS[layout], M, N, K, _ptr(A), _ld(A), _ptr(sA), _ptr(B), _ld(B),
                                       _ptr(sB), BGRAN[bgran], _ptr(C),
                                       PURO_BF16 if C.dtype == torch.bfloat16 else PURO_F32, _ld(C),
                                       _stream(stream)), "puro_fp8_gemm_noalloc")
    return C


def gemm_descs(layout, problems, bgran="128x128", out_dtype=torch.bfloat16):
    """Checked descriptors for puro_fp8_gemm_grouped.  Each problem is
    (A, sA, B, sB), (A, sA, B, sB, C), or a dict with "segments" (a list of
    (A, sA, B, sB) summed into one output), optional "C" and "accumulate"
    (C += the sum instead of C = the sum).  Missing outputs are allocated.
    Returns (ctypes array of GemmDesc, list of C)."""
    if out_dtype not in (torch.float32, torch.bfloat16):
        raise TypeError("out_dtype is float32 or bfloat16")
    descs = (GemmDesc * max(len(problems), 1))()
    outs = []
    for i, prob in enumerate(problems):
        if isinstance(prob, dict):
            segs, C, acc = prob["segments"], prob.get("C"), prob.get("accumulate", False)
        else:
            segs, C, acc = [prob[:4]], (prob[4] if len(prob) > 4 else None), False
        if acc and C is None:
            raise ValueError("accumulate needs C")
        MN = None
        raw = []
        for A, sA, B, sB in segs:
            M, N, K = gemm_dims(layout, A, B)
            if MN is not None and (M, N) != MN:
                raise ValueError("segments of one problem share M and N")
            MN = (M, N)
            if A.dtype != torch.uint8 or B.dtype != torch.uint8:
                raise TypeError("A and B hold E4M3 codes (torch.uint8)")
            sa_shape, sb_shape = scale_shapes(layout, bgran, M, N, K)
            _need_dense(sA, sa_shape, "sA")
            _need_dense(sB, sb_shape, "sB")
            raw.append((K, _ptr(A), _ld(A), _ptr(sA), _ptr(B), _ld(B), _ptr(sB)))
        M, N = MN
        if C is None:
            C = empty_2d(M, N, out_dtype, segs[0][0].device)
        _need(C, (M, N), out_dtype, "C")
        descs[i] = gemm_desc(M, N, raw, _ptr(C), _ld(C), acc)
        outs.append(C)
    return descs, outs


@_stream_allocs
def puro_fp8_gemm_grouped(layout, problems, bgran="128x128", out_dtype=torch.bfloat16, stream=None, mx=False,
                          native=False):
    """Independent blockwise-scaled E4M3 GEMMs sharing layout, B-scale
    granularity and output dtype, in as few launches as possible.
    problems: list of (A, sA, B, sB) or (A, sA, B, sB, C); returns the list of C.
    mx=True calls puro_fp8_gemm_grouped_mx, native=True puro_fp8_gemm_grouped_native."""
    if mx and native:
        raise ValueError("mx and native are two different datapaths")
    name = "puro_fp8_gemm_grouped_mx" if mx else "puro_fp8_gemm_grouped_native" if native else "puro_fp8_gemm_grouped"
    descs, outs = gemm_descs(layout, problems, bgran, out_dtype)
    _check(getattr(lib(), name)(LAYOUTS[layout], BGRAN[bgran], PURO_BF16 if out_dtype == torch.bfloat16 else PURO_F32,
                                descs, len(problems), _stream(stream)), name)
    return outs
