"""The C-ABI library on the host, without a GPU: it loads, exports every call
include/puro_fp8.h declares, and rejects bad arguments before any launch.

Every call made here either fails validation or has nothing to do (empty
extents), so no HIP work is ever enqueued.
"""
import ctypes
import os
import re
import subprocess

import pytest

import blockwise_fp8_gemm_amd as pf

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "puro_fp8.h")

OK, NULL, SHAPE, ALIGN, ENUM, WORKSPACE = 0, 1, 2, 3, 4, 5
P = ctypes.c_void_p(1 << 20)   # 16-byte aligned, never dereferenced (validation fails first)
P_ODD = ctypes.c_void_p((1 << 20) + 4)
NUL = ctypes.c_void_p(0)


def _declared():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\S[^\n;]*?\b(puro_\w+)\s*\(", text, flags=re.M)))


def test_header_declares_the_calls():
    names = _declared()
    for n in ("puro_fp8_quant_act", "puro_fp8_quant_weight", "puro_fp8_quant_transpose",
              "puro_fp8_gemm", "puro_fp8_gemm_workspace_size", "puro_fp8_gemm_grouped",
              "puro_fp8_quant_dual", "puro_fp8_quant_act_pow2", "puro_fp8_quant_weight_pow2",
              "puro_fp8_quant_transpose_pow2", "puro_fp8_quant_dual_pow2", "puro_fp8_gemm_mx",
              "puro_fp8_gemm_mx_workspace_size", "puro_status_string",
              "puro_fp8_quant_weight_grouped", "puro_fp8_quant_weight_grouped_pow2",
              "puro_fp8_swiglu_quant_dual", "puro_fp8_swiglu_quant_dual_pow2",
              "puro_fp8_gemm_native", "puro_fp8_gemm_native_workspace_size", "puro_fp8_gemm_noalloc",
              "puro_fp8_gemm_grouped_mx", "puro_fp8_gemm_grouped_native", "puro_fp8_version"):
        assert n in names


def test_library_exports_every_declared_symbol():
    L = pf.lib()
    for name in _declared():
        assert hasattr(L, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", pf.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r" T (\w+)$", out, flags=re.M))
    assert set(_declared()) <= exported


def test_status_strings():
    for st in range(8):
        assert pf.puro_status_string(st)
    assert pf.puro_status_string(99) == "unknown status"
    assert pf.puro_fp8_version() == 100


def _qa(x=P, dt=1, rows=4, cols=128, ldx=128, q=P, ldq=128, s=P):
    return pf.lib().puro_fp8_quant_act(x, dt, rows, cols, ldx, q, ldq, s, None)


def _qw(x=P, dt=0, rows=128, cols=128, ldx=128, q=P, ldq=128, s=P):
    return pf.lib().puro_fp8_quant_weight(x, dt, rows, cols, ldx, q, ldq, s, None)


def _qt(x=P, dt=1, tokens=256, cols=64, ldx=64, t=1, q=P, ldq=256, s=P):
    return pf.lib().puro_fp8_quant_transpose(x, dt, tokens, cols, ldx, t, q, ldq, s, None)


def _qa2(x=P, dt=1, rows=4, cols=128, ldx=128, q=P, ldq=128, s=P):
    return pf.lib().puro_fp8_quant_act_pow2(x, dt, rows, cols, ldx, q, ldq, s, None)


def _qw2(x=P, dt=0, rows=128, cols=128, ldx=128, q=P, ldq=128, s=P):
    return pf.lib().puro_fp8_quant_weight_pow2(x, dt, rows, cols, ldx, q, ldq, s, None)


@pytest.mark.parametrize("fn", [_qa, _qw, _qa2, _qw2])
def test_quant_validation(fn):
    assert fn(dt=2) == ENUM
    assert fn(dt=-1) == ENUM
    assert fn(rows=-1) == SHAPE
    assert fn(cols=-5) == SHAPE
    assert fn(ldx=64) == SHAPE
    assert fn(ldq=64) == SHAPE
    assert fn(rows=1 << 24) == SHAPE
    assert fn(x=NUL) == NULL
    assert fn(q=NUL) == NULL
    assert fn(s=NUL) == NULL
    assert fn(ldx=136) == ALIGN
    assert fn(ldq=136) == ALIGN
    assert fn(x=P_ODD) == ALIGN
    assert fn(q=P_ODD) == ALIGN
    assert fn(s=ctypes.c_void_p((1 << 20) + 2)) == ALIGN
    # empty: nothing to do, NULL pointers allowed
    assert fn(x=NUL, q=NUL, s=NUL, rows=0) == OK
    assert fn(x=NUL, q=NUL, s=NUL, cols=0, ldx=0, ldq=0) == OK


def test_quant_transpose_validation():
    assert _qt(t=2) == ENUM
    assert _qt(t=-1) == ENUM
    assert _qt(dt=5) == ENUM
    assert _qt(ldq=128) == SHAPE          # transposed output rows hold `tokens` codes
    assert _qt(t=0, ldq=32) == SHAPE      # untransposed output rows hold `cols` codes
    assert _qt(ldx=32) == SHAPE
    assert _qt(x=NUL) == NULL
    assert _qt(ldq=264) == ALIGN
    assert _qt(x=NUL, q=NUL, s=NUL, tokens=0, ldq=0) == OK


def _qd(x=P, dt=1, tokens=256, cols=128, ldx=128, qr=P, ldqr=128, sr=P, t=1, qt=P, ldqt=256, st=P):
    return pf.lib().puro_fp8_quant_dual(x, dt, tokens, cols, ldx, qr, ldqr, sr, t, qt, ldqt, st, None)


def test_quant_dual_validation():
    assert _qd(t=3) == ENUM
    assert _qd(dt=9) == ENUM
    assert _qd(ldqr=64) == SHAPE          # row copy rows hold `cols` codes
    assert _qd(ldqt=128) == SHAPE         # transposed copy rows hold `tokens` codes
    assert _qd(t=0, ldqt=64) == SHAPE     # untransposed copy rows hold `cols` codes
    assert _qd(tokens=-2) == SHAPE
    assert _qd(qr=NUL) == NULL
    assert _qd(st=NUL) == NULL
    assert _qd(ldqr=136) == ALIGN
    assert _qd(qt=P_ODD) == ALIGN
    assert _qd(x=NUL, qr=NUL, sr=NUL, qt=NUL, st=NUL, tokens=0, ldqt=0) == OK


def _sw(g=P, ldg=128, u=P, ldu=128, tokens=256, cols=128, h=P, ldh=128, qr=P, ldqr=128, sr=P, t=1, qt=P,
        ldqt=256, st=P, pow2=False):
    L = pf.lib()
    fn = L.puro_fp8_swiglu_quant_dual_pow2 if pow2 else L.puro_fp8_swiglu_quant_dual
    return fn(g, ldg, u, ldu, tokens, cols, h, ldh, qr, ldqr, sr, t, qt, ldqt, st, None)


def test_swiglu_quant_dual_validation():
    for pow2 in (False, True):
        assert _sw(t=2, pow2=pow2) == ENUM
        assert _sw(ldg=64, pow2=pow2) == SHAPE       # gate rows hold `cols` values
        assert _sw(ldu=64, pow2=pow2) == SHAPE
        assert _sw(ldh=64, pow2=pow2) == SHAPE
        assert _sw(ldqt=128, pow2=pow2) == SHAPE     # transposed copy rows hold `tokens` codes
        assert _sw(cols=-1, pow2=pow2) == SHAPE
        assert _sw(g=NUL, pow2=pow2) == NULL
        assert _sw(u=NUL, pow2=pow2) == NULL
        assert _sw(sr=NUL, pow2=pow2) == NULL
        assert _sw(ldu=136, pow2=pow2) == ALIGN
        assert _sw(ldh=136, pow2=pow2) == ALIGN
        assert _sw(h=P_ODD, pow2=pow2) == ALIGN
        assert _sw(u=P_ODD, pow2=pow2) == ALIGN
        # h is optional: NULL h with any ldh is valid; empty problems enqueue nothing
        assert _sw(g=NUL, u=NUL, h=NUL, ldh=0, qr=NUL, sr=NUL, qt=NUL, st=NUL, tokens=0, ldqt=0,
                   pow2=pow2) == OK


def _gemm(layout=0, M=256, N=256, K=256, A=P, lda=256, sA=P, B=P, ldb=256, sB=P, bg=1, C=P,
          cdt=1, ldc=256, ws=NUL, wsb=0):
    return pf.lib().puro_fp8_gemm(layout, M, N, K, A, lda, sA, B, ldb, sB, bg, C, cdt, ldc, ws,
                                  wsb, None)


def test_gemm_validation():
    assert _gemm(layout=3) == ENUM
    assert _gemm(bg=2) == ENUM
    assert _gemm(cdt=7) == ENUM
    assert _gemm(M=-1) == SHAPE
    assert _gemm(K=1 << 24) == SHAPE
    assert _gemm(lda=128) == SHAPE
    assert _gemm(ldb=128) == SHAPE
    assert _gemm(ldc=128) == SHAPE
    assert _gemm(layout=2, M=512, lda=256) == SHAPE       # TN: A rows hold M codes
    assert _gemm(layout=1, N=512, ldb=256) == SHAPE       # NN: B rows hold N codes
    assert _gemm(A=NUL) == NULL
    assert _gemm(sA=NUL) == NULL
    assert _gemm(B=NUL) == NULL
    assert _gemm(sB=NUL) == NULL
    assert _gemm(C=NUL) == NULL
    assert _gemm(lda=264) == ALIGN
    assert _gemm(ldc=264) == ALIGN
    assert _gemm(A=P_ODD) == ALIGN
    assert _gemm(C=P_ODD) == ALIGN
    assert _gemm(sB=ctypes.c_void_p((1 << 20) + 1)) == ALIGN
    # empty products: nothing enqueued
    assert _gemm(M=0, A=NUL, sA=NUL, C=NUL) == OK
    assert _gemm(N=0, B=NUL, sB=NUL, C=NUL, ldb=256, ldc=0) == OK


GROUPED = ["puro_fp8_gemm_grouped", "puro_fp8_gemm_grouped_mx", "puro_fp8_gemm_grouped_native"]


def _grouped(descs, count=None, layout=0, bg=1, cdt=1, arr=True, name="puro_fp8_gemm_grouped"):
    n = len(descs)
    a = (pf.GemmDesc * max(n, 1))(*descs) if arr else None
    return getattr(pf.lib(), name)(layout, bg, cdt, a, n if count is None else count, None)


def _desc(M=256, N=256, K=256, A=P, lda=256, sA=P, B=P, ldb=256, sB=P, C=P, ldc=256, nseg=1, acc=0, seg2=None):
    d = pf.gemm_desc(M, N, [(K, A, lda, sA, B, ldb, sB)] + ([seg2] if seg2 else []), C, ldc, bool(acc))
    d.nseg, d.accumulate = nseg if not seg2 else 2, acc
    return d


@pytest.mark.parametrize("name", GROUPED)
def test_gemm_grouped_validation(name):
    def g(descs, **kw):
        return _grouped(descs, name=name, **kw)
    assert g([]) == OK                                  # nothing to do
    assert g([], layout=5) == ENUM
    assert g([], cdt=3) == ENUM
    assert g([_desc()], count=-1) == SHAPE
    assert g([_desc()], count=4097) == SHAPE
    assert g([_desc()], arr=False, count=1) == NULL
    assert g([_desc()], bg=4) == ENUM
    assert g([_desc(), _desc(ldc=128)]) == SHAPE       # the second problem fails
    assert g([_desc(A=NUL), _desc()]) == NULL
    assert g([_desc(), _desc(C=P_ODD)]) == ALIGN
    assert g([_desc(), _desc(lda=264)]) == ALIGN
    assert g([_desc(nseg=0)]) == SHAPE
    assert g([_desc(nseg=5)]) == SHAPE
    assert g([_desc(acc=2)]) == ENUM
    assert g([_desc(seg2=(256, P, 128, P, P, 256, P))]) == SHAPE    # second segment's lda < K
    assert g([_desc(seg2=(256, NUL, 256, P, P, 256, P))]) == NULL
    # only empty problems: nothing enqueued
    assert g([_desc(M=0, A=NUL, sA=NUL, C=NUL), _desc(N=0, B=NUL, sB=NUL, C=NUL, ldc=0)]) == OK


@pytest.mark.parametrize("name", GROUPED[1:])
def test_gemm_grouped_fp8_datapaths_take_aligned_problems_only(name):
    # each call holds a problem that the exact launcher would accept but these reject,
    # so nothing is enqueued (the pointers are not device memory)
    def g(descs):
        return _grouped(descs, name=name)
    assert g([_desc(), _desc(K=200)]) == SHAPE                        # K not a multiple of 128
    assert g([_desc(M=192, C=P)]) == SHAPE                            # M
    assert g([_desc(N=200, ldb=256, ldc=208)]) == SHAPE               # N
    assert g([_desc(K=0)]) == SHAPE                                   # empty K with a non-empty output
    assert g([_desc(seg2=(200, P, 256, P, P, 256, P))]) == SHAPE      # the second segment's K
    big = 1 << 28
    assert g([_desc(lda=big, K=256)]) == SHAPE                        # leading dimension beyond 2^28


def test_workspace_size_is_defined_for_every_layout():
    for layout in ("NT", "NN", "TN"):
        for bg in ("1x128", "128x128"):
            assert pf.puro_fp8_gemm_workspace_size(layout, 8192, 2048, 8192, bg) >= 0
    assert pf.lib().puro_fp8_gemm_workspace_size(9, 128, 128, 128, 0) == 0


def test_pow2_transpose_and_dual_validation():
    L = pf.lib()
    assert L.puro_fp8_quant_transpose_pow2(P, 1, 256, 64, 64, 2, P, 256, P, None) == ENUM
    assert L.puro_fp8_quant_transpose_pow2(P, 1, 256, 64, 64, 1, P, 128, P, None) == SHAPE
    assert L.puro_fp8_quant_transpose_pow2(NUL, 1, 0, 64, 64, 1, NUL, 0, NUL, None) == OK
    assert L.puro_fp8_quant_dual_pow2(P, 1, 256, 128, 128, P, 128, P, 3, P, 256, P, None) == ENUM
    assert L.puro_fp8_quant_dual_pow2(P, 1, 256, 128, 128, P, 128, P, 1, NUL, 256, P, None) == NULL
    assert L.puro_fp8_quant_dual_pow2(NUL, 1, 0, 128, 128, NUL, 128, NUL, 1, NUL, 0, NUL, None) == OK


def _gmx(layout=0, M=256, N=256, K=256, A=P, lda=256, sA=P, B=P, ldb=256, sB=P, bg=1, C=P, cdt=1, ldc=256,
         ws=NUL, wsb=0):
    return pf.lib().puro_fp8_gemm_mx(layout, M, N, K, A, lda, sA, B, ldb, sB, bg, C, cdt, ldc, ws, wsb, None)


def test_gemm_mx_validation():
    assert _gmx(layout=3) == ENUM
    assert _gmx(cdt=5) == ENUM
    assert _gmx(M=-1) == SHAPE
    assert _gmx(ldc=128) == SHAPE
    assert _gmx(A=NUL) == NULL
    assert _gmx(C=P_ODD) == ALIGN
    # extents must be multiples of 128
    assert _gmx(M=200) == SHAPE
    assert _gmx(N=136, ldb=256, ldc=256) == SHAPE
    assert _gmx(K=192) == SHAPE
    assert _gmx(K=0, A=NUL, sA=NUL, B=NUL, sB=NUL) == SHAPE
    # leading dimensions of A and B below 2^28 (the tile kernel's 32-bit lane offsets)
    assert _gmx(lda=1 << 28) == SHAPE
    assert _gmx(ldb=1 << 28) == SHAPE
    # empty outputs: nothing enqueued
    assert _gmx(M=0, A=NUL, sA=NUL, C=NUL) == OK
    assert pf.puro_fp8_gemm_mx_workspace_size("NT", 200, 256, 256, "1x128") == 0
    assert pf.puro_fp8_gemm_mx_workspace_size("NT", 256, 256, 8192, "1x128") >= 0


def _gnat(layout=0, M=256, N=256, K=256, A=P, lda=256, sA=P, B=P, ldb=256, sB=P, bg=1, C=P, cdt=1, ldc=256,
          ws=NUL, wsb=0):
    return pf.lib().puro_fp8_gemm_native(layout, M, N, K, A, lda, sA, B, ldb, sB, bg, C, cdt, ldc, ws, wsb, None)


def test_gemm_native_validation():
    assert _gnat(layout=3) == ENUM
    assert _gnat(bg=2) == ENUM
    assert _gnat(cdt=5) == ENUM
    assert _gnat(M=-1) == SHAPE
    assert _gnat(ldc=128) == SHAPE
    assert _gnat(A=NUL) == NULL
    assert _gnat(sB=NUL) == NULL
    assert _gnat(C=P_ODD) == ALIGN
    assert _gnat(lda=264) == ALIGN
    # extents must be multiples of 128
    assert _gnat(M=200) == SHAPE
    assert _gnat(N=136, ldb=256, ldc=256) == SHAPE
    assert _gnat(K=192) == SHAPE
    assert _gnat(K=0, A=NUL, sA=NUL, B=NUL, sB=NUL) == SHAPE
    # leading dimensions of A and B below 2^28
    assert _gnat(lda=1 << 28) == SHAPE
    assert _gnat(ldb=1 << 28) == SHAPE
    # a split-K plan needs its workspace
    need = pf.puro_fp8_gemm_native_workspace_size("NT", 256, 256, 16384, "1x128")
    assert need > 0
    assert _gnat(K=16384, lda=16384, ldb=16384, bg=0) == WORKSPACE
    assert _gnat(K=16384, lda=16384, ldb=16384, bg=0, ws=P, wsb=need - 1) == WORKSPACE
    # empty outputs: nothing enqueued
    assert _gnat(M=0, A=NUL, sA=NUL, C=NUL) == OK
    assert pf.puro_fp8_gemm_native_workspace_size("NT", 200, 256, 256, "1x128") == 0
    assert pf.puro_fp8_gemm_native_workspace_size("NN", 256, 256, 256, "128x128") == 0


def test_gemm_noalloc_validation():
    L = pf.lib()

    def g(layout=0, M=256, N=256, K=256, A=P, lda=256, sA=P, B=P, ldb=256, sB=P, bg=1, C=P, cdt=1, ldc=256):
        return L.puro_fp8_gemm_noalloc(layout, M, N, K, A, lda, sA, B, ldb, sB, bg, C, cdt, ldc, None)
    assert g(layout=3) == ENUM
    assert g(M=-1) == SHAPE
    assert g(A=NUL) == NULL
    assert g(C=P_ODD) == ALIGN
    # a plan needing more than the fixed array is rejected before any HIP call
    assert pf.puro_fp8_gemm_workspace_size("NT", 384, 5504, 16384, "1x128") > pf.NOALLOC_SCRATCH_BYTES
    assert g(M=384, N=5504, K=16384, lda=16384, ldb=16384, bg=0, ldc=5504) == WORKSPACE
    # empty output: nothing to do
    assert g(M=0, A=NUL, sA=NUL, C=NUL) == OK


@pytest.mark.parametrize("name", ["puro_fp8_quant_weight_grouped", "puro_fp8_quant_weight_grouped_pow2"])
def test_quant_weight_grouped_validation(name):
    fn = getattr(pf.lib(), name)
    D = pf.QuantWeightDesc

    def call(items, dt=0, count=None):
        arr = (D * max(len(items), 1))(*items)
        return fn(dt, arr, len(items) if count is None else count, None)

    good = D(P, 256, 256, 256, P, 256, P)
    empty = D(NUL, 0, 256, 256, NUL, 256, NUL)
    assert call([]) == OK
    assert call([empty, empty]) == OK                     # nothing to do: no launch
    assert call([good], dt=7) == ENUM
    assert call([good], count=-1) == SHAPE
    assert call([good], count=4097) == SHAPE
    assert fn(0, None, 1, None) == NULL
    # the first failing item decides, and nothing is enqueued before validation ends
    assert call([good, D(P, 256, 256, 100, P, 256, P)]) == SHAPE        # ldw < cols
    assert call([good, D(P, 256, 256, 264, P, 256, P)]) == ALIGN        # ldw not a multiple of 16
    assert call([good, D(P_ODD, 256, 256, 256, P, 256, P)]) == ALIGN    # w not 16-byte aligned
    assert call([good, D(NUL, 256, 256, 256, P, 256, P)]) == NULL
    assert call([good, D(P, 256, 256, 256, P, 256, NUL)]) == NULL
    assert call([D(P, -1, 256, 256, P, 256, P), D(NUL, 4, 4, 16, P, 16, P)]) == SHAPE
    # the transposed copy [cols][rows] is checked like the codes, rows and cols swapped
    assert call([D(P, 256, 384, 384, P, 384, P, P, 128, P)]) == SHAPE     # ldqt < rows
    assert call([D(P, 256, 384, 384, P, 384, P, P, 264, P)]) == ALIGN     # ldqt not a multiple of 16
    assert call([D(P, 256, 384, 384, P, 384, P, P_ODD, 256, P)]) == ALIGN
    assert call([D(P, 256, 384, 384, P, 384, P, P, 256, NUL)]) == NULL    # st missing
    assert call([D(NUL, 0, 384, 384, NUL, 384, NUL, P, 0, NUL)]) == OK    # empty weight: nothing



def test_header_compiles_as_c_and_links(tmp_path):
    """The header is plain C: a C11 program includes it, links against the library and calls
    the two calls that need no GPU."""
    src = tmp_path / "use.c"
    src.write_text('#include <stdio.h>\n#include <string.h>\n#include "puro_fp8.h"\n'
                   "int main(void) {\n"
                   "    puro_quant_weight_desc_t d;\n    puro_gemm_desc_t g;\n"
                   "    memset(&d, 0, sizeof d);\n    memset(&g, 0, sizeof g);\n"
                   "    if (puro_fp8_version() != 100) return 1;\n"
                   "    if (strcmp(puro_status_string(PURO_ERR_SHAPE), puro_status_string(PURO_OK)) == 0) return 2;\n"
                   "    printf(\"%s\\n\", puro_status_string(PURO_ERR_ALIGN));\n    return 0;\n}\n")
    exe = tmp_path / "use"
    libdir = os.path.dirname(pf.LIB_PATH)
    subprocess.run(["gcc", "-std=c11", "-Wall", "-Werror", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
                    "-I" + os.path.dirname(HEADER), str(src), "-o", str(exe), "-L" + libdir, "-lpuro_fp8",
                    "-Wl,-rpath," + libdir], check=True, capture_output=True, text=True)
    out = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    assert out.returncode == 0, out.stderr
    assert out.stdout.strip() == pf.puro_status_string(3)
