// C-ABI entry points: host-side validation, then one enqueue on the caller's
// stream.  Declarations and the contract of each call are in puro_fp8.h.
#include "../../include/puro_fp8.h"
#include "kernels.h"

#include <mutex>
#include <vector>

namespace {

// Largest extent accepted along any dimension (keeps every grid dimension and
// 64-bit offset computation in range).
constexpr int64_t kMaxExtent = int64_t(1) << 23;

bool aligned(const void *p, uintptr_t a)
{
    return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0;
}

bool bad_extent(int64_t n)
{
    return n < 0 || n > kMaxExtent;
}

bool bad_ld(int64_t ld, int64_t row_len)
{
    return ld < row_len || ld > kMaxExtent;
}

// Shared checks of the three quantisers.  `elems` is the number of input
// elements, `nscale` the number of scale entries.
puro_status_t check_quant(const void *x, int xdt, int64_t rows, int64_t cols, int64_t ldx,
                          const uint8_t *q, int64_t ldq, int64_t ldq_min, const float *s)
{
    if (xdt != PURO_F32 && xdt != PURO_BF16)
        return PURO_ERR_ENUM;
    if (bad_extent(rows) || bad_extent(cols) || bad_ld(ldx, cols) || bad_ld(ldq, ldq_min))
        return PURO_ERR_SHAPE;
    const bool empty = rows == 0 || cols == 0;
    if (!empty && (!x || !q || !s))
        return PURO_ERR_NULL;
    if (ldx % 16 || ldq % 16)
        return PURO_ERR_ALIGN;
    if ((x && !aligned(x, 16)) || (q && !aligned(q, 16)) || (s && !aligned(s, 4)))
        return PURO_ERR_ALIGN;
    return PURO_OK;
}

puro_status_t from_hip(hipError_t e)
{
    return e == hipSuccess ? PURO_OK : PURO_ERR_HIP;
}

} // namespace

static puro_status_t quant_act_impl(const void *x, puro_dtype_t xdt, int64_t rows, int64_t cols, int64_t ldx,
                                    uint8_t *q, int64_t ldq, float *s, bool pow2, hipStream_t stream)
{
    try {
        puro_status_t st = check_quant(x, xdt, rows, cols, ldx, q, ldq, cols, s);
        if (st != PURO_OK)
            return st;
        if (rows == 0 || cols == 0)
            return PURO_OK;
        return from_hip(puro::launch_quant_act(x, xdt == PURO_BF16, rows, cols, ldx, q, ldq, s,
                                               pow2, stream));
    } catch (...) {
        return PURO_ERR_INTERNAL;
    }
}

static puro_status_t quant_weight_impl(const void *w, puro_dtype_t wdt, int64_t rows, int64_t cols,
                                       int64_t ldw, uint8_t *q, int64_t ldq, float *s, bool pow2,
                                       hipStream_t stream)
{
    try {
        puro_status_t st = check_quant(w, wdt, rows, cols, ldw, q, ldq, cols, s);
        if (st != PURO_OK)
            return st;
        if (rows == 0 || cols == 0)
            return PURO_OK;
        return from_hip(puro::launch_quant_weight(w, wdt == PURO_BF16, rows, cols, ldw, q, ldq, s,
                                                  pow2, stream));
    } catch (...) {
        return PURO_ERR_INTERNAL;
    }
}

static puro_status_t quant_weight_grouped_impl(puro_dtype_t wdt, const puro_quant_weight_desc_t *items,
                                               int count, bool pow2, hipStream_t stream)
{
    try {
        if (wdt != PURO_F32 && wdt != PURO_BF16)
            return PURO_ERR_ENUM;
        if (count < 0 || count > PURO_QUANT_MAX_GROUP)
            return PURO_ERR_SHAPE;
        if (count > 0 && !items)
            return PURO_ERR_NULL;
        std::vector<puro::QuantWeightItem> v;
        v.reserve((size_t)count);
        for (int i = 0; i < count; i++) {
            const puro_quant_weight_desc_t &d = items[i];
            puro_status_t st = check_quant(d.w, wdt, d.rows, d.cols, d.ldw, d.q, d.ldq, d.cols, d.s);
            if (st != PURO_OK)
                return st;
            if (d.qt) {   // transposed copy: qt [cols][rows], st [ceil(cols/128)][ceil(rows/128)]
                st = check_quant(d.w, wdt, d.rows, d.cols, d.ldw, d.qt, d.ldqt, d.rows, d.st);
                if (st != PURO_OK)
                    return st;
            }
            if (d.rows == 0 || d.cols == 0)
                continue;
            v.push_back({d.w, d.rows, d.cols, d.ldw, d.q, d.ldq, d.s, (d.cols + 127) / 128, d.qt,
                         d.qt ? d.ldqt : 0, d.qt ? d.st : nullptr, (d.rows + 127) / 128});
        }
        if (v.empty())
            return PURO_OK;
        return from_hip(puro::launch_quant_weight_group(v.data(), (int)v.size(), wdt == PURO_BF16, pow2, stream));
    } catch (...) {
        return PURO_ERR_INTERNAL;
    }
}

static puro_status_t quant_transpose_impl(const void *x, puro_dtype_t xdt, int64_t tokens, int64_t cols,
                                          int64_t ldx, int transpose_out, uint8_t *q, int64_t ldq, float *s,
                                          bool pow2, hipStream_t stream)
{
    try {
        if (transpose_out != 0 && transpose_out != 1)
            return PURO_ERR_ENUM;
        puro_status_t st = check_quant(x, xdt, tokens, cols, ldx, q, ldq,
                                       transpose_out ? tokens : cols, s);
        if (st != PURO_OK)
            return st;
        if (tokens == 0 || cols == 0)
            return PURO_OK;
        return from_hip(puro::launch_quant_transpose(x, xdt == PURO_BF16, tokens, cols, ldx,
                                                     transpose_out == 1, q, ldq, s, pow2, stream));
    } catch (...) {
        return PURO_ERR_INTERNAL;
    }
}

static puro_status_t quant_dual_impl(const void *x, puro_dtype_t xdt, int64_t tokens, int64_t cols,
                                     int64_t ldx, uint8_t *q_row, int64_t ldq_row, float *s_row,
                                     int transpose_out, uint8_t *q_tok, int64_t ldq_tok, float *s_tok,
                                     bool pow2, hipStream_t stream)
{
    try {
        if (transpose_out != 0 && transpose_out != 1)
            return PURO_ERR_ENUM;
        puro_status_t st = check_quant(x, xdt, tokens, cols, ldx, q_row, ldq_row, cols, s_row);
        if (st != PURO_OK)
            return st;
        st = check_quant(x, xdt, tokens, cols, ldx, q_tok, ldq_tok, transpose_out ? tokens : cols,
                         s_tok);
        if (st != PURO_OK)
            return st;
        if (tokens == 0 || cols == 0)
            return PURO_OK;
        return from_hip(puro::launch_quant_dual(x, xdt == PURO_BF16, tokens, cols, ldx, q_row,
                                                ldq_row, s_row, transpose_out == 1, q_tok, ldq_tok,
                                                s_tok, pow2, stream));
    } catch (...) {
        return PURO_ERR_INTERNAL;
    }
}

static puro_status_t swiglu_dual_impl(const void *gate, int64_t ldg, const void *up, int64_t ldu,
                                      int64_t tokens, int64_t cols, void *h, int64_t ldh, uint8_t *q_row,
                                      int64_t ldq_row, float *s_row, int transpose_out, uint8_t *q_tok,
                                      int64_t ldq_tok, float *s_tok, bool pow2, hipStream_t stream)
{
    try {
        if (transpose_out != 0 && transpose_out != 1)
            return PURO_ERR_ENUM;
        puro_status_t st = check_quant(gate, PURO_BF16, tokens, cols, ldg, q_row, ldq_row, cols, s_row);
        if (st != PURO_OK)
            return st;
        st = check_quant(up, PURO_BF16, tokens, cols, ldu, q_tok, ldq_tok, transpose_out ? tokens : cols,
                         s_tok);
        if (st != PURO_OK)
            return st;
        if (h) {
            if (bad_ld(ldh, cols))
                return PURO_ERR_SHAPE;
            if (ldh % 16 || !aligned(h, 16))
                return PURO_ERR_ALIGN;
        }
        if (tokens == 0 || cols == 0)
            return PURO_OK;
        return from_hip(puro::launch_swiglu_dual(static_cast<const uint16_t *>(gate), ldg,
                                                 static_cast<const uint16_t *>(up), ldu,
                                                 static_cast<uint16_t *>(h), ldh, tokens, cols, q_row, ldq_row,
                                                 s_row, transpose_out == 1, q_tok, ldq_tok, s_tok, pow2, stream));
    } catch (...) {
        return PURO_ERR_INTERNAL;
    }
}

extern "C" {

puro_status_t puro_fp8_swiglu_quant_dual(const void *gate, int64_t ldg, const void *up, int64_t ldu,
                                         int64_t tokens, int64_t cols, void *h, int64_t ldh, uint8_t *q_row,
                                         int64_t ldq_row, float *s_row, int transpose_out, uint8_t *q_tok,
                                         int64_t ldq_tok, float *s_tok, hipStream_t stream)
{
    return swiglu_dual_impl(gate, ldg, up, ldu, tokens, cols, h, ldh, q_row, ldq_row, s_row, transpose_out,
                            q_tok, ldq_tok, s_tok, false, stream);
}

puro_status_t puro_fp8_swiglu_quant_dual_pow2(const void *gate, int64_t ldg, const void *up, int64_t ldu,
                                              int64_t tokens, int64_t cols, void *h, int64_t ldh,
                                              uint8_t *q_row, int64_t ldq_row, float *s_row, int transpose_out,
                                              uint8_t *q_tok, int64_t ldq_tok, float *s_tok, hipStream_t stream)
{
    return swiglu_dual_impl(gate, ldg, up, ldu, tokens, cols, h, ldh, q_row, ldq_row, s_row, transpose_out,
                            q_tok, ldq_tok, s_tok, true, stream);
}

puro_status_t puro_fp8_quant_act(const void *x, puro_dtype_t xdt, int64_t rows, int64_t cols, int64_t ldx,
                                 uint8_t *q, int64_t ldq, float *s, hipStream_t stream)
{
    return quant_act_impl(x, xdt, rows, cols, ldx, q, ldq, s, false, stream);
}

puro_status_t puro_fp8_quant_weight(const void *w, puro_dtype_t wdt, int64_t rows, int64_t cols, int64_t ldw,
                                    uint8_t *q, int64_t ldq, float *s, hipStream_t stream)
{
    return quant_weight_impl(w, wdt, rows, cols, ldw, q, ldq, s, false, stream);
}

puro_status_t puro_fp8_quant_transpose(const void *x, puro_dtype_t xdt, int64_t tokens, int64_t cols,
                                       int64_t ldx, int transpose_out, uint8_t *q, int64_t ldq, float *s,
                                       hipStream_t stream)
{
    return quant_transpose_impl(x, xdt, tokens, cols, ldx, transpose_out, q, ldq, s, false, stream);
}

puro_status_t puro_fp8_quant_dual(const void *x, puro_dtype_t xdt, int64_t tokens, int64_t cols, int64_t ldx,
                                  uint8_t *q_row, int64_t ldq_row, float *s_row, int transpose_out,
                                  uint8_t *q_tok, int64_t ldq_tok, float *s_tok, hipStream_t stream)
{
    return quant_dual_impl(x, xdt, tokens, cols, ldx, q_row, ldq_row, s_row, transpose_out, q_tok, ldq_tok,
                           s_tok, false, stream);
}

puro_status_t puro_fp8_quant_act_pow2(const void *x, puro_dtype_t xdt, int64_t rows, int64_t cols, int64_t ldx,
                                      uint8_t *q, int64_t ldq, float *s, hipStream_t stream)
{
    return quant_act_impl(x, xdt, rows, cols, ldx, q, ldq, s, true, stream);
}

puro_status_t puro_fp8_quant_weight_grouped(puro_dtype_t wdt, const puro_quant_weight_desc_t *items, int count,
                                            hipStream_t stream)
{
    return quant_weight_grouped_impl(wdt, items, count, false, stream);
}

puro_status_t puro_fp8_quant_weight_grouped_pow2(puro_dtype_t wdt, const puro_quant_weight_desc_t *items,
                                                 int count, hipStream_t stream)
{
    return quant_weight_grouped_impl(wdt, items, count, true, stream);
}

puro_status_t puro_fp8_quant_weight_pow2(const void *w, puro_dtype_t wdt, int64_t rows, int64_t cols,
                                         int64_t ldw, uint8_t *q, int64_t ldq, float *s, hipStream_t stream)
{
    return quant_weight_impl(w, wdt, rows, cols, ldw, q, ldq, s, true, stream);
}

puro_status_t puro_fp8_quant_transpose_pow2(const void *x, puro_dtype_t xdt, int64_t tokens, int64_t cols,
                                            int64_t ldx, int transpose_out, uint8_t *q, int64_t ldq, float *s,
                                            hipStream_t stream)
{
    return quant_transpose_impl(x, xdt, tokens, cols, ldx, transpose_out, q, ldq, s, true, stream);
}

puro_status_t puro_fp8_quant_dual_pow2(const void *x, puro_dtype_t xdt, int64_t tokens, int64_t cols,
                                       int64_t ldx, uint8_t *q_row, int64_t ldq_row, float *s_row,
                                       int transpose_out, uint8_t *q_tok, int64_t ldq_tok, float *s_tok,
                                       hipStream_t stream)
{
    return quant_dual_impl(x, xdt, tokens, cols, ldx, q_row, ldq_row, s_row, transpose_out, q_tok, ldq_tok,
                           s_tok, true, stream);
}

static puro_status_t check_gemm(puro_layout_t layout, int64_t M, int64_t N, int64_t K,
                                const uint8_t *A, int64_t lda, const float *sA, const uint8_t *B,
                                int64_t ldb, const float *sB, puro_bscale_t bgran, const void *C,
                                puro_dtype_t cdt, int64_t ldc)
{
    if (layout != PURO_NT && layout != PURO_NN && layout != PURO_TN)
        return PURO_ERR_ENUM;
    if (bgran != PURO_SCALE_1x128 && bgran != PURO_SCALE_128x128)
        return PURO_ERR_ENUM;
    if (cdt != PURO_F32 && cdt != PURO_BF16)
        return PURO_ERR_ENUM;
    if (bad_extent(M) || bad_extent(N) || bad_extent(K))
        return PURO_ERR_SHAPE;
    const int64_t lda_min = layout == PURO_TN ? M : K;
    const int64_t ldb_min = layout == PURO_NT ? K : N;
    if (bad_ld(lda, lda_min) || bad_ld(ldb, ldb_min) || bad_ld(ldc, N))
        return PURO_ERR_SHAPE;
    const bool a_empty = M == 0 || K == 0, b_empty = N == 0 || K == 0, c_empty = M == 0 || N == 0;
    if ((!a_empty && (!A || !sA)) || (!b_empty && (!B || !sB)) || (!c_empty && !C))
        return PURO_ERR_NULL;
    if (lda % 16 || ldb % 16 || ldc % 16)
        return PURO_ERR_ALIGN;
    if ((A && !aligned(A, 16)) || (B && !aligned(B, 16)) || (C && !aligned(C, 16)) ||
        (sA && !aligned(sA, 4)) || (sB && !aligned(sB, 4)))
        return PURO_ERR_ALIGN;
    return PURO_OK;
}

static puro::GemmProblem make_problem(puro_layout_t layout, int64_t M, int64_t N, int64_t K,
                                      const uint8_t *A, int64_t lda, const float *sA,
                                      const uint8_t *B, int64_t ldb, const float *sB,
                                      puro_bscale_t bgran, void *C, puro_dtype_t cdt, int64_t ldc)
{
    puro::GemmProblem p;
    p.layout = (int)layout;
    p.bgran = (int)bgran;
    p.c_bf16 = cdt == PURO_BF16;
    p.accumulate = false;
    p.M = M;
    p.N = N;
    p.nseg = 1;
    p.seg[0] = puro::GemmSegment{K, A, lda, sA, B, ldb, sB};
    for (int i = 1; i < puro::kGemmMaxSeg; i++)
        p.seg[i] = puro::GemmSegment{0, nullptr, 0, nullptr, nullptr, 0, nullptr};
    p.C = C;
    p.ldc = ldc;
    return p;
}

size_t puro_fp8_gemm_workspace_size(puro_layout_t layout, int64_t M, int64_t N, int64_t K,
                                    puro_bscale_t bgran)
{
    if (layout != PURO_NT && layout != PURO_NN && layout != PURO_TN)
        return 0;
    if (bgran != PURO_SCALE_1x128 && bgran != PURO_SCALE_128x128)
        return 0;
    if (bad_extent(M) || bad_extent(N) || bad_extent(K))
        return 0;
    puro::GemmProblem p = make_problem(layout, M, N, K, nullptr, 0, nullptr, nullptr, 0, nullptr,
                                       bgran, nullptr, PURO_F32, 0);
    return puro::gemm_workspace_bytes(p);
}

puro_status_t puro_fp8_gemm(puro_layout_t layout, int64_t M, int64_t N, int64_t K,
                            const uint8_t *A, int64_t lda, const float *sA, const uint8_t *B,
                            int64_t ldb, const float *sB, puro_bscale_t bgran, void *C,
                            puro_dtype_t cdt, int64_t ldc, void *workspace, size_t ws_bytes,
                            hipStream_t stream)
{
    try {
        puro_status_t st = check_gemm(layout, M, N, K, A, lda, sA, B, ldb, sB, bgran, C, cdt, ldc);
        if (st != PURO_OK)
            return st;
        puro::GemmProblem p = make_problem(layout, M, N, K, A, lda, sA, B, ldb, sB, bgran, C, cdt,
                                           ldc);
        const size_t need = puro::gemm_workspace_bytes(p);
        if (need > 0 && (!workspace || ws_bytes < need || !aligned(workspace, 256)))
            return PURO_ERR_WORKSPACE;
        if (M == 0 || N == 0)
            return PURO_OK;
        return from_hip(puro::launch_gemm(p, workspace, stream));
    } catch (...) {
        return PURO_ERR_INTERNAL;
    }
}

// ---------------------------------------------------------------------------
// Allocation-free GEMM: the split-K partial sums go to a fixed device array
// instead of a caller workspace.  Each GPU the library runs on holds its own
// copy of `scratch` (PURO_NOALLOC_SCRATCH_BYTES) until the process ends.  In
// host code `scratch` names a host-side stand-in, not device memory: its
// device address is looked up once per device, with that device current, and
// only that address is passed to kernels.
static __device__ __align__(256) unsigned char scratch[PURO_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxScratchDevices = 256;
static std::mutex g_scratch_mutex;
static void *g_scratch_ptr[kMaxScratchDevices];

// Device address of `scratch` on the device that runs `stream` (the current
// device for the null stream).
static puro_status_t scratch_for_stream(hipStream_t stream, void **out)
{
    int cur = 0;
    if (hipGetDevice(&cur) != hipSuccess)
        return PURO_ERR_HIP;
    int dev = cur;
    if (stream) {
        hipDevice_t d = 0;
        if (hipStreamGetDevice(stream, &d) != hipSuccess)
            return PURO_ERR_HIP;
        dev = (int)d;
    }
    if (dev < 0 || dev >= kMaxScratchDevices)
        return PURO_ERR_INTERNAL;
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (!g_scratch_ptr[dev]) {
        if (dev != cur && hipSetDevice(dev) != hipSuccess)
            return PURO_ERR_HIP;
        void *ptr = nullptr;
        const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (dev != cur && hipSetDevice(cur) != hipSuccess)
            return PURO_ERR_HIP;
        if (e != hipSuccess || !ptr)
            return PURO_ERR_HIP;
        g_scratch_ptr[dev] = ptr;
    }
    *out = g_scratch_ptr[dev];
    return PURO_OK;
}

puro_status_t puro_fp8_gemm_noalloc(puro_layout_t layout, int64_t M, int64_t N, int64_t K, const uint8_t *A,
                                    int64_t lda, const float *sA, const uint8_t *B, int64_t ldb, const float *sB,
                                    puro_bscale_t bgran, void *C, puro_dtype_t cdt, int64_t ldc, hipStream_t stream)
{
    try {
        puro_status_t st = check_gemm(layout, M, N, K, A, lda, sA, B, ldb, sB, bgran, C, cdt, ldc);
        if (st != PURO_OK)
            return st;
        puro::GemmProblem p = make_problem(layout, M, N, K, A, lda, sA, B, ldb, sB, bgran, C, cdt, ldc);
        // the same plan, kernels and partial-sum layout as puro_fp8_gemm; every
        // partial is written before it is read, so nothing is cleared
        const size_t need = puro::gemm_workspace_bytes(p);
        if (need > (size_t)PURO_NOALLOC_SCRATCH_BYTES)
            return PURO_ERR_WORKSPACE;
        if (M == 0 || N == 0)
            return PURO_OK;
        void *ws = nullptr;
        if (need > 0) {
            st = scratch_for_stream(stream, &ws);
            if (st != PURO_OK)
                return st;
        }
        return from_hip(puro::launch_gemm(p, ws, stream));
    } catch (...) {
        return PURO_ERR_INTERNAL;
    }
}

static bool mx_aligned(int64_t M, int64_t N, int64_t K)
{
    return M % 128 == 0 && N % 128 == 0 && K % 128 == 0 && K > 0;
}

size_t puro_fp8_gemm_mx_workspace_size(puro_layout_t layout, int64_t M, int64_t N, int64_t K, puro_bscale_t bgran)
{
    if (layout != PURO_NT && layout != PURO_NN && layout != PURO_TN)
        return 0;
    if (bgran != PURO_SCALE_1x128 && bgran != PURO_SCALE_128x128)
        return 0;
    if (bad_extent(M) || bad_extent(N) || bad_extent(K) || !mx_aligned(M, N, K))
        return 0;
    puro::GemmProblem p = make_problem(layout, M, N, K, nullptr, 0, nullptr, nullptr, 0, nullptr, bgran, nullptr,
                                       PURO_F32, N);
    return puro::gemm_mx_workspace_bytes(p);
}

puro_status_t puro_fp8_gemm_mx(puro_layout_t layout, int64_t M, int64_t N, int64_t K, const uint8_t *A,
                               int64_t lda, const float *sA, const uint8_t *B, int64_t ldb, const float *sB,
                               puro_bscale_t bgran, void *C, puro_dtype_t cdt, int64_t ldc, void *workspace,
                               size_t ws_bytes, hipStream_t stream)
{
    try {
        puro_status_t st = check_gemm(layout, M, N, K, A, lda, sA, B, ldb, sB, bgran, C, cdt, ldc);
        if (st != PURO_OK)
            return st;
        if (M == 0 || N == 0)
            return PURO_OK;
        if (!mx_aligned(M, N, K) || lda >= ((int64_t)1 << 28) || ldb >= ((int64_t)1 << 28))
            return PURO_ERR_SHAPE;
        puro::GemmProblem p = make_problem(layout, M, N, K, A, lda, sA, B, ldb, sB, bgran, C, cdt, ldc);
        const size_t need = puro::gemm_mx_workspace_bytes(p);
        if (need > 0 && (!workspace || ws_bytes < need || !aligned(workspace, 256)))
            return PURO_ERR_WORKSPACE;
        return from_hip(puro::launch_gemm_mx(p, workspace, stream));
    } catch (...) {
        return PURO_ERR_INTERNAL;
    }
}

size_t puro_fp8_gemm_native_workspace_size(puro_layout_t layout, int64_t M, int64_t N, int64_t K,
                                           puro_bscale_t bgran)
{
    if (layout != PURO_NT && layout != PURO_NN && layout != PURO_TN)
        return 0;
    if (bgran != PURO_SCALE_1x128 && bgran != PURO_SCALE_128x128)
        return 0;
    if (bad_extent(M) || bad_extent(N) || bad_extent(K) || !mx_aligned(M, N, K))
        return 0;
    puro::GemmProblem p = make_problem(layout, M, N, K, nullptr, 0, nullptr, nullptr, 0, nullptr, bgran, nullptr,
                                       PURO_F32, N);
    return puro::gemm_native_workspace_bytes(p);
}

puro_status_t puro_fp8_gemm_native(puro_layout_t layout, int64_t M, int64_t N, int64_t K, const uint8_t *A,
                                   int64_t lda, const float *sA, const uint8_t *B, int64_t ldb, const float *sB,
                                   puro_bscale_t bgran, void *C, puro_dtype_t cdt, int64_t ldc, void *workspace,
                                   size_t ws_bytes, hipStream_t stream)
{
    try {
        puro_status_t st = check_gemm(layout, M, N, K, A, lda, sA, B, ldb, sB, bgran, C, cdt, ldc);
        if (st != PURO_OK)
            return st;
        if (M == 0 || N == 0)
            return PURO_OK;
        if (!mx_aligned(M, N, K) || lda >= ((int64_t)1 << 28) || ldb >= ((int64_t)1 << 28))
            return PURO_ERR_SHAPE;
        puro::GemmProblem p = make_problem(layout, M, N, K, A, lda, sA, B, ldb, sB, bgran, C, cdt, ldc);
        const size_t need = puro::gemm_native_workspace_bytes(p);
        if (need > 0 && (!workspace || ws_bytes < need || !aligned(workspace, 256)))
            return PURO_ERR_WORKSPACE;
        return from_hip(puro::launch_gemm_native(p, workspace, stream));
    } catch (...) {
        return PURO_ERR_INTERNAL;
    }
}

// Datapaths of the grouped launcher.
enum GroupDp { GROUP_EXACT, GROUP_MX, GROUP_NATIVE };

static puro_status_t gemm_grouped_impl(GroupDp dp, puro_layout_t layout, puro_bscale_t bgran, puro_dtype_t cdt,
                                       const puro_gemm_desc_t *problems, int count, hipStream_t stream)
{
    try {
        if (count < 0 || count > 4096)
            return PURO_ERR_SHAPE;
        if (count > 0 && !problems)
            return PURO_ERR_NULL;
        std::vector<puro::GemmProblem> ps;
        ps.reserve((size_t)count);
        for (int i = 0; i < count; i++) {
            const puro_gemm_desc_t &d = problems[i];
            if (d.nseg < 1 || d.nseg > PURO_GEMM_MAX_SEGMENTS)
                return PURO_ERR_SHAPE;
            if (d.accumulate != 0 && d.accumulate != 1)
                return PURO_ERR_ENUM;
            puro::GemmProblem p = make_problem(layout, d.M, d.N, 0, nullptr, 0, nullptr, nullptr, 0, nullptr,
                                               bgran, d.C, cdt, d.ldc);
            for (int j = 0; j < d.nseg; j++) {
                const puro_gemm_segment_t &g = d.seg[j];
                const puro_status_t st = check_gemm(layout, d.M, d.N, g.K, g.A, g.lda, g.sA, g.B, g.ldb, g.sB,
                                                    bgran, d.C, cdt, d.ldc);
                if (st != PURO_OK)
                    return st;
                // the FP8-matrix-core datapaths take aligned, non-empty products only
                if (dp != GROUP_EXACT && d.M > 0 && d.N > 0 &&
                    (!mx_aligned(d.M, d.N, g.K) || g.lda >= ((int64_t)1 << 28) || g.ldb >= ((int64_t)1 << 28)))
                    return PURO_ERR_SHAPE;
                p.seg[j] = puro::GemmSegment{g.K, g.A, g.lda, g.sA, g.B, g.ldb, g.sB};
            }
            p.nseg = d.nseg;
            p.accumulate = d.accumulate == 1;
            ps.push_back(p);
        }
        if (layout != PURO_NT && layout != PURO_NN && layout != PURO_TN)
            return PURO_ERR_ENUM;
        if (bgran != PURO_SCALE_1x128 && bgran != PURO_SCALE_128x128)
            return PURO_ERR_ENUM;
        if (cdt != PURO_F32 && cdt != PURO_BF16)
            return PURO_ERR_ENUM;
        if (ps.empty())
            return PURO_OK;
        switch (dp) {
        case GROUP_MX: return from_hip(puro::launch_gemm_group_mx(ps.data(), (int)ps.size(), stream));
        case GROUP_NATIVE: return from_hip(puro::launch_gemm_group_native(ps.data(), (int)ps.size(), stream));
        default: return from_hip(puro::launch_gemm_group(ps.data(), (int)ps.size(), stream));
        }
    } catch (...) {
        return PURO_ERR_INTERNAL;
    }
}

puro_status_t puro_fp8_gemm_grouped(puro_layout_t layout, puro_bscale_t bgran, puro_dtype_t cdt,
                                    const puro_gemm_desc_t *problems, int count, hipStream_t stream)
{
    return gemm_grouped_impl(GROUP_EXACT, layout, bgran, cdt, problems, count, stream);
}

puro_status_t puro_fp8_gemm_grouped_mx(puro_layout_t layout, puro_bscale_t bgran, puro_dtype_t cdt,
                                       const puro_gemm_desc_t *problems, int count, hipStream_t stream)
{
    return gemm_grouped_impl(GROUP_MX, layout, bgran, cdt, problems, count, stream);
}

puro_status_t puro_fp8_gemm_grouped_native(puro_layout_t layout, puro_bscale_t bgran, puro_dtype_t cdt,
                                           const puro_gemm_desc_t *problems, int count, hipStream_t stream)
{
    return gemm_grouped_impl(GROUP_NATIVE, layout, bgran, cdt, problems, count, stream);
}

const char *puro_status_string(puro_status_t status)
{
    switch (status) {
    case PURO_OK: return "success";
    case PURO_ERR_NULL: return "a required pointer is NULL";
    case PURO_ERR_SHAPE: return "invalid extent or leading dimension";
    case PURO_ERR_ALIGN: return "misaligned pointer or leading dimension";
    case PURO_ERR_ENUM: return "unknown enumeration value";
    case PURO_ERR_WORKSPACE: return "workspace missing, too small or misaligned";
    case PURO_ERR_HIP: return "HIP runtime error at launch";
    case PURO_ERR_INTERNAL: return "internal error";
    }
    return "unknown status";
}

int puro_fp8_version(void)
{
    return 100;
}

} // extern "C"
