// Internal launchers (host side).  Arguments are validated by the C-ABI layer
// before any of these is called.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>

namespace puro {

// pow2: power-of-two block scales (the scaled matrix cores' E8M0 variant)
// instead of amax / 448.
hipError_t launch_quant_act(const void *x, bool bf16, int64_t rows, int64_t cols, int64_t ldx,
                            uint8_t *q, int64_t ldq, float *s, bool pow2, hipStream_t st);
hipError_t launch_quant_weight(const void *w, bool bf16, int64_t rows, int64_t cols, int64_t ldw,
                               uint8_t *q, int64_t ldq, float *s, bool pow2, hipStream_t st);
// One weight of a grouped weight quantisation (as launch_quant_weight's
// arguments; cb = number of 128-column tiles).
struct QuantWeightItem {
    const void *w;
    int64_t rows, cols, ldw;
    uint8_t *q;
    int64_t ldq;
    float *s;
    int64_t cb;        // ceil(cols / 128)
    uint8_t *qt;       // transposed codes [cols][rows] (row stride ldqt), or NULL
    int64_t ldqt;
    float *st;         // transposed scales [cb][rb], dense (with qt)
    int64_t rb;        // ceil(rows / 128)
};
constexpr int kQuantGroupMax = 16;   // weights per launch; more take several launches
hipError_t launch_quant_weight_group(const QuantWeightItem *items, int count, bool bf16, bool pow2,
                                     hipStream_t st);
hipError_t launch_quant_transpose(const void *x, bool bf16, int64_t tokens, int64_t cols,
                                  int64_t ldx, bool transpose_out, uint8_t *q, int64_t ldq,
                                  float *s, bool pow2, hipStream_t st);
hipError_t launch_quant_dual(const void *x, bool bf16, int64_t tokens, int64_t cols, int64_t ldx,
                             uint8_t *qr, int64_t ldqr, float *sr, bool transpose_out, uint8_t *qt,
                             int64_t ldqt, float *st, bool pow2, hipStream_t stream);

// Dual quantiser of h = BF16(silu(g) * u), g and u BF16 [tokens][cols]; h is
// also stored unless NULL.
hipError_t launch_swiglu_dual(const uint16_t *g, int64_t ldg, const uint16_t *u, int64_t ldu, uint16_t *h,
                              int64_t ldh, int64_t tokens, int64_t cols, uint8_t *qr, int64_t ldqr, float *sr,
                              bool transpose_out, uint8_t *qt, int64_t ldqt, float *st, bool pow2,
                              hipStream_t stream);

constexpr int kGemmMaxSeg = 4;

// One K segment of a product: A, B and their block scales over K indices 0 .. K-1.
struct GemmSegment {
    int64_t K;
    const uint8_t *A;
    int64_t lda;
    const float *sA;
    const uint8_t *B;
    int64_t ldb;
    const float *sB;
};

// C (+)= sum over segments of the blockwise product; the segments share M, N
// and the output.
struct GemmProblem {
    int layout;   // 0 NT, 1 NN, 2 TN
    int bgran;    // 0 1x128, 1 128x128
    bool c_bf16;  // output dtype
    bool accumulate;
    int64_t M, N;
    int nseg;
    GemmSegment seg[kGemmMaxSeg];
    void *C;
    int64_t ldc;
};

// Single-segment, overwriting problems (accumulate and extra segments are the
// grouped launcher's).
size_t gemm_workspace_bytes(const GemmProblem &p);
hipError_t launch_gemm(const GemmProblem &p, void *workspace, hipStream_t st);
// Scaled-matrix-core variant: power-of-two scales, M, N, K multiples of 128.
size_t gemm_mx_workspace_bytes(const GemmProblem &p);
hipError_t launch_gemm_mx(const GemmProblem &p, void *workspace, hipStream_t st);
// Native FP8 matrix-core variant: amax/448 scales as in launch_gemm, block
// partials on the FP8 matrix cores (not FP32-exact), M, N, K multiples of 128.
size_t gemm_native_workspace_bytes(const GemmProblem &p);
hipError_t launch_gemm_native(const GemmProblem &p, void *workspace, hipStream_t st);
// Independent problems sharing layout, B-scale granularity and output dtype;
// needs no workspace.
hipError_t launch_gemm_group(const GemmProblem *probs, int count, hipStream_t st);
// The same on the scaled (MX) and on the native FP8 datapaths: aligned
// problems only (M, N and every segment's K multiples of 128).
hipError_t launch_gemm_group_mx(const GemmProblem *probs, int count, hipStream_t st);
hipError_t launch_gemm_group_native(const GemmProblem *probs, int count, hipStream_t st);

} // namespace puro
