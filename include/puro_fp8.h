/*
 * puro_fp8.h -- blockwise E4M3 FP8 quantise-and-GEMM for gfx950 (MI355X).
 *
 * The operation.  The Puro-2B-Base model card (friendli.ai and alphaneural.io
 * copies; training-setup paragraph under the Phase 1 / Phase 2 table) states
 * that the main Transformer linear-layer GEMMs of the recipe run in blockwise
 * E4M3 FP8, while numerically sensitive operations, master weights and
 * optimizer states stay in BF16 or FP32.  The Puro-2B technical report (part
 * 7/7, related-work paragraph on low-precision training) places this in the
 * DeepSeek-V3 line of FP8 mixed-precision training and cites the FP8-formats
 * paper, whose E4M3 encoding is used here (OCP E4M3FN: bias 7, largest finite
 * 448, S.1111.111 = NaN, no infinities).  The pages give neither block shapes
 * nor a scale rule; this library uses:
 *   - activations and gradients: 1x128 blocks along the contraction dimension;
 *   - weights: 128x128 tiles;
 *   - per block: s = fl32(amax / 448), q = E4M3(fl32(x / s)) with round to
 *     nearest even and saturation at +-448; a block whose s is 0 stores s = 0
 *     and codes 0x00 / 0x80 (by sign);
 *   - GEMM: for every 128-wide K block, the FP8 x FP8 block dot product is
 *     formed on the matrix cores and promoted into FP32 accumulators as
 *     acc += (sA * sB) * partial; the result is stored as FP32 or BF16 (RNE).
 * Extents need not be multiples of 128: the last block along an extent then
 * holds the remaining elements, and its scale is taken over those only.
 *
 * Conventions shared by every call.
 *   - All tensors are row-major.  Every tensor pointer (x, w, q, A, B, C) is a
 *     DEVICE pointer owned by the caller and must be 16-byte aligned; every
 *     leading dimension (ld*) is in elements, must be >= the row length and a
 *     multiple of 16.  Scale pointers are DEVICE pointers to dense FP32 arrays,
 *     4-byte aligned.  A pointer may be NULL only when its tensor is empty.
 *   - Arguments are validated on the host, synchronously, before anything is
 *     enqueued; a failed validation returns an error and enqueues nothing.
 *   - On success the work is enqueued on `stream` (NULL = the null stream) and
 *     the call returns without synchronising.  Results are defined once the
 *     stream reaches that point.
 *   - Every extent and leading dimension is at most 2^23 (8,388,608), else
 *     PURO_ERR_SHAPE.
 *   - The library allocates nothing and keeps no per-call state; calls are
 *     reentrant.  No C++ exception crosses this interface.
 *   - Inputs must be finite; results for NaN or Inf inputs are unspecified.
 *   - Outputs must not overlap inputs.
 */
#ifndef PURO_FP8_H
#define PURO_FP8_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    PURO_OK = 0,
    PURO_ERR_NULL = 1,      /* a required pointer is NULL                        */
    PURO_ERR_SHAPE = 2,     /* negative extent, or leading dimension < row length */
    PURO_ERR_ALIGN = 3,     /* misaligned pointer or leading dimension             */
    PURO_ERR_ENUM = 4,      /* unknown dtype / layout / granularity value          */
    PURO_ERR_WORKSPACE = 5, /* workspace missing or smaller than required          */
    PURO_ERR_HIP = 6,       /* the HIP runtime reported an error at launch         */
    PURO_ERR_INTERNAL = 7   /* unexpected internal failure                         */
} puro_status_t;

typedef enum { PURO_F32 = 0, PURO_BF16 = 1 } puro_dtype_t;

/* Operand orientation of puro_fp8_gemm; C is always [M][N], contraction over K. */
typedef enum {
    PURO_NT = 0, /* A [M][K], B [N][K]  -- forward Y = X W^T; weight gradient on token-transposed copies */
    PURO_NN = 1, /* A [M][K], B [K][N]  -- data gradient dX = dY W with the forward's quantised W        */
    PURO_TN = 2  /* A [K][M], B [K][N]  -- weight gradient dW = dY^T X on untransposed token-blocked copies */
} puro_layout_t;

/* Block shape of B's scales; A's scales are always 1x128 along K. */
typedef enum { PURO_SCALE_1x128 = 0, PURO_SCALE_128x128 = 1 } puro_bscale_t;

/*
 * Activation / gradient quantiser (1x128 along each row).
 * Passage: Puro-2B-Base model card (friendli.ai), training-setup paragraph
 * under the Phase 1 / Phase 2 table -- the main linear-layer GEMMs run in
 * blockwise E4M3, so each GEMM's activation and gradient operands are
 * quantised to E4M3 with per-block scales before the product.
 *   x   [rows][cols], FP32 or BF16 (xdt), row stride ldx
 *   q   [rows][cols] E4M3 codes, row stride ldq
 *   s   [rows][ceil(cols/128)] FP32, dense
 * Block (r, b) is x[r][128b .. min(cols, 128b+128)).
 * Used for the forward input X of every linear layer and for the incoming
 * gradient dY of the data-gradient GEMM (blocked along the output features).
 */
puro_status_t puro_fp8_quant_act(const void *x, puro_dtype_t xdt, int64_t rows, int64_t cols,
                                 int64_t ldx, uint8_t *q, int64_t ldq, float *s,
                                 hipStream_t stream);

/*
 * Weight quantiser (128x128 tiles).
 * Passage: the same setup paragraph -- master weights stay in BF16 or FP32,
 * and the main GEMMs that read them run in blockwise E4M3, so each GEMM takes
 * an E4M3 copy of its FP32 (or BF16) master weight.
 *   w   [rows][cols], FP32 or BF16 (wdt) master weight, row stride ldw
 *   q   [rows][cols] E4M3 codes, row stride ldq
 *   s   [ceil(rows/128)][ceil(cols/128)] FP32, dense
 * One scale per tile; the same codes and scales serve the forward GEMM (NT,
 * B = W [N_out][K_in]) and the data-gradient GEMM (NN, B = W read as [K][N]).
 */
puro_status_t puro_fp8_quant_weight(const void *w, puro_dtype_t wdt, int64_t rows, int64_t cols,
                                    int64_t ldw, uint8_t *q, int64_t ldq, float *s,
                                    hipStream_t stream);

/*
 * Grouped weight quantiser: `count` weights, each exactly as in
 * puro_fp8_quant_weight (same codes, scales and layouts), in as few launches
 * as possible.  Their tiles run side by side, which fills the GPU where one
 * weight alone does not: e.g. all projections of a layer, or every weight of a
 * model after an optimizer step, at once.
 *   wdt    element type of every weight (FP32 or BF16)
 *   items  HOST array of `count` descriptors, read before the call returns
 *   count  0 .. PURO_QUANT_MAX_GROUP (0: nothing is enqueued; more: PURO_ERR_SHAPE)
 * Every item is validated as a puro_fp8_quant_weight call before anything is
 * enqueued, and the first failing item's status is returned.  No output may
 * overlap another item's output or any input.
 * With qt not NULL an item also gets its codes and scales transposed (qt, st;
 * validated like q and s, with rows and cols swapped): the B operand of the
 * data-gradient product dX = dY W in NT form, read by the matrix cores in the
 * same K-contiguous order as the forward's.  qt = NULL: no transposed copy
 * (ldqt and st are ignored).
 */
#define PURO_QUANT_MAX_GROUP 4096
typedef struct {
    const void *w;            /* [rows][cols], row stride ldw */
    int64_t rows, cols, ldw;
    uint8_t *q;               /* [rows][cols] codes, row stride ldq */
    int64_t ldq;
    float *s;                 /* [ceil(rows/128)][ceil(cols/128)], dense */
    uint8_t *qt;              /* NULL, or the same codes transposed: [cols][rows], row stride ldqt */
    int64_t ldqt;
    float *st;                /* with qt: the scales transposed, [ceil(cols/128)][ceil(rows/128)], dense */
} puro_quant_weight_desc_t;
puro_status_t puro_fp8_quant_weight_grouped(puro_dtype_t wdt, const puro_quant_weight_desc_t *items,
                                            int count, hipStream_t stream);

/*
 * Passage: the same setup paragraph (the blockwise E4M3 GEMMs include the
 * backward ones) and the technical report's related-work paragraph on FP8
 * mixed precision (part 7/7): the weight-gradient product contracts over the
 * tokens, so its operands dY and X are blocked along the tokens.
 * Token-dimension quantiser for the weight-gradient GEMM: blocks are 128
 * consecutive tokens of one column of x [tokens][cols] (FP32 or BF16, stride ldx).
 *   transpose_out = 1: q [cols][tokens] (stride ldq), s [cols][ceil(tokens/128)]
 *                      -- operands of an NT weight-gradient GEMM
 *   transpose_out = 0: q [tokens][cols] (stride ldq), s [ceil(tokens/128)][cols]
 *                      -- operands of a TN weight-gradient GEMM
 * Both modes produce the same codes and scales, laid out differently.
 * Any other transpose_out value returns PURO_ERR_ENUM.
 */
puro_status_t puro_fp8_quant_transpose(const void *x, puro_dtype_t xdt, int64_t tokens,
                                       int64_t cols, int64_t ldx, int transpose_out, uint8_t *q,
                                       int64_t ldq, float *s, hipStream_t stream);

/*
 * Dual quantiser: one read of x [tokens][cols] (FP32 or BF16, stride ldx)
 * produces both copies a linear layer needs of its input X (or of its output
 * gradient dY), with exactly the codes and scales of the two separate calls:
 *   q_row [tokens][cols] (stride ldq_row), s_row [tokens][ceil(cols/128)]
 *        -- as puro_fp8_quant_act (1x128 blocks along each row);
 *   q_tok, s_tok -- as puro_fp8_quant_transpose with the same transpose_out
 *        (128-token blocks of each column).
 * Reading the BF16 input once instead of twice is the saving.  The two output
 * pairs must not overlap each other or x.
 */
puro_status_t puro_fp8_quant_dual(const void *x, puro_dtype_t xdt, int64_t tokens, int64_t cols,
                                  int64_t ldx, uint8_t *q_row, int64_t ldq_row, float *s_row,
                                  int transpose_out, uint8_t *q_tok, int64_t ldq_tok, float *s_tok,
                                  hipStream_t stream);

/*
 * Gated activation fused into the dual quantiser: the down projection's input.
 * The model card's configuration table names the Qwen3-1.7B configuration,
 * whose feed-forward block multiplies the up projection's output by SiLU of
 * the gate projection's (SwiGLU with Swish parameter 1; the pages do not state
 * the activation, this is the reading taken).  For g = gate[t][c] and
 * u = up[t][c] (BF16, [tokens][cols], strides ldg and ldu; the two may be the
 * halves of one [tokens][2 cols] product):
 *     h[t][c] = BF16_RNE( silu(g) * u ),   silu(g) = g / (1 + e^-g).
 * silu(g) * u is evaluated in FP32 before the one BF16 rounding, within
 * 2^-20 |silu(g) u| + 2^-149 (|g u| + 1) of the exact value (the second term
 * only matters where sigmoid(g) is below FP32's normal range, g < -87.3).
 * h is stored (BF16 [tokens][cols], stride ldh) unless h is NULL.  Either way
 * q_row/s_row and q_tok/s_tok are exactly what puro_fp8_quant_dual writes for
 * that h tensor with the same transpose_out.  |g u| must be finite in FP32.
 * Every output must be disjoint from gate and up and from each other.
 * Errors as puro_fp8_quant_dual; when h is not NULL, ldh is checked like any
 * leading dimension and h must be 16-byte aligned.
 */
puro_status_t puro_fp8_swiglu_quant_dual(const void *gate, int64_t ldg, const void *up, int64_t ldu,
                                         int64_t tokens, int64_t cols, void *h, int64_t ldh, uint8_t *q_row,
                                         int64_t ldq_row, float *s_row, int transpose_out, uint8_t *q_tok,
                                         int64_t ldq_tok, float *s_tok, hipStream_t stream);

/*
 * Workspace bytes puro_fp8_gemm needs for this problem (0 = none).  Returns 0
 * for invalid arguments as well; puro_fp8_gemm reports those.
 */
size_t puro_fp8_gemm_workspace_size(puro_layout_t layout, int64_t M, int64_t N, int64_t K,
                                    puro_bscale_t bgran);

/*
 * Blockwise-scaled FP8 GEMM.
 * Passage: the setup paragraph (main linear-layer GEMMs in blockwise E4M3,
 * FP32 kept where needed) and the related-work paragraph's DeepSeek-V3 design
 * (FP8 block products promoted into FP32 accumulators):
 *   C[m][n] = sum_kb sA(m,kb) * sB(n,kb) * sum_{k in block kb} a(m,k) b(k,n)
 * with a, b the E4M3 values of A and B, kb over the ceil(K/128) blocks of K.
 * Storage (KB = ceil(K/128), NB = ceil(N/128)); scales are dense and indexed
 * in the operand's storage orientation:
 *   layout   A        sA         B        sB (1x128)  sB (128x128)
 *   NT       [M][K]   [M][KB]    [N][K]   [N][KB]     [NB][KB]
 *   NN       [M][K]   [M][KB]    [K][N]   [KB][N]     [KB][NB]
 *   TN       [K][M]   [KB][M]    [K][N]   [KB][N]     [KB][NB]
 * C [M][N] (row stride ldc) is written as FP32 or BF16 (cdt, round to nearest
 * even); it is overwritten, not accumulated into.  K = 0 writes zeros.
 * workspace may be NULL when puro_fp8_gemm_workspace_size returns 0;
 * otherwise it must hold at least that many bytes (device memory, 256-byte
 * aligned) and must not be used by other work in flight on other streams.
 */
puro_status_t puro_fp8_gemm(puro_layout_t layout, int64_t M, int64_t N, int64_t K,
                            const uint8_t *A, int64_t lda, const float *sA, const uint8_t *B,
                            int64_t ldb, const float *sB, puro_bscale_t bgran, void *C,
                            puro_dtype_t cdt, int64_t ldc, void *workspace, size_t ws_bytes,
                            hipStream_t stream);

/*
 * One K segment of a grouped-GEMM problem: A, B and their scales over the
 * segment's own K indices 0 .. K-1, with the storage, scale layout and rules
 * of puro_fp8_gemm's A, lda, sA, B, ldb, sB for (M, N, K).
 */
typedef struct {
    int64_t K;
    const uint8_t *A;
    int64_t lda;
    const float *sA;
    const uint8_t *B;
    int64_t ldb;
    const float *sB;
} puro_gemm_segment_t;

#define PURO_GEMM_MAX_SEGMENTS 4

/*
 * One problem of a grouped GEMM:
 *   C = sum over s < nseg of A_s B_s           (accumulate = 0)
 *   C = C + sum over s < nseg of A_s B_s       (accumulate = 1)
 * where each A_s B_s is the blockwise product of puro_fp8_gemm (blocks of
 * 128 along each segment's own K).  The sum and the addition of the old C
 * happen in FP32 and C is rounded once.  Several segments sum the partial
 * products of one output (the data gradient of the q, k and v projections,
 * dX = dY_q W_q + dY_k W_k + dY_v W_v, in one pass); accumulate adds into
 * an existing output (weight gradients summed over micro-batches).  With
 * accumulate = 1, C is read: it must hold finite values.
 *   nseg        1 .. PURO_GEMM_MAX_SEGMENTS; seg[nseg ..] are ignored.
 */
typedef struct {
    int64_t M, N;
    int nseg;
    int accumulate;
    puro_gemm_segment_t seg[PURO_GEMM_MAX_SEGMENTS];
    void *C;
    int64_t ldc;
} puro_gemm_desc_t;

/*
 * Grouped GEMM: `count` independent problems that share layout, B-scale
 * granularity and output dtype, in as few launches as possible (the
 * problems' tiles run side by side, which fills the GPU where single small
 * problems cannot -- e.g. the q, k and v projections of one input, or all
 * weight gradients of a layer).
 *   problems  HOST array of `count` descriptors, read before the call returns;
 *             the device buffers they point to follow the rules of
 *             puro_fp8_gemm.  No output may overlap another problem's output
 *             or any input.
 *   count     0 .. 4096 (0: nothing is enqueued).
 * Needs no workspace.  Every problem is validated before anything is
 * enqueued and the first failing problem's status is returned: nseg outside
 * 1 .. PURO_GEMM_MAX_SEGMENTS is PURO_ERR_SHAPE, accumulate other than 0 or 1
 * is PURO_ERR_ENUM, and every segment is checked as a puro_fp8_gemm call.
 */
puro_status_t puro_fp8_gemm_grouped(puro_layout_t layout, puro_bscale_t bgran, puro_dtype_t cdt,
                                    const puro_gemm_desc_t *problems, int count, hipStream_t stream);

/*
 * Power-of-two scale variant (for the scaled FP8 matrix cores).
 *
 * Not the recipe: the pages give no scale rule, and the recipe's reading
 * (s = amax / 448) is what the calls above implement.  gfx950's scaled MFMA
 * takes one E8M0 scale (a power of two) per 32 K values of each row of A and
 * column of B, applies it inside the matrix core and accumulates across K
 * blocks without a separate promotion step, on E4M3 codes as they are.  With
 * power-of-two block scales the same 1x128 / 128x128 blocks map onto it.
 *
 * The _pow2 quantisers take the arguments of their counterparts above and
 * write the same layouts; per block the scale is the smallest power of two
 * s = 2^k with 448 s >= amax (k limited to [-127, 127]; a zero block gets
 * 2^-127) and q = E4M3(x / s), where x / s is exact.
 */
puro_status_t puro_fp8_quant_act_pow2(const void *x, puro_dtype_t xdt, int64_t rows, int64_t cols, int64_t ldx,
                                      uint8_t *q, int64_t ldq, float *s, hipStream_t stream);
puro_status_t puro_fp8_quant_weight_pow2(const void *w, puro_dtype_t wdt, int64_t rows, int64_t cols,
                                         int64_t ldw, uint8_t *q, int64_t ldq, float *s, hipStream_t stream);
puro_status_t puro_fp8_quant_weight_grouped_pow2(puro_dtype_t wdt, const puro_quant_weight_desc_t *items,
                                                 int count, hipStream_t stream);
puro_status_t puro_fp8_quant_transpose_pow2(const void *x, puro_dtype_t xdt, int64_t tokens, int64_t cols,
                                            int64_t ldx, int transpose_out, uint8_t *q, int64_t ldq, float *s,
                                            hipStream_t stream);
puro_status_t puro_fp8_quant_dual_pow2(const void *x, puro_dtype_t xdt, int64_t tokens, int64_t cols,
                                       int64_t ldx, uint8_t *q_row, int64_t ldq_row, float *s_row,
                                       int transpose_out, uint8_t *q_tok, int64_t ldq_tok, float *s_tok,
                                       hipStream_t stream);
puro_status_t puro_fp8_swiglu_quant_dual_pow2(const void *gate, int64_t ldg, const void *up, int64_t ldu,
                                              int64_t tokens, int64_t cols, void *h, int64_t ldh,
                                              uint8_t *q_row, int64_t ldq_row, float *s_row, int transpose_out,
                                              uint8_t *q_tok, int64_t ldq_tok, float *s_tok, hipStream_t stream);

/*
 * GEMM on the scaled FP8 matrix cores: arguments, storage and result
 * definition of puro_fp8_gemm, with two differences.
 *   - sA and sB must hold powers of two in [2^-127, 2^127] (as written by the
 *     _pow2 quantisers): only their exponents reach the matrix cores, so any
 *     other value gives wrong results.
 *   - M, N and K must be multiples of 128, and lda and ldb below 2^28 (else
 *     PURO_ERR_SHAPE; empty products are allowed and do nothing).
 * Precision: the FP8 matrix cores add each run of 8 consecutive products in
 * fixed point, dropping bits more than about 13 binary places below the
 * run's largest product (measured on gfx950), so the result is not FP32-exact
 * per block: the relative error is of order 1e-5 to 1e-4, against 2e-6 for
 * puro_fp8_gemm.  workspace as for puro_fp8_gemm, sized by
 * puro_fp8_gemm_mx_workspace_size (0 for invalid arguments).
 */
size_t puro_fp8_gemm_mx_workspace_size(puro_layout_t layout, int64_t M, int64_t N, int64_t K,
                                       puro_bscale_t bgran);
puro_status_t puro_fp8_gemm_mx(puro_layout_t layout, int64_t M, int64_t N, int64_t K, const uint8_t *A,
                               int64_t lda, const float *sA, const uint8_t *B, int64_t ldb, const float *sB,
                               puro_bscale_t bgran, void *C, puro_dtype_t cdt, int64_t ldc, void *workspace,
                               size_t ws_bytes, hipStream_t stream);

/*
 * GEMM with the block partials formed on the native FP8 matrix cores: the
 * arguments, storage, scales (amax / 448, as written by the quantisers
 * above) and result definition of puro_fp8_gemm, computed the way the
 * DeepSeek-V3 design that the Puro-2B report's related-work paragraph cites
 * computes it -- each 128-wide K block's E4M3 x E4M3 partial on the FP8
 * matrix cores, promoted into FP32 accumulators as acc += (sA * sB) * partial.
 * Differences from puro_fp8_gemm:
 *   - M, N and K must be multiples of 128, and lda and ldb below 2^28 (else
 *     PURO_ERR_SHAPE; empty products are allowed and do nothing).
 *   - Precision: the FP8 matrix cores add each run of 8 consecutive products
 *     in fixed point, dropping bits more than about 13 binary places below the
 *     run's largest product (measured on gfx950), so a block partial is not
 *     FP32-exact.  Per element |C - C_exact| <= 2^-9 C_abs + (4 KB + 4)
 *     2^-23 C_abs (C_abs: the blockwise product of |A| and |B|; KB = K / 128;
 *     plus one BF16 rounding for BF16 output), the bound the power-of-two
 *     variant is held to; the relative Frobenius error is of order 1e-5,
 *     against 2e-6 for puro_fp8_gemm.
 *     Twice the matrix-core peak of puro_fp8_gemm's FP16 datapath.
 * workspace as for puro_fp8_gemm, sized by puro_fp8_gemm_native_workspace_size
 * (0 for invalid arguments).
 */
size_t puro_fp8_gemm_native_workspace_size(puro_layout_t layout, int64_t M, int64_t N, int64_t K,
                                           puro_bscale_t bgran);
puro_status_t puro_fp8_gemm_native(puro_layout_t layout, int64_t M, int64_t N, int64_t K, const uint8_t *A,
                                   int64_t lda, const float *sA, const uint8_t *B, int64_t ldb, const float *sB,
                                   puro_bscale_t bgran, void *C, puro_dtype_t cdt, int64_t ldc, void *workspace,
                                   size_t ws_bytes, hipStream_t stream);

/*
 * Grouped GEMMs on the two FP8-matrix-core datapaths: puro_fp8_gemm_grouped's
 * arguments, descriptors, segment sums, accumulate-into outputs and
 * validation, with every product computed as by puro_fp8_gemm_mx (power-of-two
 * scales applied by the scaled MFMA) or by puro_fp8_gemm_native (amax / 448
 * scales, FP8 block partials promoted in FP32), and with their precision.
 * Passage: the setup paragraph of the model card (the main linear-layer GEMMs,
 * backward ones included, in blockwise E4M3) and the DeepSeek-V3 design that
 * the technical report's related-work paragraph cites; grouping is how one
 * layer's seven weight gradients fill the GPU.
 * Additionally, every non-empty problem needs M, N and each segment's K to be
 * positive multiples of 128 and lda, ldb below 2^28 (else PURO_ERR_SHAPE,
 * before anything is enqueued).  Needs no workspace.
 */
puro_status_t puro_fp8_gemm_grouped_mx(puro_layout_t layout, puro_bscale_t bgran, puro_dtype_t cdt,
                                       const puro_gemm_desc_t *problems, int count, hipStream_t stream);
puro_status_t puro_fp8_gemm_grouped_native(puro_layout_t layout, puro_bscale_t bgran, puro_dtype_t cdt,
                                           const puro_gemm_desc_t *problems, int count, hipStream_t stream);

/*
 * puro_fp8_gemm without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  Arguments, validation, result and
 * kernels are those of puro_fp8_gemm; the split-K partial sums go to a fixed
 * device array of PURO_NOALLOC_SCRATCH_BYTES that the library holds on each
 * GPU it runs on until the process ends.  The call allocates nothing (no
 * hipMalloc, hipFree or allocating library routine).
 *   - A problem whose plan needs more than PURO_NOALLOC_SCRATCH_BYTES
 *     (puro_fp8_gemm_workspace_size above it) returns PURO_ERR_WORKSPACE
 *     before anything is enqueued.
 *   - All calls on one GPU share that GPU's array: calls that may overlap in
 *     time on one GPU (other streams, other host threads) race on it and give
 *     undefined results.  Calls in one stream's order are safe.
 */
#define PURO_NOALLOC_SCRATCH_BYTES (64u << 20)
puro_status_t puro_fp8_gemm_noalloc(puro_layout_t layout, int64_t M, int64_t N, int64_t K, const uint8_t *A,
                                    int64_t lda, const float *sA, const uint8_t *B, int64_t ldb, const float *sB,
                                    puro_bscale_t bgran, void *C, puro_dtype_t cdt, int64_t ldc,
                                    hipStream_t stream);

/* Static, NUL-terminated description of a status code. */
const char *puro_status_string(puro_status_t status);

/* Library version as MAJOR*10000 + MINOR*100 + PATCH. */
int puro_fp8_version(void);

#ifdef __cplusplus
}
#endif

#endif /* PURO_FP8_H */
