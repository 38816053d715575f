/*
 * ORACLE for blockwise E4M3 FP8 quantise-and-GEMM.  TEST INFRASTRUCTURE ONLY.
 *
 * This file is the plain, slow, obviously-correct CPU statement of what the
 * library under blockwise_fp8_gemm_amd/ computes.  Only the tests, the smoke
 * check and the CPU-baseline leg of the benchmark may load it.  It shares no
 * code, header, table or constant with the HIP library, and the HIP library
 * never calls it.
 *
 * What it follows:
 *  - Puro-2B-Base model card (friendli.ai and alphaneural.io copies), the
 *    training-setup paragraph under the Phase 1 / Phase 2 table: the main
 *    Transformer linear-layer GEMMs run in blockwise E4M3 FP8, while master
 *    weights, optimizer states and sensitive operations stay in BF16/FP32.
 *  - Puro-2B technical report, part 7/7, related-work paragraph on low
 *    precision training: FP8 mixed precision in the style of DeepSeek-V3,
 *    citing the FP8-formats paper (Micikevicius et al., 2022) whose E4M3
 *    definition is used here: bias 7, 3 mantissa bits, no infinities,
 *    S.1111.111 is NaN, largest finite 448.
 *  The pages fix neither block shapes nor the scale rule.  The readings taken
 *  (1x128 activation/gradient blocks along the contraction dimension, 128x128
 *  weight tiles, scale = amax/448 in FP32, q = RNE_E4M3(fl32(x/s)) with
 *  saturation, zero blocks give scale 0 and signed-zero codes, FP64 exact
 *  per-block dot products) are listed with their reasons in the design notes
 *  at the repository root.
 *
 * Build: gcc -O2 -fopenmp -ffp-contract=off -fPIC -shared (no -ffast-math:
 * IEEE binary32 division with round-to-nearest-even and subnormals kept).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

/* ------------------------------------------------------------------------ */
/* E4M3 (FP8-formats paper, E4M3 column of its format table)                 */
/* ------------------------------------------------------------------------ */

/* Value of a code, straight from the format definition.  NaN for S.1111.111. */
double ref_e4m3_decode(uint8_t c)
{
    int sign = c >> 7;
    int e = (c >> 3) & 15;
    int f = c & 7;
    double v;
    if (e == 15 && f == 7)
        return NAN;
    if (e == 0)
        v = ldexp((double)f, -9);               /* subnormal: f/8 * 2^(1-7) */
    else
        v = ldexp(1.0 + f / 8.0, e - 7);        /* normal: 1.f * 2^(e-7)    */
    return sign ? -v : v;
}

/* Non-negative finite values in code order (code order is value order). */
static double g_pos[127];
static int g_pos_ready = 0;

static void ref_init_table(void)
{
    if (g_pos_ready)
        return;
    for (int c = 0; c < 127; c++)
        g_pos[c] = ref_e4m3_decode((uint8_t)c);
    g_pos_ready = 1;
}

/*
 * Encode y: the finite E4M3 value nearest to y, ties to the code with an even
 * mantissa LSB; magnitudes at or above 448 saturate to 448.  The sign bit is
 * kept, so -0 and negative values that round to zero give 0x80.  NaN input is
 * outside the contract (finite inputs only).
 */
uint8_t ref_e4m3_encode(float y)
{
    ref_init_table();
    uint8_t sign = signbit(y) ? 0x80 : 0x00;
    double m = fabs((double)y);
    if (m >= 448.0)
        return sign | 0x7E;
    /* largest code lo with value(lo) <= m (value(0) = 0 <= m always) */
    int lo = 0, hi = 0x7E;
    while (lo < hi) {
        int mid = (lo + hi + 1) / 2;
        if (g_pos[mid] <= m)
            lo = mid;
        else
            hi = mid - 1;
    }
    double below = m - g_pos[lo];        /* both exact in double */
    double above = g_pos[lo + 1] - m;
    int c;
    if (below < above)
        c = lo;
    else if (above < below)
        c = lo + 1;
    else
        c = (lo & 1) ? lo + 1 : lo;      /* tie: even mantissa LSB */
    return sign | (uint8_t)c;
}

void ref_e4m3_encode_array(const float *y, int64_t n, uint8_t *out)
{
    ref_init_table();
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; i++)
        out[i] = ref_e4m3_encode(y[i]);
}

void ref_e4m3_decode_array(const uint8_t *c, int64_t n, double *out)
{
    for (int64_t i = 0; i < n; i++)
        out[i] = ref_e4m3_decode(c[i]);
}

/* ------------------------------------------------------------------------ */
/* Input widening.  dtype 0 = FP32, 1 = BF16 (raw 16-bit patterns).          */
/* ------------------------------------------------------------------------ */

static float ref_load(const void *x, int dtype, int64_t idx)
{
    if (dtype == 0)
        return ((const float *)x)[idx];
    uint32_t bits = (uint32_t)((const uint16_t *)x)[idx] << 16;  /* BF16 is the top half of FP32 */
    float f;
    memcpy(&f, &bits, 4);
    return f;
}

/* ------------------------------------------------------------------------ */
/* One block: amax -> s = fl32(amax / 448) -> q_i = E4M3(fl32(x_i / s)).     */
/* vals[i] are the block's elements (already widened), n of them.            */
/* Returns s; writes codes[i].                                               */
/* ------------------------------------------------------------------------ */

static float ref_quant_block(const float *vals, int64_t n, uint8_t *codes)
{
    float amax = 0.0f;
    for (int64_t i = 0; i < n; i++) {
        float a = fabsf(vals[i]);
        if (a > amax)
            amax = a;
    }
    float s = amax / 448.0f;             /* IEEE binary32 division, RNE */
    if (s == 0.0f) {                     /* zero block, or amax/448 underflows */
        for (int64_t i = 0; i < n; i++)
            codes[i] = signbit(vals[i]) ? 0x80 : 0x00;
        return 0.0f;
    }
    for (int64_t i = 0; i < n; i++) {
        float y = vals[i] / s;           /* IEEE binary32 division, RNE */
        codes[i] = ref_e4m3_encode(y);
    }
    return s;
}

/*
 * Power-of-two rule, a variant for the scaled matrix cores (their block
 * scales are E8M0: powers of two 2^k, k in [-127, 127]).  The scale is the
 * smallest power of two s = 2^k with 448 * s >= amax, k limited to that range
 * (a zero block gets 2^-127); q_i = E4M3(x_i / s).  x_i / s is exact in FP64
 * and, in the range that can round to a non-zero code, in FP32 as well.
 */
static float ref_quant_block_pow2(const float *vals, int64_t n, uint8_t *codes)
{
    double amax = 0.0;
    for (int64_t i = 0; i < n; i++) {
        double a = fabs((double)vals[i]);
        if (a > amax)
            amax = a;
    }
    int k = -127;
    while (k < 127 && 448.0 * ldexp(1.0, k) < amax)
        k++;
    double s = ldexp(1.0, k);
    for (int64_t i = 0; i < n; i++)
        codes[i] = ref_e4m3_encode((float)((double)vals[i] / s));
    return (float)s;
}

/* Scale rules: 0 = amax / 448 (the recipe), 1 = power of two (above). */
static float ref_quant_rule(const float *vals, int64_t n, uint8_t *codes, int rule)
{
    return rule ? ref_quant_block_pow2(vals, n, codes) : ref_quant_block(vals, n, codes);
}

/* Status codes shared in meaning (not in code) with the library's. */
#define REF_OK 0
#define REF_ERR_SHAPE 2

/*
 * Block count along an extent of n elements: blocks of 128, the last one
 * holding the remaining n % 128 elements when n is not a multiple of 128.
 */
static int64_t ref_nblk(int64_t n)
{
    return (n + 127) / 128;
}

static int64_t ref_blen(int64_t n, int64_t b)
{
    int64_t rest = n - b * 128;
    return rest < 128 ? rest : 128;
}

/*
 * Activation / gradient quantiser: x[rows][cols] (row stride ldx), blocks of
 * 128 consecutive elements along each row.  q[rows][cols] (stride ldq),
 * s[rows][ceil(cols/128)] dense.
 */
int ref_quant_act_rule(const void *x, int dtype, int64_t rows, int64_t cols, int64_t ldx,
                       uint8_t *q, int64_t ldq, float *s, int rule)
{
    if (rows < 0 || cols < 0 || ldx < cols || ldq < cols)
        return REF_ERR_SHAPE;
    int64_t nb = ref_nblk(cols);
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; r++) {
        float vals[128];
        for (int64_t b = 0; b < nb; b++) {
            int64_t len = ref_blen(cols, b);
            for (int64_t i = 0; i < len; i++)
                vals[i] = ref_load(x, dtype, r * ldx + b * 128 + i);
            s[r * nb + b] = ref_quant_rule(vals, len, q + r * ldq + b * 128, rule);
        }
    }
    return REF_OK;
}

/*
 * Weight quantiser: w[rows][cols] (stride ldw), one block per 128x128 tile
 * (edge tiles hold what remains).  q[rows][cols] (stride ldq),
 * s[ceil(rows/128)][ceil(cols/128)] dense.
 */
int ref_quant_weight_rule(const void *w, int dtype, int64_t rows, int64_t cols, int64_t ldw,
                          uint8_t *q, int64_t ldq, float *s, int rule)
{
    if (rows < 0 || cols < 0 || ldw < cols || ldq < cols)
        return REF_ERR_SHAPE;
    int64_t rb = ref_nblk(rows), cb = ref_nblk(cols);
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t tr = 0; tr < rb; tr++) {
        for (int64_t tc = 0; tc < cb; tc++) {
            int64_t nr = ref_blen(rows, tr), nc = ref_blen(cols, tc);
            float *vals = (float *)malloc(sizeof(float) * 128 * 128);
            uint8_t *codes = (uint8_t *)malloc(128 * 128);
            for (int64_t i = 0; i < nr; i++)
                for (int64_t j = 0; j < nc; j++)
                    vals[i * nc + j] = ref_load(w, dtype, (tr * 128 + i) * ldw + tc * 128 + j);
            s[tr * cb + tc] = ref_quant_rule(vals, nr * nc, codes, rule);
            for (int64_t i = 0; i < nr; i++)
                for (int64_t j = 0; j < nc; j++)
                    q[(tr * 128 + i) * ldq + tc * 128 + j] = codes[i * nc + j];
            free(vals);
            free(codes);
        }
    }
    return REF_OK;
}

/*
 * Token-dimension quantiser for the weight-gradient GEMM: x[tokens][cols]
 * (stride ldx); blocks are 128 consecutive tokens of one column.
 *   transpose_out = 1: q[cols][tokens] (stride ldq), s[cols][ceil(tokens/128)]
 *   transpose_out = 0: q[tokens][cols] (stride ldq), s[ceil(tokens/128)][cols]
 */
int ref_quant_transpose_rule(const void *x, int dtype, int64_t tokens, int64_t cols, int64_t ldx,
                             int transpose_out, uint8_t *q, int64_t ldq, float *s, int rule)
{
    if (tokens < 0 || cols < 0 || ldx < cols)
        return REF_ERR_SHAPE;
    if (transpose_out ? (ldq < tokens) : (ldq < cols))
        return REF_ERR_SHAPE;
    int64_t tb = ref_nblk(tokens);
#pragma omp parallel for schedule(static)
    for (int64_t c = 0; c < cols; c++) {
        float vals[128];
        uint8_t codes[128];
        for (int64_t b = 0; b < tb; b++) {
            int64_t len = ref_blen(tokens, b);
            for (int64_t i = 0; i < len; i++)
                vals[i] = ref_load(x, dtype, (b * 128 + i) * ldx + c);
            float sc = ref_quant_rule(vals, len, codes, rule);
            for (int64_t i = 0; i < len; i++) {
                int64_t t = b * 128 + i;
                if (transpose_out)
                    q[c * ldq + t] = codes[i];
                else
                    q[t * ldq + c] = codes[i];
            }
            if (transpose_out)
                s[c * tb + b] = sc;
            else
                s[b * cols + c] = sc;
        }
    }
    return REF_OK;
}

/* The recipe's rule (amax / 448). */
int ref_quant_act(const void *x, int dtype, int64_t rows, int64_t cols, int64_t ldx, uint8_t *q, int64_t ldq,
                  float *s)
{
    return ref_quant_act_rule(x, dtype, rows, cols, ldx, q, ldq, s, 0);
}

int ref_quant_weight(const void *w, int dtype, int64_t rows, int64_t cols, int64_t ldw, uint8_t *q, int64_t ldq,
                     float *s)
{
    return ref_quant_weight_rule(w, dtype, rows, cols, ldw, q, ldq, s, 0);
}

int ref_quant_transpose(const void *x, int dtype, int64_t tokens, int64_t cols, int64_t ldx, int transpose_out,
                        uint8_t *q, int64_t ldq, float *s)
{
    return ref_quant_transpose_rule(x, dtype, tokens, cols, ldx, transpose_out, q, ldq, s, 0);
}

/* ------------------------------------------------------------------------ */
/* Blockwise GEMM                                                            */
/*                                                                           */
/*   C[m][n] = sum_kb  sA(m,kb) * sB(n,kb) * sum_{k in kb} a(m,k) * b(k,n)   */
/*                                                                           */
/* a, b are decoded E4M3 values; kb runs over the ceil(K/128) blocks, the    */
/* last one holding K % 128 positions when K is not a multiple.  The inner   */
/* 128-term sum is exact in FP64 (products are 8-bit significands times      */
/* powers of two in [2^-18, 2^10]; 128 of them fit in 43 bits) and sA*sB is  */
/* exact (two 24-bit significands), so C differs from the real-number result */
/* only by the FP64 rounding of the block products and the block sum.        */
/*                                                                           */
/* Layouts (row-major, C is [M][N]):                                         */
/*   0 NT: A [M][K] (lda), B [N][K] (ldb)                                    */
/*   1 NN: A [M][K] (lda), B [K][N] (ldb)                                    */
/*   2 TN: A [K][M] (lda), B [K][N] (ldb)                                    */
/* Scales are dense and indexed in the operand's storage orientation, with  */
/* KB = ceil(K/128) and NB = ceil(N/128):                                    */
/*   A, K-contiguous: sA[M][KB];  A, M-contiguous (TN): sA[KB][M]            */
/*   B 1x128 (bgran 0):   NT sB[N][KB];   NN/TN sB[KB][N]                    */
/*   B 128x128 (bgran 1): NT sB[NB][KB];  NN/TN sB[KB][NB]                   */
/* ------------------------------------------------------------------------ */

static int ref_gemm_check(int layout, int64_t M, int64_t N, int64_t K, int64_t lda, int64_t ldb,
                          int bgran)
{
    if (layout < 0 || layout > 2 || bgran < 0 || bgran > 1)
        return REF_ERR_SHAPE;
    if (M < 0 || N < 0 || K < 0)
        return REF_ERR_SHAPE;
    if (layout == 2 ? lda < M : lda < K)
        return REF_ERR_SHAPE;
    if (layout == 0 ? ldb < K : ldb < N)
        return REF_ERR_SHAPE;
    return REF_OK;
}

static inline uint8_t ref_a_code(int layout, const uint8_t *A, int64_t lda, int64_t m, int64_t k)
{
    return layout == 2 ? A[k * lda + m] : A[m * lda + k];
}

static inline uint8_t ref_b_code(int layout, const uint8_t *B, int64_t ldb, int64_t k, int64_t n)
{
    return layout == 0 ? B[n * ldb + k] : B[k * ldb + n];
}

static inline double ref_a_scale(int layout, const float *sA, int64_t M, int64_t K, int64_t m,
                                 int64_t kb)
{
    return layout == 2 ? (double)sA[kb * M + m] : (double)sA[m * ref_nblk(K) + kb];
}

static inline double ref_b_scale(int layout, int bgran, const float *sB, int64_t N, int64_t K,
                                 int64_t n, int64_t kb)
{
    if (layout == 0)
        return bgran ? (double)sB[(n / 128) * ref_nblk(K) + kb] : (double)sB[n * ref_nblk(K) + kb];
    return bgran ? (double)sB[kb * ref_nblk(N) + n / 128] : (double)sB[kb * N + n];
}

static double ref_gemm_one(int layout, int64_t M, int64_t N, int64_t K, const uint8_t *A,
                           int64_t lda, const float *sA, const uint8_t *B, int64_t ldb,
                           const float *sB, int bgran, int64_t m, int64_t n)
{
    double c = 0.0;
    for (int64_t kb = 0; kb < ref_nblk(K); kb++) {
        double p = 0.0;
        for (int64_t k = kb * 128; k < kb * 128 + ref_blen(K, kb); k++)
            p += ref_e4m3_decode(ref_a_code(layout, A, lda, m, k)) *
                 ref_e4m3_decode(ref_b_code(layout, B, ldb, k, n));
        double sab = ref_a_scale(layout, sA, M, K, m, kb) * ref_b_scale(layout, bgran, sB, N, K, n, kb);
        c += sab * p;
    }
    return c;
}

/* Full product into C[M][N] (FP64, stride ldc). */
int ref_gemm(int layout, int64_t M, int64_t N, int64_t K, const uint8_t *A, int64_t lda,
             const float *sA, const uint8_t *B, int64_t ldb, const float *sB, int bgran, double *C,
             int64_t ldc)
{
    int st = ref_gemm_check(layout, M, N, K, lda, ldb, bgran);
    if (st != REF_OK || ldc < N)
        return st != REF_OK ? st : REF_ERR_SHAPE;
    ref_init_table();
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t m = 0; m < M; m++)
        for (int64_t n = 0; n < N; n++)
            C[m * ldc + n] = ref_gemm_one(layout, M, N, K, A, lda, sA, B, ldb, sB, bgran, m, n);
    return REF_OK;
}

/* Selected entries only: out[i] = C[ms[i]][ns[i]]. */
int ref_gemm_entries(int layout, int64_t M, int64_t N, int64_t K, const uint8_t *A, int64_t lda,
                     const float *sA, const uint8_t *B, int64_t ldb, const float *sB, int bgran,
                     const int64_t *ms, const int64_t *ns, int64_t count, double *out)
{
    int st = ref_gemm_check(layout, M, N, K, lda, ldb, bgran);
    if (st != REF_OK)
        return st;
    for (int64_t i = 0; i < count; i++)
        if (ms[i] < 0 || ms[i] >= M || ns[i] < 0 || ns[i] >= N)
            return REF_ERR_SHAPE;
    ref_init_table();
#pragma omp parallel for schedule(dynamic, 16)
    for (int64_t i = 0; i < count; i++)
        out[i] = ref_gemm_one(layout, M, N, K, A, lda, sA, B, ldb, sB, bgran, ms[i], ns[i]);
    return REF_OK;
}

/*
 * Brute force: dequantise both operands to FP64 (value(q) * s, exact), then a
 * textbook triple loop for C = A_hat * B_hat in FP64.  Used on tiny shapes to
 * pin ref_gemm's block bookkeeping.
 */
int ref_gemm_brute(int layout, int64_t M, int64_t N, int64_t K, const uint8_t *A, int64_t lda,
                   const float *sA, const uint8_t *B, int64_t ldb, const float *sB, int bgran,
                   double *C, int64_t ldc)
{
    int st = ref_gemm_check(layout, M, N, K, lda, ldb, bgran);
    if (st != REF_OK || ldc < N)
        return st != REF_OK ? st : REF_ERR_SHAPE;
    double *Ah = (double *)malloc(sizeof(double) * (size_t)(M * K > 0 ? M * K : 1));
    double *Bh = (double *)malloc(sizeof(double) * (size_t)(K * N > 0 ? K * N : 1));
    for (int64_t m = 0; m < M; m++)
        for (int64_t k = 0; k < K; k++)
            Ah[m * K + k] = ref_e4m3_decode(ref_a_code(layout, A, lda, m, k)) *
                            ref_a_scale(layout, sA, M, K, m, k / 128);
    for (int64_t k = 0; k < K; k++)
        for (int64_t n = 0; n < N; n++)
            Bh[k * N + n] = ref_e4m3_decode(ref_b_code(layout, B, ldb, k, n)) *
                            ref_b_scale(layout, bgran, sB, N, K, n, k / 128);
    for (int64_t m = 0; m < M; m++)
        for (int64_t n = 0; n < N; n++) {
            double acc = 0.0;
            for (int64_t k = 0; k < K; k++)
                acc += Ah[m * K + k] * Bh[k * N + n];
            C[m * ldc + n] = acc;
        }
    free(Ah);
    free(Bh);
    return REF_OK;
}

/* ------------------------------------------------------------------------ */
/* Output roundings used when the product is stored narrower than FP64.     */
/* ------------------------------------------------------------------------ */

/* FP64 -> nearest BF16 pattern, ties to even (finite inputs). */
uint16_t ref_bf16_rne(double v)
{
    if (v == 0.0)
        return signbit(v) ? 0x8000 : 0x0000;
    /* Candidates: truncate the FP32 image toward zero and step one BF16 ulp up. */
    float f = (float)v;                  /* only to locate the neighbourhood */
    uint32_t u;
    memcpy(&u, &f, 4);
    uint32_t t = u & 0xFFFF0000u;
    double best = 0, cand[3];
    uint32_t pats[3] = {t - 0x10000u, t, t + 0x10000u};
    int bi = -1;
    for (int i = 0; i < 3; i++) {
        float g;
        memcpy(&g, &pats[i], 4);
        cand[i] = (double)g;
        if (!isfinite(cand[i]))
            continue;
        double d = fabs(cand[i] - v);
        if (bi < 0 || d < best || (d == best && ((pats[i] >> 16) & 1u) == 0)) {
            best = d;
            bi = i;
        }
    }
    return (uint16_t)(pats[bi] >> 16);
}

void ref_bf16_rne_array(const double *v, int64_t n, uint16_t *out)
{
    for (int64_t i = 0; i < n; i++)
        out[i] = ref_bf16_rne(v[i]);
}

/* ------------------------------------------------------------------------ */
/* Gated feed-forward activation feeding the down projection.               */
/* ------------------------------------------------------------------------ */

/* The model card's configuration table gives the architecture as the Qwen3-1.7B
 * configuration (feed-forward size 6,144); that configuration's feed-forward
 * block is the SiLU-gated linear unit (SwiGLU of the GLU-variants paper,
 * Shazeer 2020, with the Swish parameter fixed at 1):
 *     h = silu(g) * u,   silu(g) = g * sigmoid(g) = g / (1 + e^-g),
 * with g the gate projection's output and u the up projection's.  The pages
 * do not state it; this is the reading taken.  Evaluated in FP64 straight
 * from the definition (exp(-g) overflows to +inf for g < -709, where the
 * quotient is the correctly signed zero). */
double ref_swiglu(double g, double u)
{
    return g * u / (1.0 + exp(-g));
}

void ref_swiglu_array(const double *g, const double *u, int64_t n, double *out)
{
    for (int64_t i = 0; i < n; i++)
        out[i] = ref_swiglu(g[i], u[i]);
}

int ref_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
