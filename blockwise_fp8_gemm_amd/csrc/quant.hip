// Blockwise E4M3 quantisers for gfx950.
//
// Each block of values x_i gets one FP32 dequantisation scale
//   s = fl32(amax / 448),  q_i = E4M3_RNE(fl32(x_i / s)),
// or, with pow2, s = the smallest power of two with 448 s >= amax (the scaled
// matrix cores' E8M0 block scales),
// with s == 0 (all-zero block, or amax/448 underflowing) stored as 0 and the
// codes set to +-0 by sign.  Blocks are 1x128 along rows (activations and
// gradients), 128x128 tiles (weights), or 128 consecutive tokens of one
// column (the token-dimension copies the weight-gradient GEMM contracts over).
// This is the "blockwise E4M3" of the Puro-2B-Base model card's setup
// paragraph under the Phase 1 / Phase 2 table, with the DeepSeek-V3 block
// shapes the technical report's related-work paragraph points to.
//
// All three kernels are HBM-bound: each input element is read once, held in
// registers across the amax reduction, and written once as a byte.
#include "common.h"
#include "kernels.h"

namespace puro {

// Streaming stores for the quantisers' codes (and the fused form's
// activation): the writing kernel never reads them back, and the
// non-temporal hint keeps them from displacing in the caches the inputs that
// are still being read.  Measured on gfx950 with identical outputs: the dual
// quantiser at 8192 x 2048 in 14.2 us instead of 17.1, at 8192 x 12288 in
// 70.6 us instead of 89.0.  (Non-temporal loads of the inputs made it slower.)
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ void store_nt(void *p, uint32_t a, uint32_t b)
{
    const u32x2 v = {a, b};
    __builtin_nontemporal_store(v, reinterpret_cast<u32x2 *>(p));
}
__device__ __forceinline__ void store_nt(void *p, uint32_t a, uint32_t b, uint32_t c, uint32_t d)
{
    const u32x4 v = {a, b, c, d};
    __builtin_nontemporal_store(v, reinterpret_cast<u32x4 *>(p));
}

// ---------------------------------------------------------------------------
// 1x128 row blocks.  One 16-lane group per run of BPG consecutive blocks of a
// row, 8 consecutive elements of each block per lane (one 16-byte load for
// BF16, two for FP32); all of a lane's loads are issued before any arithmetic
// so that each wave keeps BPG KB (BF16) in flight.  amax by cross-lane max
// within the 16-lane group.
// ---------------------------------------------------------------------------
constexpr int BPG = 4;

template <typename T>
__global__ __launch_bounds__(256) void quant_act_kernel(const T *__restrict__ x, int64_t rows,
                                                        int64_t cols, int64_t ldx,
                                                        uint8_t *__restrict__ q, int64_t ldq,
                                                        float *__restrict__ s, int64_t nb, int pow2)
{
    const int64_t runs = (nb + BPG - 1) / BPG;
    const int64_t grp = ((int64_t)blockIdx.x * 256 + threadIdx.x) >> 4;
    if (grp >= rows * runs)
        return;  // whole 16-lane groups leave together
    const int l16 = threadIdx.x & 15;
    const int64_t r = grp / runs;
    const int64_t b0 = (grp - r * runs) * BPG;
    const T *xr = x + r * ldx;

    float v[BPG][8];
#pragma unroll
    for (int u = 0; u < BPG; u++) {
        const int64_t c0 = (b0 + u) * 128 + l16 * 8;
        if (c0 + 8 <= cols) {
            Elem<T>::load8(xr + c0, v[u]);
        } else {
#pragma unroll
            for (int i = 0; i < 8; i++)
                v[u][i] = (c0 + i < cols) ? Elem<T>::load(xr + c0 + i) : 0.0f;
        }
    }
    uint8_t *qr = q + r * ldq;
#pragma unroll
    for (int u = 0; u < BPG; u++) {
        const int64_t b = b0 + u;
        if (b >= nb)
            break;
        float amax = 0.0f;
#pragma unroll
        for (int i = 0; i < 8; i++)
            amax = fmaxf(amax, fabsf(v[u][i]));
#pragma unroll
        for (int off = 8; off >= 1; off >>= 1)
            amax = fmaxf(amax, __shfl_xor(amax, off, 16));
        const float sc = block_scale(amax, pow2);
        const Divider dv = make_divider(sc);
        const uint32_t lo = quant4(v[u][0], v[u][1], v[u][2], v[u][3], dv);
        const uint32_t hi = quant4(v[u][4], v[u][5], v[u][6], v[u][7], dv);
        const int64_t c0 = b * 128 + l16 * 8;
        if (c0 + 8 <= cols) {
            store_nt(qr + c0, lo, hi);
        } else {
#pragma unroll
            for (int i = 0; i < 8; i++)
                if (c0 + i < cols)
                    qr[c0 + i] = (uint8_t)(((i < 4 ? lo : hi) >> (8 * (i & 3))) & 0xFF);
        }
        if (l16 == 0)
            s[r * nb + b] = sc;
    }
}

// ---------------------------------------------------------------------------
// 128x128 weight tiles.  One 1024-thread workgroup per tile (weights have few
// tiles, so many threads per tile keep the GPU busy); thread t owns columns
// 8*(t%16) .. +7 of rows t/16 and t/16 + 64: 16 values in registers.  amax:
// cross-lane max per wave, then across the 16 waves through LDS.
// ---------------------------------------------------------------------------
// Tile (tx, ty) of one weight: columns [128 tx, +128) x rows [128 ty, +128).
// With qt, the tile's codes are also written transposed, to qt[c][r] (row
// stride ldqt), and its scale to st[tx][ty] (rb = tile rows of the weight).
template <typename T>
__device__ __forceinline__ void quant_weight_tile(const T *__restrict__ w, int64_t rows, int64_t cols,
                                                  int64_t ldw, uint8_t *__restrict__ q, int64_t ldq,
                                                  float *__restrict__ s, int64_t cb, int64_t tx,
                                                  int64_t ty, int pow2, uint8_t *__restrict__ qt = nullptr,
                                                  int64_t ldqt = 0, float *__restrict__ st = nullptr,
                                                  int64_t rb = 0)
{
    __shared__ float red[16];
    __shared__ uint8_t tt[128][128 + 4];   // transposed codes [column][row], padded rows
    const int t = threadIdx.x;
    const int cc = t & 15, rg = t >> 4;
    const int64_t r0 = ty * 128, cbase = tx * 128;
    const int64_t c0 = cbase + cc * 8;
    const bool full_tile = (r0 + 128 <= rows) && (cbase + 128 <= cols);

    float v[2][8];
#pragma unroll
    for (int i = 0; i < 2; i++) {
        const int64_t r = r0 + rg + 64 * i;
        const T *wr = w + r * ldw;
        if (full_tile) {
            Elem<T>::load8(wr + c0, v[i]);
        } else {
#pragma unroll
            for (int j = 0; j < 8; j++)
                v[i][j] = (r < rows && c0 + j < cols) ? Elem<T>::load(wr + c0 + j) : 0.0f;
        }
    }
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 2; i++)
#pragma unroll
        for (int j = 0; j < 8; j++)
            amax = fmaxf(amax, fabsf(v[i][j]));
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1)
        amax = fmaxf(amax, __shfl_xor(amax, off, 64));
    if ((t & 63) == 0)
        red[t >> 6] = amax;
    __syncthreads();
    amax = red[0];
#pragma unroll
    for (int i = 1; i < 16; i++)
        amax = fmaxf(amax, red[i]);
    const float sc = block_scale(amax, pow2);
    const Divider dv = make_divider(sc);

#pragma unroll
    for (int i = 0; i < 2; i++) {
        const int64_t r = r0 + rg + 64 * i;
        const uint32_t lo = quant4(v[i][0], v[i][1], v[i][2], v[i][3], dv);
        const uint32_t hi = quant4(v[i][4], v[i][5], v[i][6], v[i][7], dv);
        uint8_t *qr = q + r * ldq;
        if (full_tile) {
            store_nt(qr + c0, lo, hi);
        } else if (r < rows) {
#pragma unroll
            for (int j = 0; j < 8; j++)
                if (c0 + j < cols)
                    qr[c0 + j] = (uint8_t)(((j < 4 ? lo : hi) >> (8 * (j & 3))) & 0xFF);
        }
        if (qt) {
#pragma unroll
            for (int j = 0; j < 8; j++)
                tt[cc * 8 + j][rg + 64 * i] = (uint8_t)(((j < 4 ? lo : hi) >> (8 * (j & 3))) & 0xFF);
        }
    }
    if (t == 0) {
        s[ty * cb + tx] = sc;
        if (qt)
            st[tx * rb + ty] = sc;
    }
    if (qt) {
        // thread t writes bytes [16 (t % 8), +16) of transposed row t / 8
        __syncthreads();
        const int c = t >> 3, sg = t & 7;
        const int64_t cg = cbase + c, rs = r0 + 16 * sg;
        const uint32_t *src = reinterpret_cast<const uint32_t *>(&tt[c][16 * sg]);
        uint8_t *dst = qt + cg * ldqt + rs;
        if (full_tile) {
            store_nt(dst, src[0], src[1], src[2], src[3]);
        } else if (cg < cols) {
            for (int e = 0; e < 16; e++)
                if (rs + e < rows)
                    dst[e] = tt[c][16 * sg + e];
        }
    }
}

template <typename T>
__global__ __launch_bounds__(1024) void quant_weight_kernel(const T *__restrict__ w, int64_t rows,
                                                            int64_t cols, int64_t ldw,
                                                            uint8_t *__restrict__ q, int64_t ldq,
                                                            float *__restrict__ s, int64_t cb, int pow2)
{
    quant_weight_tile<T>(w, rows, cols, ldw, q, ldq, s, cb, blockIdx.x, blockIdx.y, pow2);
}

// Several weights in one launch: weight i owns workgroups [first[i], first[i+1]),
// one per tile, row-major over its tiles.
struct QuantWeightGroup {
    QuantWeightItem it[kQuantGroupMax];
    int first[kQuantGroupMax + 1];
    int count;
    int pow2;
};

template <typename T>
__global__ __launch_bounds__(1024) void quant_weight_group_kernel(QuantWeightGroup args)
{
    (void)args;   // read through the argument segment pointer: no copy to scratch memory
    typedef __attribute__((address_space(4))) const QuantWeightGroup *KernargQ;
    const KernargQ g = (KernargQ)__builtin_amdgcn_kernarg_segment_ptr();
    const int b = blockIdx.x;
    int i = 0;
    while (i + 1 < g->count && b >= g->first[i + 1])
        i++;
    i = __builtin_amdgcn_readfirstlane(i);   // uniform: the item's fields stay in scalar registers
    const int64_t local = b - g->first[i], cb = g->it[i].cb;
    quant_weight_tile<T>((const T *)g->it[i].w, g->it[i].rows, g->it[i].cols, g->it[i].ldw, g->it[i].q,
                         g->it[i].ldq, g->it[i].s, cb, local % cb, local / cb, g->pow2, g->it[i].qt,
                         g->it[i].ldqt, g->it[i].st, g->it[i].rb);
}

// ---------------------------------------------------------------------------
// Token blocks (128 tokens x 1 column), for a tile of 128 tokens x 64 columns
// per workgroup.  Thread t owns columns 8*(t%8) .. +7 of the 4 consecutive
// tokens 4*(t/8) .. +3.  Column amax: per-thread max over its 4 tokens,
// cross-lane max over lanes with equal t%8, then across the 4 waves through
// LDS.  For the transposed output each thread packs its 4 token codes of a
// column into one 32-bit LDS word; the tile is written out as 128-byte rows.
// ---------------------------------------------------------------------------
template <typename T, bool TRANSPOSE_OUT>
__global__ __launch_bounds__(256) void quant_transpose_kernel(const T *__restrict__ x,
                                                              int64_t tokens, int64_t cols,
                                                              int64_t ldx, uint8_t *__restrict__ q,
                                                              int64_t ldq, float *__restrict__ s,
                                                              int64_t ntb, int pow2)
{
    __shared__ float red[4][64];
    __shared__ float scl[64];
    __shared__ uint32_t tile[64][32 + 1];   // [column][token/4], odd stride: no bank conflicts

    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    const int cc = t & 7, rq = t >> 3;
    const int64_t tok0 = (int64_t)blockIdx.y * 128;
    const int64_t col0 = (int64_t)blockIdx.x * 64;
    const int64_t c0 = col0 + cc * 8;
    const bool full = (tok0 + 128 <= tokens) && (col0 + 64 <= cols);

    float v[4][8];
#pragma unroll
    for (int i = 0; i < 4; i++) {
        const int64_t tk = tok0 + 4 * rq + i;
        const T *xr = x + tk * ldx;
        if (full) {
            Elem<T>::load8(xr + c0, v[i]);
        } else {
#pragma unroll
            for (int j = 0; j < 8; j++)
                v[i][j] = (tk < tokens && c0 + j < cols) ? Elem<T>::load(xr + c0 + j) : 0.0f;
        }
    }
    float m[8];
#pragma unroll
    for (int j = 0; j < 8; j++) {
        m[j] = fmaxf(fmaxf(fabsf(v[0][j]), fabsf(v[1][j])), fmaxf(fabsf(v[2][j]), fabsf(v[3][j])));
        m[j] = fmaxf(m[j], __shfl_xor(m[j], 8, 64));
        m[j] = fmaxf(m[j], __shfl_xor(m[j], 16, 64));
        m[j] = fmaxf(m[j], __shfl_xor(m[j], 32, 64));
    }
    if (lane < 8) {
#pragma unroll
        for (int j = 0; j < 8; j++)
            red[wave][lane * 8 + j] = m[j];
    }
    __syncthreads();
    if (t < 64) {
        const float amax = fmaxf(fmaxf(red[0][t], red[1][t]), fmaxf(red[2][t], red[3][t]));
        const float sc = block_scale(amax, pow2);
        scl[t] = sc;
        const int64_t c = col0 + t;
        if (c < cols) {
            if (TRANSPOSE_OUT)
                s[c * ntb + blockIdx.y] = sc;
            else
                s[(int64_t)blockIdx.y * cols + c] = sc;
        }
    }
    __syncthreads();

    uint32_t word[8];   // word[j]: the 4 token codes of column cc*8+j
#pragma unroll
    for (int j = 0; j < 8; j++)
        word[j] = quant4(v[0][j], v[1][j], v[2][j], v[3][j], make_divider(scl[cc * 8 + j]));
    if (TRANSPOSE_OUT) {
#pragma unroll
        for (int j = 0; j < 8; j++)
            tile[cc * 8 + j][rq] = word[j];
        __syncthreads();
#pragma unroll
        for (int it = 0; it < 2; it++) {
            const int chunk = t + 256 * it;
            const int row = chunk >> 3, seg = chunk & 7;
            const int64_t c = col0 + row;
            const int64_t tk = tok0 + seg * 16;
            if (c >= cols)
                continue;
            uint8_t *dst = q + c * ldq + tk;
            const uint32_t *src = &tile[row][seg * 4];
            if (tk + 16 <= tokens) {
                store_nt(dst, src[0], src[1], src[2], src[3]);
            } else {
                for (int e = 0; e < 16; e++)
                    if (tk + e < tokens)
                        dst[e] = (uint8_t)((src[e >> 2] >> (8 * (e & 3))) & 0xFF);
            }
        }
    } else {
        // untransposed: row (token) 4*rq+i gets byte i of each column word
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const int64_t tk = tok0 + 4 * rq + i;
            uint32_t b[8];
#pragma unroll
            for (int j = 0; j < 8; j++)
                b[j] = (word[j] >> (8 * i)) & 0xFFu;
            uint8_t *qr = q + tk * ldq;
            if (full) {
                store_nt(qr + c0, b[0] | (b[1] << 8) | (b[2] << 16) | (b[3] << 24),
                               b[4] | (b[5] << 8) | (b[6] << 16) | (b[7] << 24));
            } else if (tk < tokens) {
#pragma unroll
                for (int j = 0; j < 8; j++)
                    if (c0 + j < cols)
                        qr[c0 + j] = (uint8_t)b[j];
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Dual quantiser: one read of x [tokens][cols] produces both the 1x128
// row-blocked copy (each token's 128-column blocks) and the token-blocked
// copy (each column's 128-token blocks), exactly as the two separate kernels
// do.  One workgroup per 128-token x 128-column tile, which holds one block
// of each kind per token and per column.  Thread t owns columns 8*(t%16) .. +7
// of the 8 consecutive tokens 8*(t/16) .. +7 (64 values in registers).
// Row amax: cross-lane max over the 16 lanes with equal t/16.  Column amax:
// per-thread max over its 8 tokens, cross-lane max over lanes with equal
// t%16, then across the 4 waves through LDS.  This general form serves FP32
// input, the untransposed token-block copy and the ragged edge tiles of the
// packed BF16 kernel below; (bx0, by0) offsets the tile grid for the latter.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float lo16f(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float hi16f(uint32_t u) { return __uint_as_float(u & 0xFFFF0000u); }

// SiLU-gated activation h = silu(g) * u, silu(g) = g / (1 + e^-g), in FP32 for
// BF16 g and u (the feed-forward block of the Qwen3-1.7B configuration the
// model card names).  g * u is exact (two 8-bit significands).  e = exp(-|g|)
// lies in (0, 1]: sigmoid(g) = 1 / (1 + e) for g >= 0 and e / (1 + e) for
// g < 0, so nothing overflows.  Relative error: a few FP32 ulps (expf, the
// reciprocal, two products); where e is subnormal (g < -87.3) its absolute
// error 2^-149 carries over as 2^-149 |g u|.
__device__ __forceinline__ float swiglu_f32(float g, float u)
{
    const float e = expf(-fabsf(g));
    const float sig = (g < 0.0f ? e : 1.0f) * __builtin_amdgcn_rcpf(1.0f + e);
    return (g * u) * sig;
}

// Two packed BF16 gate values and two up values -> two packed BF16 activations.
__device__ __forceinline__ uint32_t swiglu2(uint32_t g2, uint32_t u2)
{
    return to_bf16x2(swiglu_f32(lo16f(g2), lo16f(u2)), swiglu_f32(hi16f(g2), hi16f(u2)));
}

template <typename T, bool TRANSPOSE_OUT, bool SWIGLU>
__global__ __launch_bounds__(256) void quant_dual_kernel(const T *__restrict__ x, int64_t tokens,
                                                         int64_t cols, int64_t ldx,
                                                         uint8_t *__restrict__ qr, int64_t ldqr,
                                                         float *__restrict__ sr, int64_t nbr,
                                                         uint8_t *__restrict__ qt, int64_t ldqt,
                                                         float *__restrict__ st, int64_t ntb, int pow2,
                                                         int bx0, int by0,
                                                         const uint16_t *__restrict__ up, int64_t ldu,
                                                         uint16_t *__restrict__ hout, int64_t ldh)
{
    __shared__ float red[4][128];
    __shared__ float scl[128];
    __shared__ uint32_t tile[128][32 + 1];   // [column][token/4] codes, odd stride

    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    const int cc = t & 15, rq = t >> 4;
    const unsigned bx = blockIdx.x + bx0, by = blockIdx.y + by0;
    const int64_t tok0 = (int64_t)by * 128;
    const int64_t col0 = (int64_t)bx * 128;
    const int64_t c0 = col0 + cc * 8;
    const bool full = (tok0 + 128 <= tokens) && (col0 + 128 <= cols);

    float v[8][8];
#pragma unroll
    for (int i = 0; i < 8; i++) {
        const int64_t tk = tok0 + 8 * rq + i;
        const T *xr = x + tk * ldx;
        if constexpr (SWIGLU) {
            // x is the gate, up the up projection; h = BF16(silu(gate) * up)
            const uint16_t *ur = up + tk * ldu;
            if (full) {
                const uint4 a = *reinterpret_cast<const uint4 *>(xr + c0);
                const uint4 b = *reinterpret_cast<const uint4 *>(ur + c0);
                const uint32_t hv[4] = {swiglu2(a.x, b.x), swiglu2(a.y, b.y), swiglu2(a.z, b.z),
                                        swiglu2(a.w, b.w)};
                if (hout)
                    store_nt(hout + tk * ldh + c0, hv[0], hv[1], hv[2], hv[3]);
#pragma unroll
                for (int p = 0; p < 4; p++) {
                    v[i][2 * p] = lo16f(hv[p]);
                    v[i][2 * p + 1] = hi16f(hv[p]);
                }
            } else {
#pragma unroll
                for (int j = 0; j < 8; j++) {
                    v[i][j] = 0.0f;
                    if (tk < tokens && c0 + j < cols) {
                        const uint32_t hb = swiglu2(xr[c0 + j], ur[c0 + j]) & 0xFFFFu;
                        if (hout)
                            hout[tk * ldh + c0 + j] = (uint16_t)hb;
                        v[i][j] = lo16f(hb);
                    }
                }
            }
        } else if (full) {
            Elem<T>::load8(xr + c0, v[i]);
        } else {
#pragma unroll
            for (int j = 0; j < 8; j++)
                v[i][j] = (tk < tokens && c0 + j < cols) ? Elem<T>::load(xr + c0 + j) : 0.0f;
        }
    }

    // ---- column (token-block) scales
    float m[8];
#pragma unroll
    for (int j = 0; j < 8; j++) {
        float a = fabsf(v[0][j]);
#pragma unroll
        for (int i = 1; i < 8; i++)
            a = fmaxf(a, fabsf(v[i][j]));
        a = fmaxf(a, __shfl_xor(a, 16, 64));
        a = fmaxf(a, __shfl_xor(a, 32, 64));
        m[j] = a;
    }
    if (lane < 16) {
#pragma unroll
        for (int j = 0; j < 8; j++)
            red[wave][lane * 8 + j] = m[j];
    }
    __syncthreads();
    if (t < 128) {
        const float amax = fmaxf(fmaxf(red[0][t], red[1][t]), fmaxf(red[2][t], red[3][t]));
        const float sc = block_scale(amax, pow2);
        scl[t] = sc;
        const int64_t c = col0 + t;
        if (c < cols) {
            if (TRANSPOSE_OUT)
                st[c * ntb + by] = sc;
            else
                st[(int64_t)by * cols + c] = sc;
        }
    }

    // ---- row blocks: quantise and store while the column scales settle
#pragma unroll
    for (int i = 0; i < 8; i++) {
        const int64_t tk = tok0 + 8 * rq + i;
        float a = 0.0f;
#pragma unroll
        for (int j = 0; j < 8; j++)
            a = fmaxf(a, fabsf(v[i][j]));
#pragma unroll
        for (int off = 8; off >= 1; off >>= 1)
            a = fmaxf(a, __shfl_xor(a, off, 16));
        const float sc = block_scale(a, pow2);
        const Divider dv = make_divider(sc);
        const uint32_t lo = quant4(v[i][0], v[i][1], v[i][2], v[i][3], dv);
        const uint32_t hi = quant4(v[i][4], v[i][5], v[i][6], v[i][7], dv);
        uint8_t *q = qr + tk * ldqr;
        if (full) {
            store_nt(q + c0, lo, hi);
        } else if (tk < tokens) {
#pragma unroll
            for (int j = 0; j < 8; j++)
                if (c0 + j < cols)
                    q[c0 + j] = (uint8_t)(((j < 4 ? lo : hi) >> (8 * (j & 3))) & 0xFF);
        }
        if (cc == 0 && tk < tokens)
            sr[tk * nbr + bx] = sc;
    }
    __syncthreads();

    // ---- token blocks
    uint32_t word[2][8];   // word[h][j]: codes of tokens 8rq+4h .. +3 of column cc*8+j
#pragma unroll
    for (int j = 0; j < 8; j++) {
        const Divider dv = make_divider(scl[cc * 8 + j]);
        word[0][j] = quant4(v[0][j], v[1][j], v[2][j], v[3][j], dv);
        word[1][j] = quant4(v[4][j], v[5][j], v[6][j], v[7][j], dv);
    }
    if (TRANSPOSE_OUT) {
#pragma unroll
        for (int j = 0; j < 8; j++) {
            tile[cc * 8 + j][2 * rq] = word[0][j];
            tile[cc * 8 + j][2 * rq + 1] = word[1][j];
        }
        __syncthreads();
#pragma unroll
        for (int it = 0; it < 4; it++) {
            const int chunk = t + 256 * it;
            const int row = chunk >> 3, seg = chunk & 7;
            const int64_t c = col0 + row;
            const int64_t tk = tok0 + seg * 16;
            if (c >= cols)
                continue;
            uint8_t *dst = qt + c * ldqt + tk;
            const uint32_t *src = &tile[row][seg * 4];
            if (tk + 16 <= tokens) {
                store_nt(dst, src[0], src[1], src[2], src[3]);
            } else {
                for (int e = 0; e < 16; e++)
                    if (tk + e < tokens)
                        dst[e] = (uint8_t)((src[e >> 2] >> (8 * (e & 3))) & 0xFF);
            }
        }
    } else {
#pragma unroll
        for (int i = 0; i < 8; i++) {
            const int64_t tk = tok0 + 8 * rq + i;
            uint32_t b[8];
#pragma unroll
            for (int j = 0; j < 8; j++)
                b[j] = (word[i >> 2][j] >> (8 * (i & 3))) & 0xFFu;
            uint8_t *q = qt + tk * ldqt;
            if (full) {
                store_nt(q + c0, b[0] | (b[1] << 8) | (b[2] << 16) | (b[3] << 24),
                               b[4] | (b[5] << 8) | (b[6] << 16) | (b[7] << 24));
            } else if (tk < tokens) {
#pragma unroll
                for (int j = 0; j < 8; j++)
                    if (c0 + j < cols)
                        q[c0 + j] = (uint8_t)b[j];
            }
        }
    }
}


// ---------------------------------------------------------------------------
// Dual quantiser, BF16 input, token-blocked copy transposed.  Same tile and
// thread mapping as quant_dual_kernel, but the 64 values stay packed as BF16
// pairs (32 registers), block maxima are taken on the magnitude bits as
// 16-bit integers (finite inputs: the order of |x| is the order of its bits),
// two at a time, and each block's scale and reciprocal are computed once and
// shared through LDS.
// ---------------------------------------------------------------------------
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t pmax16(uint32_t a, uint32_t b)
{
    return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(__builtin_bit_cast(u16x2, a),
                                                                  __builtin_bit_cast(u16x2, b)));
}

__device__ __forceinline__ uint32_t pshl1(uint32_t a)
{
    return __builtin_bit_cast(uint32_t, __builtin_bit_cast(u16x2, a) << (unsigned short)1);
}

// Max over each row of 16 lanes (DPP row rotates; every lane ends with it).
__device__ __forceinline__ uint32_t rowmax16(uint32_t v)
{
    v = pmax16(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x128, 0xF, 0xF, false));
    v = pmax16(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x124, 0xF, 0xF, false));
    v = pmax16(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x122, 0xF, 0xF, false));
    v = pmax16(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x121, 0xF, 0xF, false));
    return v;
}

// Scale and reciprocal of a block; r = 0 for a zero scale (codes +-0 by sign
// through the fast path) and for scales below 2^-80 (divided exactly).
struct ScaleRcp {
    float s, r;
};
__device__ __forceinline__ ScaleRcp scale_rcp(uint32_t amax_bits, int pow2)
{
    ScaleRcp o;
    o.s = block_scale(__uint_as_float(amax_bits), pow2);
    // a power-of-two scale divides exactly through its reciprocal at any size
    o.r = (pow2 || o.s >= 0x1p-80f) ? 1.0f / o.s : 0.0f;
    return o;
}
__device__ __forceinline__ bool slow_div(float s, float r) { return r == 0.0f && s != 0.0f; }

template <bool SLOW>
__device__ __forceinline__ float qdiv(float x, float s, float r)
{
    if (SLOW && slow_div(s, r))
        return x / s;
    const float y0 = x * r;
    const float e = fmaf(-y0, s, x);
    return __builtin_copysignf(fmaf(e, r, y0), x);
}

template <bool SLOW>
__device__ __forceinline__ uint32_t q4(float a, float b, float c, float d, float s, float r)
{
    return e4m3x4(qdiv<SLOW>(a, s, r), qdiv<SLOW>(b, s, r), qdiv<SLOW>(c, s, r), qdiv<SLOW>(d, s, r));
}

// Quantise this thread's 8 tokens x 8 columns both ways: row codes straight to
// global memory, token-block codes into the LDS tile.
template <bool SLOW>
__device__ __forceinline__ void dual_bf16_quant(uint32_t (&raw)[8][4], const float2 *rsc,
                                                const float *scl, const float *rcl,
                                                uint32_t (*tile)[33], uint8_t *qr_t, int ldqr,
                                                int rq, int cc)
{
#pragma unroll
    for (int i = 0; i < 8; i++) {
        const float2 sr = rsc[8 * rq + i];
        const uint32_t lo = e4m3x4(qdiv<SLOW>(lo16f(raw[i][0]), sr.x, sr.y), qdiv<SLOW>(hi16f(raw[i][0]), sr.x, sr.y),
                                   qdiv<SLOW>(lo16f(raw[i][1]), sr.x, sr.y), qdiv<SLOW>(hi16f(raw[i][1]), sr.x, sr.y));
        const uint32_t hi = e4m3x4(qdiv<SLOW>(lo16f(raw[i][2]), sr.x, sr.y), qdiv<SLOW>(hi16f(raw[i][2]), sr.x, sr.y),
                                   qdiv<SLOW>(lo16f(raw[i][3]), sr.x, sr.y), qdiv<SLOW>(hi16f(raw[i][3]), sr.x, sr.y));
        store_nt(qr_t + (8 * rq + i) * ldqr + cc * 8, lo, hi);
    }
    // Keep the values packed between the two passes: without this the compiler
    // holds the row pass's 64 unpacked floats for the column pass.
#pragma unroll
    for (int i = 0; i < 8; i++)
#pragma unroll
        for (int p = 0; p < 4; p++)
            asm volatile("" : "+v"(raw[i][p]));
#pragma unroll
    for (int p = 0; p < 4; p++) {
        const float s0 = scl[cc * 8 + 2 * p], r0 = rcl[cc * 8 + 2 * p];
        const float s1 = scl[cc * 8 + 2 * p + 1], r1 = rcl[cc * 8 + 2 * p + 1];
#pragma unroll
        for (int h = 0; h < 2; h++) {
            tile[cc * 8 + 2 * p][2 * rq + h] =
                q4<SLOW>(lo16f(raw[4 * h][p]), lo16f(raw[4 * h + 1][p]), lo16f(raw[4 * h + 2][p]),
                         lo16f(raw[4 * h + 3][p]), s0, r0);
            tile[cc * 8 + 2 * p + 1][2 * rq + h] =
                q4<SLOW>(hi16f(raw[4 * h][p]), hi16f(raw[4 * h + 1][p]), hi16f(raw[4 * h + 2][p]),
                         hi16f(raw[4 * h + 3][p]), s1, r1);
        }
    }
}

// Where a tile's BF16 values come from: read from x (DualPlain), or formed
// from the gate and up projections' outputs and optionally stored (DualSwiglu).
// at() moves a source to a tile's first element; in-tile offsets fit 32 bits.
struct DualPlain {
    const uint16_t *x;
    int ldx;
    __device__ __forceinline__ DualPlain at(int64_t t0, int64_t c0) const { return {x + t0 * ldx + c0, ldx}; }
    __device__ __forceinline__ void load(uint32_t (&raw)[8][4], int rq, int cc) const
    {
#pragma unroll
        for (int i = 0; i < 8; i++) {
            const uint4 a = *reinterpret_cast<const uint4 *>(x + (8 * rq + i) * ldx + cc * 8);
            raw[i][0] = a.x; raw[i][1] = a.y; raw[i][2] = a.z; raw[i][3] = a.w;
        }
    }
};

struct DualSwiglu {
    const uint16_t *g, *u;
    uint16_t *h;   // NULL: the activation is not stored
    int ldg, ldu, ldh;
    __device__ __forceinline__ DualSwiglu at(int64_t t0, int64_t c0) const
    {
        return {g + t0 * ldg + c0, u + t0 * ldu + c0, h ? h + t0 * ldh + c0 : nullptr, ldg, ldu, ldh};
    }
    __device__ __forceinline__ void load(uint32_t (&raw)[8][4], int rq, int cc) const
    {
#pragma unroll
        for (int i = 0; i < 8; i++) {
            const int r = 8 * rq + i;
            const uint4 a = *reinterpret_cast<const uint4 *>(g + r * ldg + cc * 8);
            const uint4 b = *reinterpret_cast<const uint4 *>(u + r * ldu + cc * 8);
            raw[i][0] = swiglu2(a.x, b.x);
            raw[i][1] = swiglu2(a.y, b.y);
            raw[i][2] = swiglu2(a.z, b.z);
            raw[i][3] = swiglu2(a.w, b.w);
            if (h)
                store_nt(h + r * ldh + cc * 8, raw[i][0], raw[i][1], raw[i][2], raw[i][3]);
        }
    }
};

// Tiles holding a block whose scale is below 2^-80 (never in practice): reload
// the values and divide those blocks exactly, outside the fast kernel body.
template <class Src>
__device__ __attribute__((noinline)) void dual_bf16_slow(const Src src, const float2 *rsc, const float *scl,
                                                         const float *rcl, uint32_t (*tile)[33],
                                                         uint8_t *qr_t, int ldqr, int rq, int cc)
{
    uint32_t raw[8][4];
    src.load(raw, rq, cc);
    dual_bf16_quant<true>(raw, rsc, scl, rcl, tile, qr_t, ldqr, rq, cc);
}

// One full 128 x 128 tile (the launcher sends ragged edge tiles to
// quant_dual_kernel); offsets inside a tile fit 32 bits (checked by the launcher).
template <class Src>
__device__ __forceinline__ void dual_bf16_tile(const Src &src, uint8_t *__restrict__ qr, int ldqr,
                                               float *__restrict__ sr, int64_t nbr, uint8_t *__restrict__ qt,
                                               int ldqt, float *__restrict__ st, int64_t ntb, int pow2)
{
    __shared__ uint32_t red[4][64];           // [wave][column pair] packed column maxima
    __shared__ float scl[128], rcl[128];       // column scales and reciprocals
    __shared__ float2 rsc[128];                // row (token) scale and reciprocal
    __shared__ uint32_t tile[128][32 + 1];     // [column][token/4] codes, odd stride

    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    const int cc = t & 15, rq = t >> 4, l16 = t & 15;
    const int64_t tok0 = (int64_t)blockIdx.y * 128;
    const int64_t col0 = (int64_t)blockIdx.x * 128;
    const Src src_t = src.at(tok0, col0);

    uint32_t raw[8][4];
    src_t.load(raw, rq, cc);
    constexpr uint32_t MAG = 0x7FFF7FFFu;

    // ---- column partial maxima over this thread's 8 tokens, then the wave's 4 rows
#pragma unroll
    for (int p = 0; p < 4; p++) {
        // magnitudes doubled (each half shifted left by one, dropping its sign)
        uint32_t m = pshl1(raw[0][p]);
#pragma unroll
        for (int i = 1; i < 8; i++)
            m = pmax16(m, pshl1(raw[i][p]));
        m = pmax16(m, (uint32_t)__shfl_xor((int)m, 16, 64));
        m = pmax16(m, (uint32_t)__shfl_xor((int)m, 32, 64));
        if (lane < 16)
            red[wave][cc * 4 + p] = m;
    }

    // ---- row maxima: tokens 2k, 2k+1 packed into one register, reduced over the 16 lanes
    uint32_t rp[4];
#pragma unroll
    for (int k = 0; k < 4; k++) {
        const uint32_t a = pmax16(pmax16(raw[2 * k][0] & MAG, raw[2 * k][1] & MAG),
                                  pmax16(raw[2 * k][2] & MAG, raw[2 * k][3] & MAG));
        const uint32_t b = pmax16(pmax16(raw[2 * k + 1][0] & MAG, raw[2 * k + 1][1] & MAG),
                                  pmax16(raw[2 * k + 1][2] & MAG, raw[2 * k + 1][3] & MAG));
        rp[k] = rowmax16(pmax16(__builtin_amdgcn_perm(b, a, 0x05040100u),
                                __builtin_amdgcn_perm(b, a, 0x07060302u)));
    }
    // lane l16 < 8 of each row group owns token 8 rq + l16
    bool slow;
    {
        const int i = l16 & 7;
        const uint32_t pr = (i >> 1) == 0 ? rp[0] : (i >> 1) == 1 ? rp[1] : (i >> 1) == 2 ? rp[2] : rp[3];
        const ScaleRcp o = scale_rcp((i & 1) ? (pr & 0xFFFF0000u) : (pr << 16), pow2);
        slow = slow_div(o.s, o.r);
        if (l16 < 8) {
            rsc[8 * rq + i] = make_float2(o.s, o.r);
            sr[(tok0 + 8 * rq + i) * nbr + blockIdx.x] = o.s;
        }
    }
    __syncthreads();
    if (t < 128) {
        const uint32_t m = pmax16(pmax16(red[0][t >> 1], red[1][t >> 1]), pmax16(red[2][t >> 1], red[3][t >> 1]));
        const ScaleRcp o = scale_rcp((t & 1) ? ((m >> 1) & 0x7FFF0000u) : ((m & 0xFFFFu) << 15), pow2);
        scl[t] = o.s;
        rcl[t] = o.r;
        st[(col0 + t) * ntb + blockIdx.y] = o.s;
        slow = slow || slow_div(o.s, o.r);
    }
    uint8_t *qr_t = qr + tok0 * ldqr + col0;
    if (__syncthreads_or(slow))
        dual_bf16_slow(src_t, rsc, scl, rcl, tile, qr_t, ldqr, rq, cc);
    else
        dual_bf16_quant<false>(raw, rsc, scl, rcl, tile, qr_t, ldqr, rq, cc);
    __syncthreads();
    uint8_t *qt_t = qt + col0 * ldqt + tok0;
#pragma unroll
    for (int it = 0; it < 4; it++) {
        const int chunk = t + 256 * it;
        const int row = chunk >> 3, seg = chunk & 7;
        const uint32_t *src = &tile[row][seg * 4];
        store_nt(qt_t + row * ldqt + seg * 16, src[0], src[1], src[2], src[3]);
    }
}

__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(8)))
void quant_dual_bf16_kernel(const uint16_t *__restrict__ x, int ldx, uint8_t *__restrict__ qr,
                            int ldqr, float *__restrict__ sr, int64_t nbr,
                            uint8_t *__restrict__ qt, int ldqt, float *__restrict__ st,
                            int64_t ntb, int pow2)
{
    dual_bf16_tile(DualPlain{x, ldx}, qr, ldqr, sr, nbr, qt, ldqt, st, ntb, pow2);
}

// The same with the tile's values formed as silu(gate) * up (and stored to h
// unless h is NULL).
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(4)))
void swiglu_dual_bf16_kernel(const uint16_t *__restrict__ g, int ldg, const uint16_t *__restrict__ u,
                             int ldu, uint16_t *__restrict__ h, int ldh, uint8_t *__restrict__ qr,
                             int ldqr, float *__restrict__ sr, int64_t nbr,
                             uint8_t *__restrict__ qt, int ldqt, float *__restrict__ st,
                             int64_t ntb, int pow2)
{
    dual_bf16_tile(DualSwiglu{g, u, h, ldg, ldu, ldh}, qr, ldqr, sr, nbr, qt, ldqt, st, ntb, pow2);
}

// ---------------------------------------------------------------------------

hipError_t launch_quant_act(const void *x, bool bf16, int64_t rows, int64_t cols, int64_t ldx,
                            uint8_t *q, int64_t ldq, float *s, bool pow2, hipStream_t st)
{
    const int64_t nb = (cols + 127) / 128;
    const int64_t groups = rows * ((nb + BPG - 1) / BPG);
    if (groups == 0)
        return hipSuccess;
    const dim3 grid((unsigned)((groups + 15) / 16));
    if (bf16)
        hipLaunchKernelGGL(quant_act_kernel<uint16_t>, grid, dim3(256), 0, st,
                           (const uint16_t *)x, rows, cols, ldx, q, ldq, s, nb, (int)pow2);
    else
        hipLaunchKernelGGL(quant_act_kernel<float>, grid, dim3(256), 0, st, (const float *)x, rows,
                           cols, ldx, q, ldq, s, nb, (int)pow2);
    return hipGetLastError();
}

hipError_t launch_quant_weight(const void *w, bool bf16, int64_t rows, int64_t cols, int64_t ldw,
                               uint8_t *q, int64_t ldq, float *s, bool pow2, hipStream_t st)
{
    const int64_t rb = (rows + 127) / 128, cb = (cols + 127) / 128;
    if (rb == 0 || cb == 0)
        return hipSuccess;
    const dim3 grid((unsigned)cb, (unsigned)rb);
    if (bf16)
        hipLaunchKernelGGL(quant_weight_kernel<uint16_t>, grid, dim3(1024), 0, st,
                           (const uint16_t *)w, rows, cols, ldw, q, ldq, s, cb, (int)pow2);
    else
        hipLaunchKernelGGL(quant_weight_kernel<float>, grid, dim3(1024), 0, st, (const float *)w,
                           rows, cols, ldw, q, ldq, s, cb, (int)pow2);
    return hipGetLastError();
}

hipError_t launch_quant_weight_group(const QuantWeightItem *items, int count, bool bf16, bool pow2,
                                     hipStream_t st)
{
    for (int lo = 0; lo < count; lo += kQuantGroupMax) {
        QuantWeightGroup g;
        g.count = 0;
        g.first[0] = 0;
        g.pow2 = pow2 ? 1 : 0;
        for (int i = lo; i < count && g.count < kQuantGroupMax; i++) {
            const int64_t tiles = ((items[i].rows + 127) / 128) * items[i].cb;
            if (tiles == 0)
                continue;   // empty weight: nothing to do
            g.it[g.count] = items[i];
            g.first[g.count + 1] = g.first[g.count] + (int)tiles;
            g.count++;
        }
        if (g.count == 0)
            continue;
        const dim3 grid((unsigned)g.first[g.count]);
        if (bf16)
            hipLaunchKernelGGL(quant_weight_group_kernel<uint16_t>, grid, dim3(1024), 0, st, g);
        else
            hipLaunchKernelGGL(quant_weight_group_kernel<float>, grid, dim3(1024), 0, st, g);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess)
            return e;
    }
    return hipSuccess;
}

hipError_t launch_quant_transpose(const void *x, bool bf16, int64_t tokens, int64_t cols,
                                  int64_t ldx, bool transpose_out, uint8_t *q, int64_t ldq,
                                  float *s, bool pow2, hipStream_t st)
{
    const int64_t ntb = (tokens + 127) / 128, ncg = (cols + 63) / 64;
    if (ntb == 0 || ncg == 0)
        return hipSuccess;
    const dim3 grid((unsigned)ncg, (unsigned)ntb);
    if (bf16) {
        if (transpose_out)
            hipLaunchKernelGGL((quant_transpose_kernel<uint16_t, true>), grid, dim3(256), 0, st,
                               (const uint16_t *)x, tokens, cols, ldx, q, ldq, s, ntb, (int)pow2);
        else
            hipLaunchKernelGGL((quant_transpose_kernel<uint16_t, false>), grid, dim3(256), 0, st,
                               (const uint16_t *)x, tokens, cols, ldx, q, ldq, s, ntb, (int)pow2);
    } else {
        if (transpose_out)
            hipLaunchKernelGGL((quant_transpose_kernel<float, true>), grid, dim3(256), 0, st,
                               (const float *)x, tokens, cols, ldx, q, ldq, s, ntb, (int)pow2);
        else
            hipLaunchKernelGGL((quant_transpose_kernel<float, false>), grid, dim3(256), 0, st,
                               (const float *)x, tokens, cols, ldx, q, ldq, s, ntb, (int)pow2);
    }
    return hipGetLastError();
}

// The gate's partner and the activation output of the fused SwiGLU variant.
struct SwigluIn {
    const uint16_t *u;
    int64_t ldu;
    uint16_t *h;
    int64_t ldh;
};

static hipError_t dual_launch(const void *x, bool bf16, int64_t tokens, int64_t cols, int64_t ldx,
                              uint8_t *qr, int64_t ldqr, float *sr, bool transpose_out, uint8_t *qt,
                              int64_t ldqt, float *st, bool pow2, const SwigluIn *sw, hipStream_t stream)
{
    const int64_t ntb = (tokens + 127) / 128, ncb = (cols + 127) / 128;
    if (ntb == 0 || ncb == 0)
        return hipSuccess;
    // full tiles of BF16 input with a transposed token-block copy: packed kernel
    // (in-tile offsets of at most 127 leading dimensions must fit 32 bits)
    int64_t fb_x = 0, fb_y = 0;
    const int64_t lim = ((int64_t)1 << 31) / 256;
    const bool sw_ld_ok = !sw || (sw->ldu < lim && sw->ldh < lim);
    if (bf16 && transpose_out && ldx < lim && ldqr < lim && ldqt < lim && sw_ld_ok) {
        fb_x = cols / 128;
        fb_y = tokens / 128;
        if (fb_x > 0 && fb_y > 0) {
            const dim3 grid((unsigned)fb_x, (unsigned)fb_y);
            if (sw)
                hipLaunchKernelGGL(swiglu_dual_bf16_kernel, grid, dim3(256), 0, stream, (const uint16_t *)x,
                                   (int)ldx, sw->u, (int)sw->ldu, sw->h, (int)sw->ldh, qr, (int)ldqr, sr, ncb,
                                   qt, (int)ldqt, st, ntb, (int)pow2);
            else
                hipLaunchKernelGGL(quant_dual_bf16_kernel, grid, dim3(256), 0, stream, (const uint16_t *)x,
                                   (int)ldx, qr, (int)ldqr, sr, ncb, qt, (int)ldqt, st, ntb, (int)pow2);
        } else {
            fb_x = fb_y = 0;
        }
    }
    // the rest: tiles right of the full columns (all token tiles), then the tiles
    // below the full rows (full columns only)
    const uint16_t *u = sw ? sw->u : nullptr;
    uint16_t *h = sw ? sw->h : nullptr;
    const int64_t ldu = sw ? sw->ldu : 0, ldh = sw ? sw->ldh : 0;
    auto rest = [&](dim3 grid, int bx0, int by0) {
#define PURO_DUAL(T, TR, SW)                                                                          \
    hipLaunchKernelGGL((quant_dual_kernel<T, TR, SW>), grid, dim3(256), 0, stream, (const T *)x, tokens, \
                       cols, ldx, qr, ldqr, sr, ncb, qt, ldqt, st, ntb, (int)pow2, bx0, by0, u, ldu, h, ldh)
        if (sw) {
            if (transpose_out)
                PURO_DUAL(uint16_t, true, true);
            else
                PURO_DUAL(uint16_t, false, true);
        } else if (bf16) {
            if (transpose_out)
                PURO_DUAL(uint16_t, true, false);
            else
                PURO_DUAL(uint16_t, false, false);
        } else {
            if (transpose_out)
                PURO_DUAL(float, true, false);
            else
                PURO_DUAL(float, false, false);
        }
#undef PURO_DUAL
    };
    if (fb_x == 0 || fb_y == 0) {
        rest(dim3((unsigned)ncb, (unsigned)ntb), 0, 0);
    } else {
        if (ncb > fb_x)
            rest(dim3((unsigned)(ncb - fb_x), (unsigned)ntb), (int)fb_x, 0);
        if (ntb > fb_y)
            rest(dim3((unsigned)fb_x, (unsigned)(ntb - fb_y)), 0, (int)fb_y);
    }
    return hipGetLastError();
}

hipError_t launch_quant_dual(const void *x, bool bf16, int64_t tokens, int64_t cols, int64_t ldx,
                             uint8_t *qr, int64_t ldqr, float *sr, bool transpose_out, uint8_t *qt,
                             int64_t ldqt, float *st, bool pow2, hipStream_t stream)
{
    return dual_launch(x, bf16, tokens, cols, ldx, qr, ldqr, sr, transpose_out, qt, ldqt, st, pow2, nullptr,
                       stream);
}

hipError_t launch_swiglu_dual(const uint16_t *g, int64_t ldg, const uint16_t *u, int64_t ldu, uint16_t *h,
                              int64_t ldh, int64_t tokens, int64_t cols, uint8_t *qr, int64_t ldqr, float *sr,
                              bool transpose_out, uint8_t *qt, int64_t ldqt, float *st, bool pow2,
                              hipStream_t stream)
{
    const SwigluIn sw{u, ldu, h, h ? ldh : 0};   // ldh means nothing without h
    return dual_launch(g, true, tokens, cols, ldg, qr, ldqr, sr, transpose_out, qt, ldqt, st, pow2, &sw,
                       stream);
}

} // namespace puro
