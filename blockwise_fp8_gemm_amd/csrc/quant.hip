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
            *reinterpret_cast<uint2 *>(qr + c0) = make_uint2(lo, hi);
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
template <typename T>
__global__ __launch_bounds__(1024) void quant_weight_kernel(const T *__restrict__ w, int64_t rows,
                                                            int64_t cols, int64_t ldw,
                                                            uint8_t *__restrict__ q, int64_t ldq,
                                                            float *__restrict__ s, int64_t cb, int pow2)
{
    __shared__ float red[16];
    const int t = threadIdx.x;
    const int cc = t & 15, rg = t >> 4;
    const int64_t r0 = (int64_t)blockIdx.y * 128, cbase = (int64_t)blockIdx.x * 128;
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
            *reinterpret_cast<uint2 *>(qr + c0) = make_uint2(lo, hi);
        } else if (r < rows) {
#pragma unroll
            for (int j = 0; j < 8; j++)
                if (c0 + j < cols)
                    qr[c0 + j] = (uint8_t)(((j < 4 ? lo : hi) >> (8 * (j & 3))) & 0xFF);
        }
    }
    if (t == 0)
        s[blockIdx.y * cb + blockIdx.x] = sc;
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
                *reinterpret_cast<uint4 *>(dst) = make_uint4(src[0], src[1], src[2], src[3]);
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
                *reinterpret_cast<uint2 *>(qr + c0) =
                    make_uint2(b[0] | (b[1] << 8) | (b[2] << 16) | (b[3] << 24),
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
// t%16, then across the 4 waves through LDS.
// ---------------------------------------------------------------------------
template <typename T, bool TRANSPOSE_OUT>
__global__ __launch_bounds__(256) void quant_dual_kernel(const T *__restrict__ x, int64_t tokens,
                                                         int64_t cols, int64_t ldx,
                                                         uint8_t *__restrict__ qr, int64_t ldqr,
                                                         float *__restrict__ sr, int64_t nbr,
                                                         uint8_t *__restrict__ qt, int64_t ldqt,
                                                         float *__restrict__ st, int64_t ntb, int pow2)
{
    __shared__ float red[4][128];
    __shared__ float scl[128];
    __shared__ uint32_t tile[128][32 + 1];   // [column][token/4] codes, odd stride

    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    const int cc = t & 15, rq = t >> 4;
    const int64_t tok0 = (int64_t)blockIdx.y * 128;
    const int64_t col0 = (int64_t)blockIdx.x * 128;
    const int64_t c0 = col0 + cc * 8;
    const bool full = (tok0 + 128 <= tokens) && (col0 + 128 <= cols);

    float v[8][8];
#pragma unroll
    for (int i = 0; i < 8; i++) {
        const int64_t tk = tok0 + 8 * rq + i;
        const T *xr = x + tk * ldx;
        if (full) {
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
                st[c * ntb + blockIdx.y] = sc;
            else
                st[(int64_t)blockIdx.y * cols + c] = sc;
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
            *reinterpret_cast<uint2 *>(q + c0) = make_uint2(lo, hi);
        } else if (tk < tokens) {
#pragma unroll
            for (int j = 0; j < 8; j++)
                if (c0 + j < cols)
                    q[c0 + j] = (uint8_t)(((j < 4 ? lo : hi) >> (8 * (j & 3))) & 0xFF);
        }
        if (cc == 0 && tk < tokens)
            sr[tk * nbr + blockIdx.x] = sc;
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
                *reinterpret_cast<uint4 *>(dst) = make_uint4(src[0], src[1], src[2], src[3]);
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
                *reinterpret_cast<uint2 *>(q + c0) =
                    make_uint2(b[0] | (b[1] << 8) | (b[2] << 16) | (b[3] << 24),
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

hipError_t launch_quant_dual(const void *x, bool bf16, int64_t tokens, int64_t cols, int64_t ldx,
                             uint8_t *qr, int64_t ldqr, float *sr, bool transpose_out, uint8_t *qt,
                             int64_t ldqt, float *st, bool pow2, hipStream_t stream)
{
    const int64_t ntb = (tokens + 127) / 128, ncb = (cols + 127) / 128;
    if (ntb == 0 || ncb == 0)
        return hipSuccess;
    const dim3 grid((unsigned)ncb, (unsigned)ntb);
#define PURO_DUAL(T, TR)                                                                            \
    hipLaunchKernelGGL((quant_dual_kernel<T, TR>), grid, dim3(256), 0, stream, (const T *)x, tokens, \
                       cols, ldx, qr, ldqr, sr, ncb, qt, ldqt, st, ntb, (int)pow2)
    if (bf16) {
        if (transpose_out)
            PURO_DUAL(uint16_t, true);
        else
            PURO_DUAL(uint16_t, false);
    } else {
        if (transpose_out)
            PURO_DUAL(float, true);
        else
            PURO_DUAL(float, false);
    }
#undef PURO_DUAL
    return hipGetLastError();
}

} // namespace puro
