// Blockwise E4M3 quantisers for gfx950.
//
// Each block of values x_i gets one FP32 dequantisation scale
//   s = fl32(amax / 448),  q_i = E4M3_RNE(fl32(x_i / s)),
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
// 1x128 row blocks.  One 16-lane group per block, 8 consecutive elements per
// lane (one 16-byte load for BF16, two for FP32), amax by cross-lane max.
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(256) void quant_act_kernel(const T *__restrict__ x, int64_t rows,
                                                        int64_t cols, int64_t ldx,
                                                        uint8_t *__restrict__ q, int64_t ldq,
                                                        float *__restrict__ s, int64_t nb)
{
    const int64_t blk = ((int64_t)blockIdx.x * 256 + threadIdx.x) >> 4;
    if (blk >= rows * nb)
        return;  // whole 16-lane groups leave together
    const int l16 = threadIdx.x & 15;
    const int64_t r = blk / nb;
    const int64_t b = blk - r * nb;
    const int64_t c0 = b * 128 + l16 * 8;
    const bool full = (b * 128 + 128 <= cols);
    const T *xr = x + r * ldx;

    float v[8];
    if (full) {
        Elem<T>::load8(xr + c0, v);
    } else {
#pragma unroll
        for (int i = 0; i < 8; i++)
            v[i] = (c0 + i < cols) ? Elem<T>::load(xr + c0 + i) : 0.0f;
    }
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; i++)
        amax = fmaxf(amax, fabsf(v[i]));
#pragma unroll
    for (int off = 8; off >= 1; off >>= 1)
        amax = fmaxf(amax, __shfl_xor(amax, off, 16));
    const float sc = amax / 448.0f;

    const uint32_t lo = quant4(v[0], v[1], v[2], v[3], sc);
    const uint32_t hi = quant4(v[4], v[5], v[6], v[7], sc);
    uint8_t *qr = q + r * ldq;
    if (full) {
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

// ---------------------------------------------------------------------------
// 128x128 weight tiles.  One workgroup per tile; thread t owns columns
// 8*(t%16) .. +7 of rows t/16 + 16 i (i = 0..7): 64 values in registers.
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(256) void quant_weight_kernel(const T *__restrict__ w, int64_t rows,
                                                           int64_t cols, int64_t ldw,
                                                           uint8_t *__restrict__ q, int64_t ldq,
                                                           float *__restrict__ s, int64_t cb)
{
    __shared__ float red[4];
    const int t = threadIdx.x;
    const int cc = t & 15, rg = t >> 4;
    const int64_t r0 = (int64_t)blockIdx.y * 128, cbase = (int64_t)blockIdx.x * 128;
    const int64_t c0 = cbase + cc * 8;
    const bool full_tile = (r0 + 128 <= rows) && (cbase + 128 <= cols);

    float v[8][8];
#pragma unroll
    for (int i = 0; i < 8; i++) {
        const int64_t r = r0 + rg + 16 * i;
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
    for (int i = 0; i < 8; i++)
#pragma unroll
        for (int j = 0; j < 8; j++)
            amax = fmaxf(amax, fabsf(v[i][j]));
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1)
        amax = fmaxf(amax, __shfl_xor(amax, off, 64));
    if ((t & 63) == 0)
        red[t >> 6] = amax;
    __syncthreads();
    amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    const float sc = amax / 448.0f;

#pragma unroll
    for (int i = 0; i < 8; i++) {
        const int64_t r = r0 + rg + 16 * i;
        const uint32_t lo = quant4(v[i][0], v[i][1], v[i][2], v[i][3], sc);
        const uint32_t hi = quant4(v[i][4], v[i][5], v[i][6], v[i][7], sc);
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
// per workgroup.  Thread t owns columns 8*(t%8) .. +7 of tokens t/8 + 32 i
// (i = 0..3).  Column amax: per-thread max over its 4 tokens, cross-lane max
// over lanes with equal t%8, then across the 4 waves through LDS.  The
// transposed output is assembled in LDS and written as 128-byte rows.
// ---------------------------------------------------------------------------
template <typename T, bool TRANSPOSE_OUT>
__global__ __launch_bounds__(256) void quant_transpose_kernel(const T *__restrict__ x,
                                                              int64_t tokens, int64_t cols,
                                                              int64_t ldx, uint8_t *__restrict__ q,
                                                              int64_t ldq, float *__restrict__ s,
                                                              int64_t ntb)
{
    __shared__ float red[4][64];
    __shared__ float scl[64];
    __shared__ __attribute__((aligned(16))) uint8_t tile[64][128 + 16];

    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    const int cc = t & 7, rr = t >> 3;
    const int64_t tok0 = (int64_t)blockIdx.y * 128;
    const int64_t col0 = (int64_t)blockIdx.x * 64;
    const int64_t c0 = col0 + cc * 8;
    const bool full = (tok0 + 128 <= tokens) && (col0 + 64 <= cols);

    float v[4][8];
#pragma unroll
    for (int i = 0; i < 4; i++) {
        const int64_t tk = tok0 + rr + 32 * i;
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
        const float sc = amax / 448.0f;
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

    float scj[8];
#pragma unroll
    for (int j = 0; j < 8; j++)
        scj[j] = scl[cc * 8 + j];

#pragma unroll
    for (int i = 0; i < 4; i++) {
        uint32_t code[8];
#pragma unroll
        for (int j = 0; j < 8; j++) {
            const float sc = scj[j];
            code[j] = (sc == 0.0f) ? sign_code(v[i][j])
                                   : ((uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(v[i][j] / sc, 0.0f, 0, false) & 0xFFu);
        }
        const int tl = rr + 32 * i;
        if (TRANSPOSE_OUT) {
#pragma unroll
            for (int j = 0; j < 8; j++)
                tile[cc * 8 + j][tl] = (uint8_t)code[j];
        } else {
            const int64_t tk = tok0 + tl;
            uint8_t *qr = q + tk * ldq;
            if (full) {
                *reinterpret_cast<uint2 *>(qr + c0) =
                    make_uint2(code[0] | (code[1] << 8) | (code[2] << 16) | (code[3] << 24),
                               code[4] | (code[5] << 8) | (code[6] << 16) | (code[7] << 24));
            } else if (tk < tokens) {
#pragma unroll
                for (int j = 0; j < 8; j++)
                    if (c0 + j < cols)
                        qr[c0 + j] = (uint8_t)code[j];
            }
        }
    }
    if (TRANSPOSE_OUT) {
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
            if (tk + 16 <= tokens) {
                *reinterpret_cast<uint4 *>(dst) = *reinterpret_cast<const uint4 *>(&tile[row][seg * 16]);
            } else {
                for (int e = 0; e < 16; e++)
                    if (tk + e < tokens)
                        dst[e] = tile[row][seg * 16 + e];
            }
        }
    }
}

// ---------------------------------------------------------------------------

hipError_t launch_quant_act(const void *x, bool bf16, int64_t rows, int64_t cols, int64_t ldx,
                            uint8_t *q, int64_t ldq, float *s, hipStream_t st)
{
    const int64_t nb = (cols + 127) / 128;
    const int64_t nblocks = rows * nb;
    if (nblocks == 0)
        return hipSuccess;
    const dim3 grid((unsigned)((nblocks + 15) / 16));
    if (bf16)
        hipLaunchKernelGGL(quant_act_kernel<uint16_t>, grid, dim3(256), 0, st,
                           (const uint16_t *)x, rows, cols, ldx, q, ldq, s, nb);
    else
        hipLaunchKernelGGL(quant_act_kernel<float>, grid, dim3(256), 0, st, (const float *)x, rows,
                           cols, ldx, q, ldq, s, nb);
    return hipGetLastError();
}

hipError_t launch_quant_weight(const void *w, bool bf16, int64_t rows, int64_t cols, int64_t ldw,
                               uint8_t *q, int64_t ldq, float *s, hipStream_t st)
{
    const int64_t rb = (rows + 127) / 128, cb = (cols + 127) / 128;
    if (rb == 0 || cb == 0)
        return hipSuccess;
    const dim3 grid((unsigned)cb, (unsigned)rb);
    if (bf16)
        hipLaunchKernelGGL(quant_weight_kernel<uint16_t>, grid, dim3(256), 0, st,
                           (const uint16_t *)w, rows, cols, ldw, q, ldq, s, cb);
    else
        hipLaunchKernelGGL(quant_weight_kernel<float>, grid, dim3(256), 0, st, (const float *)w,
                           rows, cols, ldw, q, ldq, s, cb);
    return hipGetLastError();
}

hipError_t launch_quant_transpose(const void *x, bool bf16, int64_t tokens, int64_t cols,
                                  int64_t ldx, bool transpose_out, uint8_t *q, int64_t ldq,
                                  float *s, hipStream_t st)
{
    const int64_t ntb = (tokens + 127) / 128, ncg = (cols + 63) / 64;
    if (ntb == 0 || ncg == 0)
        return hipSuccess;
    const dim3 grid((unsigned)ncg, (unsigned)ntb);
    if (bf16) {
        if (transpose_out)
            hipLaunchKernelGGL((quant_transpose_kernel<uint16_t, true>), grid, dim3(256), 0, st,
                               (const uint16_t *)x, tokens, cols, ldx, q, ldq, s, ntb);
        else
            hipLaunchKernelGGL((quant_transpose_kernel<uint16_t, false>), grid, dim3(256), 0, st,
                               (const uint16_t *)x, tokens, cols, ldx, q, ldq, s, ntb);
    } else {
        if (transpose_out)
            hipLaunchKernelGGL((quant_transpose_kernel<float, true>), grid, dim3(256), 0, st,
                               (const float *)x, tokens, cols, ldx, q, ldq, s, ntb);
        else
            hipLaunchKernelGGL((quant_transpose_kernel<float, false>), grid, dim3(256), 0, st,
                               (const float *)x, tokens, cols, ldx, q, ldq, s, ntb);
    }
    return hipGetLastError();
}

} // namespace puro
