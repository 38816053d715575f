// Blockwise-scaled E4M3 GEMM on the gfx950 matrix cores.
//
//   C[m][n] = sum_kb sA(m,kb) * sB(n,kb) * P_kb[m][n],
//   P_kb[m][n] = sum_{k in block kb} a(m,k) b(k,n)
//
// P_kb (one 128-wide K block) is formed on the matrix cores from a zero
// accumulator, then promoted into FP32 accumulators with one FMA per element:
// acc = fma(sA*sB, P_kb, acc).  This is the FP8 linear-layer GEMM of the
// Puro-2B-Base model card's setup paragraph (blockwise E4M3, FP32 kept where
// needed), with the per-block promotion of the DeepSeek-V3 design the
// technical report's related-work paragraph cites.
//
// Three matrix-core datapaths, each behind its own entry point:
//  * F16 (puro_fp8_gemm): each E4M3 code is widened to FP16 in registers
//    (v_cvt_scalef32_pk_f16_fp8, exact: every E4M3 value is an FP16 value) and
//    P_kb is four chained v_mfma_f32_16x16x32_f16.  Measured on gfx950, these
//    sums are FP32-grade (relative error ~1e-8 on quantised data).
//  * FP8 (puro_fp8_gemm_native): one v_mfma_f32_16x16x128_f8f6f4 per block,
//    promoted the same way.  Twice the peak rate, but measured on gfx950 the
//    instruction adds each run of 8 consecutive products in a fixed-point
//    window about 13 bits below the largest of them, so small products next
//    to large ones are truncated (relative error ~1e-5 to 1e-4 on quantised
//    data).
//  * MX (puro_fp8_gemm_mx): power-of-two block scales applied inside
//    v_mfma_scale_f32_16x16x128_f8f6f4 as E8M0 exponents; no promotion step.
//
// Tiles: 128 x 128 per workgroup (4 waves of 64 x 64, two workgroups per CU)
// or 256 x 256 (8 waves of 128 x 64, one per CU), picked per problem by a
// host-side cost model from step times measured on gfx950.
//
// Register layouts, measured on gfx950: for v_mfma_f32_16x16x128_f8f6f4 lane l
// holds A row l%16 and B column l%16, bytes 0..31 being K slots
// 32*(l/16) .. +31 (the same K index in A and B); result register r of lane l
// is P[4*(l/16) + r][l%16].  The F16 path feeds bytes 8c .. 8c+7 of the same
// fragments to MFMA c (c = 0..3), keeping A and B K-aligned, with the same
// result layout.
//
// Operands whose K dimension is contiguous are staged in LDS as [row][128 k]
// with a 16-byte XOR swizzle and read with 16-byte loads; operands whose M or
// N dimension is contiguous (B of NN, A and B of TN) are staged as
// [128 k][row] and read with ds_read_b64_tr_b8, whose 8x16-byte transpose
// within each 16-lane group yields the same K-contiguous fragments.
#include "common.h"
#include "kernels.h"

#include <algorithm>
#include <cmath>
#include <vector>

namespace puro {

namespace {

constexpr int BM = 128, BN = 128, BK = 128;
constexpr int kMaxKSeg = kGemmMaxSeg;

// One K segment of a product: A, B and their scales over K indices 0 .. K-1.
struct KSeg {
    const uint8_t *A;
    const uint8_t *B;
    const float *sA;
    const float *sB;
    int64_t K, lda, ldb, KB;
};

// C (+)= sum over the segments of each segment's blockwise product; the
// segments share M, N and the output, and are accumulated in FP32 before the
// single rounding of the output.
struct GemmArgs {
    KSeg seg[kMaxKSeg];
    int nseg;
    int accumulate;   // 0: C = sum; 1: C = C + sum
    void *C;
    int64_t M, N, ldc, NB;
};

// Stage a 128 x 128-byte tile of a row-major byte matrix into LDS.
//   rows [row0, row0+128) limited to nrows, bytes [col0, col0+128) limited to ncols;
//   out-of-range bytes are zero.  SWZ: 16-byte segment index XOR (row & 7).
template <bool SWZ>
__device__ __forceinline__ void stage_tile(uint8_t *lds, const uint8_t *g, int64_t ld,
                                           int64_t row0, int64_t nrows, int64_t col0,
                                           int64_t ncols, int tid)
{
#pragma unroll
    for (int it = 0; it < 4; it++) {
        const int chunk = tid + 256 * it;
        const int row = chunk >> 3, seg = chunk & 7;
        const int64_t gr = row0 + row, gc = col0 + seg * 16;
        uint4 val = make_uint4(0, 0, 0, 0);
        if (gr < nrows) {
            const uint8_t *src = g + gr * ld + gc;
            if (gc + 16 <= ncols) {
                val = *reinterpret_cast<const uint4 *>(src);
            } else if (gc < ncols) {
                uint32_t w[4] = {0, 0, 0, 0};
                for (int e = 0; e < 16; e++)
                    if (gc + e < ncols)
                        w[e >> 2] |= (uint32_t)src[e] << (8 * (e & 3));
                val = make_uint4(w[0], w[1], w[2], w[3]);
            }
        }
        const int pseg = SWZ ? (seg ^ (row & 7)) : seg;
        *reinterpret_cast<uint4 *>(lds + row * 128 + pseg * 16) = val;
    }
}

// Fragment of a K-contiguous tile ([row][128 k], swizzled): 16 rows from row_base.
__device__ __forceinline__ v8i frag_kmajor(const uint8_t *lds, int row_base, int lane)
{
    const int row = row_base + (lane & 15);
    const int g = lane >> 4;
    const int s0 = (2 * g) ^ (row & 7), s1 = (2 * g + 1) ^ (row & 7);
    const uint4 lo = *reinterpret_cast<const uint4 *>(lds + row * 128 + s0 * 16);
    const uint4 hi = *reinterpret_cast<const uint4 *>(lds + row * 128 + s1 * 16);
    v8i f;
    f[0] = lo.x; f[1] = lo.y; f[2] = lo.z; f[3] = lo.w;
    f[4] = hi.x; f[5] = hi.y; f[6] = hi.z; f[7] = hi.w;
    return f;
}

// Fragment of an MN-contiguous tile ([128 k][128 mn], unswizzled): 16 columns from col_base.
__device__ __forceinline__ v8i frag_mnmajor(const uint8_t *lds, int col_base, int lane)
{
    const int i = lane & 15, g = lane >> 4;
    v8i f;
#pragma unroll
    for (int t = 0; t < 4; t++) {
        const int k = 32 * g + 8 * t + (i >> 1);
        const int c = col_base + 8 * (i & 1);
        typedef __attribute__((address_space(3))) v2i lds_v2i;
        const v2i r = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_v2i *)(lds + k * 128 + c));
        f[2 * t] = r[0];
        f[2 * t + 1] = r[1];
    }
    return f;
}

typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef _Float16 v2h __attribute__((ext_vector_type(2)));

// Bytes 8c .. 8c+7 of an E4M3 fragment as eight FP16 values (exact).
__device__ __forceinline__ v8h widen8(const v8i &f, int c)
{
    const v2h a = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((unsigned)f[2 * c], 1.0f, false);
    const v2h b = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((unsigned)f[2 * c], 1.0f, true);
    const v2h d = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((unsigned)f[2 * c + 1], 1.0f, false);
    const v2h e = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((unsigned)f[2 * c + 1], 1.0f, true);
    v8h r;
    r[0] = a[0]; r[1] = a[1]; r[2] = b[0]; r[3] = b[1];
    r[4] = d[0]; r[5] = d[1]; r[6] = e[0]; r[7] = e[1];
    return r;
}

// Sum over one 128-wide K block of a(m,k) b(k,n) for a 16x16 output tile, on
// the FP16 matrix cores (four chained v_mfma_f32_16x16x32_f16).
__device__ __forceinline__ v4f block_partial(const v8i &a, const v8i &b)
{
    const v4f zero = {0.0f, 0.0f, 0.0f, 0.0f};
    v4f p = __builtin_amdgcn_mfma_f32_16x16x32_f16(widen8(a, 0), widen8(b, 0), zero, 0, 0, 0);
    p = __builtin_amdgcn_mfma_f32_16x16x32_f16(widen8(a, 1), widen8(b, 1), p, 0, 0, 0);
    p = __builtin_amdgcn_mfma_f32_16x16x32_f16(widen8(a, 2), widen8(b, 2), p, 0, 0, 0);
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(widen8(a, 3), widen8(b, 3), p, 0, 0, 0);
}

template <int LAYOUT, int BGRAN, bool CBF16>
__global__ __launch_bounds__(256) void gemm_kernel(GemmArgs p)
{
    constexpr bool A_KMAJ = (LAYOUT != 2);
    constexpr bool B_KMAJ = (LAYOUT == 0);
    __shared__ __attribute__((aligned(16))) uint8_t lds_a[BM * BK];
    __shared__ __attribute__((aligned(16))) uint8_t lds_b[BN * BK];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int64_t m0 = (int64_t)blockIdx.y * BM, n0 = (int64_t)blockIdx.x * BN;

    float acc[4][4][4];
#pragma unroll
    for (int i = 0; i < 4; i++)
#pragma unroll
        for (int j = 0; j < 4; j++)
#pragma unroll
            for (int r = 0; r < 4; r++)
                acc[i][j][r] = 0.0f;

    // Rows (m) and columns (n) of this lane's accumulator elements.
    int64_t mrow[4][4], ncol[4];
#pragma unroll
    for (int i = 0; i < 4; i++)
#pragma unroll
        for (int r = 0; r < 4; r++)
            mrow[i][r] = m0 + wm * 64 + i * 16 + 4 * (lane >> 4) + r;
#pragma unroll
    for (int j = 0; j < 4; j++)
        ncol[j] = n0 + wn * 64 + j * 16 + (lane & 15);

    for (int sgi = 0; sgi < p.nseg; sgi++)
    for (int64_t kb = 0; kb < p.seg[sgi].KB; kb++) {
        const KSeg &sg = p.seg[sgi];
        const int64_t k0 = kb * BK;
        __syncthreads();
        if (A_KMAJ)
            stage_tile<true>(lds_a, sg.A, sg.lda, m0, p.M, k0, sg.K, tid);
        else
            stage_tile<false>(lds_a, sg.A, sg.lda, k0, sg.K, m0, p.M, tid);
        if (B_KMAJ)
            stage_tile<true>(lds_b, sg.B, sg.ldb, n0, p.N, k0, sg.K, tid);
        else
            stage_tile<false>(lds_b, sg.B, sg.ldb, k0, sg.K, n0, p.N, tid);
        __syncthreads();

        // Scales of this K block for this lane's rows and columns.
        float sa[4][4], sb[4];
#pragma unroll
        for (int i = 0; i < 4; i++)
#pragma unroll
            for (int r = 0; r < 4; r++) {
                const int64_t m = mrow[i][r];
                sa[i][r] = (m < p.M) ? (A_KMAJ ? sg.sA[m * sg.KB + kb] : sg.sA[kb * p.M + m]) : 0.0f;
            }
#pragma unroll
        for (int j = 0; j < 4; j++) {
            const int64_t n = ncol[j];
            float v = 0.0f;
            if (n < p.N) {
                if (LAYOUT == 0)
                    v = BGRAN ? sg.sB[(n >> 7) * sg.KB + kb] : sg.sB[n * sg.KB + kb];
                else
                    v = BGRAN ? sg.sB[kb * p.NB + (n >> 7)] : sg.sB[kb * p.N + n];
            }
            sb[j] = v;
        }

        v8i af[4], bf[4];
#pragma unroll
        for (int i = 0; i < 4; i++)
            af[i] = A_KMAJ ? frag_kmajor(lds_a, wm * 64 + i * 16, lane)
                           : frag_mnmajor(lds_a, wm * 64 + i * 16, lane);
#pragma unroll
        for (int j = 0; j < 4; j++)
            bf[j] = B_KMAJ ? frag_kmajor(lds_b, wn * 64 + j * 16, lane)
                           : frag_mnmajor(lds_b, wn * 64 + j * 16, lane);

#pragma unroll
        for (int i = 0; i < 4; i++)
#pragma unroll
            for (int j = 0; j < 4; j++) {
                const v4f P = block_partial(af[i], bf[j]);
#pragma unroll
                for (int r = 0; r < 4; r++)
                    acc[i][j][r] = fmaf(sa[i][r] * sb[j], P[r], acc[i][j][r]);
            }
    }

    // Epilogue: FP32 or BF16 (round to nearest even).
#pragma unroll
    for (int i = 0; i < 4; i++)
#pragma unroll
        for (int r = 0; r < 4; r++) {
            const int64_t m = mrow[i][r];
            if (m >= p.M)
                continue;
#pragma unroll
            for (int j = 0; j < 4; j++) {
                const int64_t n = ncol[j];
                if (n >= p.N)
                    continue;
                if (CBF16) {
                    uint16_t *c = reinterpret_cast<uint16_t *>(p.C) + m * p.ldc + n;
                    *c = to_bf16(p.accumulate ? __uint_as_float((uint32_t)*c << 16) + acc[i][j][r] : acc[i][j][r]);
                } else {
                    float *c = reinterpret_cast<float *>(p.C) + m * p.ldc + n;
                    *c = p.accumulate ? *c + acc[i][j][r] : acc[i][j][r];
                }
            }
        }
}

// ===========================================================================
// Fast path for aligned problems (M % TM == 0, N % TN == 0, K % 128 == 0).
//
// Workgroup tile TM x TN computed by WM x WN waves, each wave IT x JT MFMA
// tiles of 16 x 16 (so (16 IT) x (16 JT) outputs).  Each 128-wide K block of
// A and B is copied straight from HBM into LDS with global_load_lds_dwordx4
// (lane l's 16 bytes land at the wave's LDS base + 16 l, so lanes fetch
// permuted global addresses to produce the swizzled layout), double-buffered
// so that block kb+1 streams in while block kb is multiplied; one barrier per
// K block.  The block's scales travel the same way (4-byte direct loads).
//
// LDS layouts (bank-conflict-free fragment reads):
//   K-major tile [rows][128 B]: segment s of row r at s ^ (r & 7) ^ ((r >> 3) & 1)
//   MN-major tile [128 k][W B]: segment s of row k at s ^ mnswz<W>(k)
// ===========================================================================

typedef __attribute__((address_space(3))) v2i lds_v2i_t;

// GEMM outputs are stored non-temporally (`nt`): the kernel never reads them
// back, and the hint keeps hundreds of MB of dirty output lines from sitting
// in the caches, where their write-back slowed the quantiser launched next by
// about 10% (measured in the benchmarked step: dual quantiser 8.6 -> 7.7 ms per
// step, weight quantiser 1.94 -> 1.74 ms, the GEMMs unchanged).
typedef unsigned int v4u_t __attribute__((ext_vector_type(4)));
typedef unsigned int v2u_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ void store_out_nt(uint4 *p, uint4 v)
{
    const v4u_t w = {v.x, v.y, v.z, v.w};
    __builtin_nontemporal_store(w, reinterpret_cast<v4u_t *>(p));
}
__device__ __forceinline__ void store_out_nt(float4 *p, float4 v)
{
    const v4f w = {v.x, v.y, v.z, v.w};
    __builtin_nontemporal_store(w, reinterpret_cast<v4f *>(p));
}
__device__ __forceinline__ void store_out_nt(uint2 *p, uint2 v)
{
    const v2u_t w = {v.x, v.y};
    __builtin_nontemporal_store(w, reinterpret_cast<v2u_t *>(p));
}

// Direct copies from global memory to LDS (global_load_lds_*): lane l's bytes
// land at the LDS address in M0 plus size * l.  They are written as inline
// assembly, not through the compiler's builtin.  While a builtin copy is in
// flight the compiler treats every LDS read as completing out of order and
// waits for each with lgkmcnt(0), so a fragment read a row block ahead was
// waited for as soon as the next one was needed.  The hardware counts these
// copies in the vector-memory counter, which the K loop waits on explicitly
// (s_waitcnt before its barrier, and before the epilogue reuses a stage).
// Should the LDS counter also count them, a wait for it only becomes stricter.
// Each statement sets M0 itself; no other instruction of these kernels reads
// M0 (gfx9 and later LDS instructions do not).  The memory clobber keeps the
// copies in program order with every other memory access.
__device__ __forceinline__ uint32_t lds_addr(const void *p)
{
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void *)p;
}

// M0 is a reserved register, and clang says so about the clobber below; the
// clobber is kept so that the compiler knows M0 changed.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
// 16 bytes per lane from base + off (base wave-uniform, off a 32-bit per-lane
// byte offset).
__device__ __forceinline__ void load_lds16(const uint8_t *base, uint32_t off, uint8_t *lds_wave_base)
{
    asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1"
                 :: "v"(off), "s"(base), "s"(lds_addr(lds_wave_base)) : "memory", "m0");
}

// 4 bytes per lane from the lane's own address g.
__device__ __forceinline__ void load_lds4(const void *g, void *lds_wave_base)
{
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dword %0, off"
                 :: "v"(g), "s"(lds_addr(lds_wave_base)) : "memory", "m0");
}
#pragma clang diagnostic pop

// Swizzle of K-major stages: 16-byte segment s of row r sits at s ^ kswz(r).
// A fragment read (lane i: row base + i % 16, 16 bytes) then touches 16
// different 16-byte bank groups in every 16 consecutive lanes and 8 in every
// 8, so it is conflict-free whether the LDS serves 8 or 16 lanes of a
// 16-byte read per cycle.
__device__ __forceinline__ int kswz(int row)
{
    return (row & 7) ^ ((row >> 3) & 1);
}

// Swizzle of M- or N-contiguous stages ([128 k][W bytes]): segment s of row k
// sits at s ^ mnswz(k).  A transposed fragment read covers 8 consecutive rows
// per 16 lanes, and the next 16 lanes the rows 32 further on, which the
// (k & 7) term alone would put on the same banks; bit 5 of k moves them to
// the other half of each row's segments (bit 0 for 128-byte rows, bit 3 for
// 256-byte rows).
template <int W>
__device__ __forceinline__ int mnswz(int k)
{
    static_assert(W == 128 || W == 256, "stage widths of the tile configurations");
    return (k & 7) ^ (((k >> 5) & 1) << (W == 128 ? 0 : 3));
}

// The copies below address global memory as a wave-uniform base (scalar
// registers: the wave number is uniform) plus a 32-bit per-lane offset of at
// most 7 rows (the fast path needs leading dimensions below 2^28), the
// instruction's scalar-base form, so that the per-block address arithmetic
// runs on the scalar unit.

// Rows [row0, row0+ROWS) x bytes [k0, k0+128) of a K-contiguous operand, NW waves.
template <int ROWS, int NW>
__device__ __forceinline__ void fast_stage_k(uint8_t *t, const uint8_t *g, int64_t ld, int64_t row0,
                                             int64_t k0, int wave, int lane)
{
    static_assert((ROWS / 8) % NW == 0, "whole 1 KB chunks per wave");
#pragma unroll
    for (int it = 0; it < ROWS / 8 / NW; it++) {
        const int c = wave + NW * it;   // rows 8c .. 8c+7, lane's row 8c + lane / 8
        const int seg = (lane & 7) ^ (((lane >> 3) & 7) ^ (c & 1));   // kswz(8c + lane / 8)
        const uint8_t *base = g + (row0 + 8 * c) * ld + k0;
        const uint32_t off = (uint32_t)(lane >> 3) * (uint32_t)ld + (uint32_t)(seg * 16);
        load_lds16(base, off, t + c * 1024);
    }
}

// Rows k [k0, k0+128) x bytes [mn0, mn0+W) of an M- or N-contiguous operand, NW waves.
template <int W, int NW>
__device__ __forceinline__ void fast_stage_mn(uint8_t *t, const uint8_t *g, int64_t ld, int64_t k0,
                                              int64_t mn0, int wave, int lane)
{
    constexpr int SEGS = W / 16, RPC = 1024 / W;
    static_assert((128 / RPC) % NW == 0, "whole 1 KB chunks per wave");
#pragma unroll
    for (int it = 0; it < 128 / RPC / NW; it++) {
        const int c = wave + NW * it;   // rows RPC c .. RPC c + RPC - 1
        const int seg = (lane % SEGS) ^ mnswz<W>(c * RPC + lane / SEGS);
        const uint8_t *base = g + (k0 + RPC * c) * ld + mn0;
        const uint32_t off = (uint32_t)(lane / SEGS) * (uint32_t)ld + (uint32_t)(seg * 16);
        load_lds16(base, off, t + c * 1024);
    }
}

__device__ __forceinline__ v8i fast_frag_k(const uint8_t *t, int row_base, int lane)
{
    const int row = row_base + (lane & 15);
    const int g = lane >> 4, f = kswz(row);
    // whole 16-byte vector loads (not four dword loads merged later), which
    // keeps each read's LDS object visible to the compiler
    const v4i lo = *reinterpret_cast<const v4i *>(t + (row * 128 + (((2 * g) ^ f) << 4)));
    const v4i hi = *reinterpret_cast<const v4i *>(t + (row * 128 + (((2 * g + 1) ^ f) << 4)));
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

template <int W>
__device__ __forceinline__ v8i fast_frag_mn(const uint8_t *t, int col_base, int lane)
{
    const int i = lane & 15, g = lane >> 4;
    const int seg = (col_base >> 4), within = 8 * (i & 1);
    v8i r;
#pragma unroll
    for (int q = 0; q < 4; q++) {
        const int k = 32 * g + 8 * q + (i >> 1);
        // one offset added to the stage pointer (not a chain of pointer
        // additions), which keeps the read's LDS object visible to the compiler
        const uint8_t *a = t + (k * W + ((seg ^ mnswz<W>(k)) << 4) + within);
        const v2i v = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_v2i_t *)a);
        r[2 * q] = v[0];
        r[2 * q + 1] = v[1];
    }
    return r;
}

// E8M0 encoding of a power-of-two scale 2^k, k in [-127, 127]: the biased
// exponent k + 127, which is the FP32 exponent field (0 for 2^-127, whose FP32
// encoding is subnormal with only the top mantissa bit set).
__device__ __forceinline__ int e8m0(float s)
{
    return (int)((__float_as_uint(s) >> 23) & 0xFFu);
}

struct V8H4 {
    v8h c[4];
};

__device__ __forceinline__ V8H4 widen32(const v8i &f)
{
    V8H4 h;
#pragma unroll
    for (int q = 0; q < 4; q++)
        h.c[q] = widen8(f, q);
    return h;
}

template <int WM_, int WN_, int IT_, int JT_, int STAGES_>
struct FastCfg {
    static constexpr int WM = WM_, WN = WN_, IT = IT_, JT = JT_, STAGES = STAGES_;
    static constexpr int NW = WM * WN, THREADS = 64 * NW;
    static constexpr int TM = WM * IT * 16, TN = WN * JT * 16;
    static constexpr int A_BYTES = TM * 128, B_BYTES = TN * 128;
    // direct copies each wave issues per K block: A and B tiles in 1 KB
    // pieces, plus one 4-byte-per-lane copy for the block's scales
    static constexpr int LOADS = TM / 8 / NW + TN / 8 / NW + 1;
    // K loop unrolled by the two stages, so that each stage is addressed by a
    // compile-time name: the compiler then sees that the copies into one stage
    // do not touch the other and lets the copies overlap the reads.
    static constexpr bool STATIC_STAGES = true;
    // Stage unconditionally (an idle copy after the last block): the 8-wave
    // tile has no registers for the partials of two blocks at once, which
    // is what the compiler builds when a branch separates them.
    static constexpr bool IDLE_COPY = NW > 4;
};

// 256 x 256 workgroup tiles (8 waves of 128 x 64, two LDS stages, one
// workgroup per CU) and 128 x 128 tiles (4 waves of 64 x 64, two LDS stages,
// two workgroups per CU).
typedef FastCfg<2, 4, 8, 4, 2> CfgL;
typedef FastCfg<2, 2, 4, 4, 2> CfgQ;
enum { CFG_L = 0, CFG_Q = 1 };

// Split-K: workgroup b handles K blocks [kb_lo, kb_hi) of split s = b / tiles
// and, with OUT_PARTIAL, stores FP32 partial sums to ws[s][M][N] (row stride N)
// instead of C; gemm_split_reduce then adds the splits in order.
// Position of tile t (of tiles_m x tiles_n) in the walk order: groups of 8 tile
// rows, column by column inside a group, so that the workgroups resident
// together share A and B panels in L2.
__device__ __forceinline__ void tile_coords(int t, int tiles_m, int tiles_n, int &tm, int &tn)
{
    constexpr int GROUP = 8;
    const int group = t / (GROUP * tiles_n);
    const int first_m = group * GROUP;
    const int gm = min(tiles_m - first_m, GROUP);
    tm = first_m + (t % (GROUP * tiles_n)) % gm;
    tn = (t % (GROUP * tiles_n)) / gm;
}

// Workgroups are dispatched round-robin over the 8 XCDs.  Maps dispatch index
// b of a range of n workgroups (n a multiple of 8) so that each XCD gets a
// contiguous eighth of the range.
__device__ __forceinline__ int xcd_contiguous(int b, int n)
{
    return (n & 7) ? b : (b & 7) * (n >> 3) + (b >> 3);
}

// Matrix-core datapaths of the tile kernels.
//  DP_F16: E4M3 widened to FP16, block partials on FP16 matrix cores
//          (FP32-grade sums), promoted with one FMA per element.
//  DP_MX:  power-of-two scales applied by the scaled FP8 matrix cores as
//          E8M0 exponents; no promotion step.
//  DP_FP8: block partials on the FP8 matrix cores as they are, promoted with
//          one FMA per element; the instruction's own accumulation of each
//          run of products is not FP32-exact.
enum { DP_F16 = 0, DP_MX = 1, DP_FP8 = 2 };

// One workgroup's output tile: rows [m0, m0 + TM) x columns [n0, n0 + TN) of
// problem p, over K blocks [kb_lo, kb_hi) numbered across its segments.  With
// OUT_PARTIAL the FP32 result goes to ws[split][M][N] (row stride N) instead
// of C.  MULTI: p may have more than one segment.  DP: the datapath above.
template <class Cfg, int LAYOUT, int BGRAN, bool CBF16, bool OUT_PARTIAL, bool MULTI, int DP = DP_F16>
__device__ __forceinline__ void fast_tile(const GemmArgs &p, int64_t m0, int64_t n0, int64_t kb_lo,
                                          int64_t kb_hi, int split, float *ws)
{
    constexpr bool A_KMAJ = (LAYOUT != 2);
    constexpr bool B_KMAJ = (LAYOUT == 0);
    constexpr int NW = Cfg::NW, TM = Cfg::TM, TN = Cfg::TN, IT = Cfg::IT, JT = Cfg::JT;
    constexpr int A_BYTES = Cfg::A_BYTES, B_BYTES = Cfg::B_BYTES;
    static_assert(TN % 128 == 0 || !BGRAN || TN <= 128, "tile columns within 128-wide weight tiles");
    static_assert(Cfg::STAGES == 2, "two LDS stages");
    // Two stages in distinct LDS objects.  With STATIC_STAGES the K loop names
    // them only at compile time, so the compiler can tell a stage being filled
    // by direct copies from the one being read and does not make the reads wait
    // for the copies in flight.
    __shared__ __attribute__((aligned(16))) uint8_t lds0[A_BYTES + B_BYTES];
    __shared__ __attribute__((aligned(16))) uint8_t lds1[A_BYTES + B_BYTES];
    // per stage: A scales [0, TM), B scales from TM on, then unused slots
    __shared__ __attribute__((aligned(16))) float lds_sc0[NW * 64];
    __shared__ __attribute__((aligned(16))) float lds_sc1[NW * 64];
    static_assert(TM + TN <= NW * 64, "one scale slot per lane");
    constexpr bool MX = DP == DP_MX;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: keeps wave-level addresses scalar
    const int wm = wave / Cfg::WN, wn = wave % Cfg::WN;

    float acc[IT][JT][4];
#pragma unroll
    for (int i = 0; i < IT; i++)
#pragma unroll
        for (int j = 0; j < JT; j++)
#pragma unroll
            for (int r = 0; r < 4; r++)
                acc[i][j][r] = 0.0f;

    // K blocks are numbered across the segments, in order: block v of the
    // product is block v - (blocks of the segments before) of its segment.
    // Scales: thread q copies, for every K block, A's scale of tile row q
    // (q < TM), then B's scales (one per tile column, or one per 128-wide
    // weight tile), then harmless duplicates of A's first, so that every wave
    // issues the same copies.
    const int nsb = BGRAN ? TN / 128 : TN;
    // This thread's scale source for block kb of segment sg: base + kb * step.
    auto scale_source = [&](const KSeg &sg, const float *&base, int64_t &step) {
        if (tid < TM) {
            const int64_t m = m0 + tid;
            base = A_KMAJ ? sg.sA + m * sg.KB : sg.sA + m;
            step = A_KMAJ ? 1 : p.M;
        } else if (tid < TM + nsb) {
            const int64_t q = tid - TM;
            if (BGRAN) {
                const int64_t nb = (n0 >> 7) + q;
                base = B_KMAJ ? sg.sB + nb * sg.KB : sg.sB + nb;
                step = B_KMAJ ? 1 : p.NB;
            } else {
                const int64_t n = n0 + q;
                base = B_KMAJ ? sg.sB + n * sg.KB : sg.sB + n;
                step = B_KMAJ ? 1 : p.N;
            }
        } else {
            base = A_KMAJ ? sg.sA + m0 * sg.KB : sg.sA + m0;
            step = A_KMAJ ? 1 : p.M;
        }
    };
    auto stage_seg = [&](const KSeg &sg, int64_t kb, const float *sc, uint8_t *L, float *LSC) {
        const int64_t k0 = kb * 128;
        uint8_t *ta = L;
        uint8_t *tb = L + A_BYTES;
        if (A_KMAJ)
            fast_stage_k<TM, NW>(ta, sg.A, sg.lda, m0, k0, wave, lane);
        else
            fast_stage_mn<TM, NW>(ta, sg.A, sg.lda, k0, m0, wave, lane);
        if (B_KMAJ)
            fast_stage_k<TN, NW>(tb, sg.B, sg.ldb, n0, k0, wave, lane);
        else
            fast_stage_mn<TN, NW>(tb, sg.B, sg.ldb, k0, n0, wave, lane);
        load_lds4(sc, &LSC[wave * 64]);
    };

    // One segment (the common case): operands and scale source fixed.
    const KSeg seg0 = p.seg[0];
    const float *sc0_base;
    int64_t sc0_step;
    scale_source(seg0, sc0_base, sc0_step);
    auto stage = [&](int64_t v, uint8_t *L, float *LSC) {
        stage_seg(seg0, v, sc0_base + v * sc0_step, L, LSC);
    };

    // K block kb of a run of blocks [.., end) with fixed operands, computed
    // from stage (L, LSC) while the run's block kb + 1 is copied into the
    // other stage (LN, LSCN) by stg.
    auto kblock = [&](auto &&stg, int64_t kb, int64_t end, const uint8_t *L, const float *LSC, uint8_t *LN,
                      float *LSCN) {
        __builtin_amdgcn_s_waitcnt(0);   // this wave's copies of block kb have landed
        __syncthreads();   // everyone's have; block kb-1 (in LN) is no longer read
        if constexpr (Cfg::IDLE_COPY) {
            // the next block, or block kb again after the last one (into an
            // idle stage, never read): no branch in the K loop, so the
            // compiler cannot move a block's promotion past the next block's
            // staging (which keeps every block's partials live at once)
            stg(kb + 1 < end ? kb + 1 : kb, LN, LSCN);
        } else if (kb + 1 < end) {
            stg(kb + 1, LN, LSCN);
        }

        const uint8_t *ta = L;
        const uint8_t *tb = L + A_BYTES;
        const int wrow = wm * IT * 16, wcol = wn * JT * 16;

        if constexpr (MX) {
            // Scaled matrix cores: the E8M0 exponent of each power-of-two block
            // scale goes to the MFMA, which scales the block's partial by
            // sA sB and adds it to the accumulator (no promotion step and no
            // widening: the MFMA takes the E4M3 codes as they are).
            static_assert(!BGRAN || 128 % (JT * 16) == 0, "wave columns within one weight tile");
            int sbe[JT];
            v8i bf[JT];
#pragma unroll
            for (int j = 0; j < JT; j++) {
                sbe[j] = e8m0(BGRAN ? LSC[TM + (wcol >> 7)] : LSC[TM + wcol + j * 16 + (lane & 15)]);
                bf[j] = B_KMAJ ? fast_frag_k(tb, wcol + j * 16, lane) : fast_frag_mn<TN>(tb, wcol + j * 16, lane);
            }
            // Each row block's A fragment and scale are read one row block ahead
            // (before this block's MFMAs are issued, a fence keeping the order),
            // so that the MFMAs never wait for the LDS read just before them.
            v8i af_next = A_KMAJ ? fast_frag_k(ta, wrow, lane) : fast_frag_mn<TM>(ta, wrow, lane);
            float sa_next = LSC[wrow + (lane & 15)];
#pragma unroll
            for (int i = 0; i < IT; i++) {
                const v8i af = af_next;
                const int sae = e8m0(sa_next);
                if (i + 1 < IT) {
                    af_next = A_KMAJ ? fast_frag_k(ta, wrow + (i + 1) * 16, lane)
                                     : fast_frag_mn<TM>(ta, wrow + (i + 1) * 16, lane);
                    sa_next = LSC[wrow + (i + 1) * 16 + (lane & 15)];
                }
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int j = 0; j < JT; j++) {
                    v4f c = {acc[i][j][0], acc[i][j][1], acc[i][j][2], acc[i][j][3]};
                    c = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(af, bf[j], c, 0, 0, 0, sae, 0, sbe[j]);
#pragma unroll
                    for (int r = 0; r < 4; r++)
                        acc[i][j][r] = c[r];
                }
                __builtin_amdgcn_sched_barrier(0);
            }
        } else if constexpr (DP == DP_FP8) {
            // Native FP8 matrix cores: one v_mfma_f32_16x16x128_f8f6f4 per 16x16
            // tile and K block (zero scale operands select the unscaled
            // instruction), promoted like the F16 path.
            static_assert(!BGRAN || 128 % (JT * 16) == 0, "wave columns within one weight tile");
            float sbv[JT];
            v8i bf[JT];
#pragma unroll
            for (int j = 0; j < JT; j++) {
                sbv[j] = BGRAN ? LSC[TM + (wcol >> 7)] : LSC[TM + wcol + j * 16 + (lane & 15)];
                bf[j] = B_KMAJ ? fast_frag_k(tb, wcol + j * 16, lane) : fast_frag_mn<TN>(tb, wcol + j * 16, lane);
            }
            // As on the MX path, each row block's A fragment and scales are read
            // one row block ahead (except on 256 x 256 tiles with an N-contiguous
            // B, whose transposing reads leave no registers for it); and, as on
            // the FP16 path, a tile's promotion runs after the next tile's MFMA
            // is issued, so that its FMAs do not wait for the matrix core.
            constexpr bool PREFETCH = B_KMAJ || NW <= 4;
            v8i af_next = A_KMAJ ? fast_frag_k(ta, wrow, lane) : fast_frag_mn<TM>(ta, wrow, lane);
            float4 sa_next = *reinterpret_cast<const float4 *>(&LSC[wrow + 4 * (lane >> 4)]);
            v4f prev_P = {0.0f, 0.0f, 0.0f, 0.0f};
            float prev_s[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int i = 0; i < IT; i++) {
                if (!PREFETCH && i > 0) {
                    af_next = A_KMAJ ? fast_frag_k(ta, wrow + i * 16, lane) : fast_frag_mn<TM>(ta, wrow + i * 16, lane);
                    sa_next = *reinterpret_cast<const float4 *>(&LSC[wrow + i * 16 + 4 * (lane >> 4)]);
                }
                const v8i af = af_next;
                const float sa[4] = {sa_next.x, sa_next.y, sa_next.z, sa_next.w};
                if (PREFETCH && i + 1 < IT) {
                    af_next = A_KMAJ ? fast_frag_k(ta, wrow + (i + 1) * 16, lane)
                                     : fast_frag_mn<TM>(ta, wrow + (i + 1) * 16, lane);
                    sa_next = *reinterpret_cast<const float4 *>(&LSC[wrow + (i + 1) * 16 + 4 * (lane >> 4)]);
                }
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int j = 0; j < JT; j++) {
                    const v4f zero = {0.0f, 0.0f, 0.0f, 0.0f};
                    const v4f P = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(af, bf[j], zero, 0, 0, 0, 0, 0, 0);
                    // On 256 x 256 tiles a fence keeps the MFMA ahead of the FMAs
                    // that promote the tile before: left alone, the compiler
                    // issues those FMAs first and gives both partials the same
                    // registers, so that every MFMA waits for the one before it
                    // to drain (measured 9-13% slower; on 128 x 128 tiles, two
                    // workgroups per CU, the compiler's order measured 5% faster).
                    if constexpr (NW > 4)
                        __builtin_amdgcn_sched_barrier(0);
                    if (i > 0 || j > 0) {
                        const int pi = j > 0 ? i : i - 1, pj = j > 0 ? j - 1 : JT - 1;
#pragma unroll
                        for (int r = 0; r < 4; r++)
                            acc[pi][pj][r] = fmaf(prev_s[r], prev_P[r], acc[pi][pj][r]);
                    }
                    prev_P = P;
#pragma unroll
                    for (int r = 0; r < 4; r++)
                        prev_s[r] = sa[r] * sbv[j];
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
#pragma unroll
            for (int r = 0; r < 4; r++)
                acc[IT - 1][JT - 1][r] = fmaf(prev_s[r], prev_P[r], acc[IT - 1][JT - 1][r]);
        } else {

            // B's scales: with 128x128 weight tiles the wave's JT * 16 columns lie in
            // one tile, so one scale serves them all and sA * sB is formed once per
            // row; with 1x128 blocks each lane's column has its own scale.
            static_assert(!BGRAN || 128 % (JT * 16) == 0, "wave columns within one weight tile");
            float sbv[JT];
#pragma unroll
            for (int j = 0; j < JT; j++)
                sbv[j] = BGRAN ? LSC[TM + (wcol >> 7)] : LSC[TM + wcol + j * 16 + (lane & 15)];

            V8H4 bh[JT];
#pragma unroll
            for (int j = 0; j < JT; j++)
                bh[j] = widen32(B_KMAJ ? fast_frag_k(tb, wcol + j * 16, lane)
                                       : fast_frag_mn<TN>(tb, wcol + j * 16, lane));

            // A is widened one K sub-step (8 values per lane) at a time, right
            // before its MFMAs, and the next row block's fragment is read as soon
            // as the last sub-step of this one is widened; each sub-step runs over
            // all JT tiles so that no MFMA waits on the one just issued.  Larger
            // wave tiles (not INTERLEAVE) have no registers to spare for that:
            // there each tile's four MFMAs run back to back, and a tile's
            // promotion waits until the next tile's MFMAs are issued (two
            // partials live), so that its FMAs do not wait for the matrix core
            // to drain the chain they read.
            constexpr bool INTERLEAVE = IT * JT <= 16;
            v8i araw = A_KMAJ ? fast_frag_k(ta, wrow, lane) : fast_frag_mn<TM>(ta, wrow, lane);
            v4f prev_P = {0.0f, 0.0f, 0.0f, 0.0f};   // the last tile's partial, not yet promoted
            float prev_s[4] = {0.0f, 0.0f, 0.0f, 0.0f};   // and its scales
#pragma unroll
            for (int i = 0; i < IT; i++) {
                const float4 sa4 = *reinterpret_cast<const float4 *>(&LSC[wrow + i * 16 + 4 * (lane >> 4)]);
                const float sa[4] = {sa4.x, sa4.y, sa4.z, sa4.w};
                float sab[4];
#pragma unroll
                for (int r = 0; r < 4; r++)
                    sab[r] = sa[r] * sbv[0];
                auto scale = [&](int j, int r) { return BGRAN ? sab[r] : sa[r] * sbv[j]; };
                if (INTERLEAVE) {
                    v4f P[JT];
#pragma unroll
                    for (int q = 0; q < 4; q++) {
                        const v8h aq = widen8(araw, q);
                        if (q == 3 && i + 1 < IT)
                            araw = A_KMAJ ? fast_frag_k(ta, wrow + (i + 1) * 16, lane)
                                          : fast_frag_mn<TM>(ta, wrow + (i + 1) * 16, lane);
#pragma unroll
                        for (int j = 0; j < JT; j++) {
                            const v4f zero = {0.0f, 0.0f, 0.0f, 0.0f};
                            P[j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(aq, bh[j].c[q], q ? P[j] : zero, 0, 0, 0);
                        }
                    }
#pragma unroll
                    for (int j = 0; j < JT; j++)
#pragma unroll
                        for (int r = 0; r < 4; r++)
                            acc[i][j][r] = fmaf(scale(j, r), P[j][r], acc[i][j][r]);
                } else {
                    // Row block i, in issue order: tile 0's four MFMAs, each after
                    // the widening of its K step of A; then tiles 1..JT-1, the
                    // MFMAs of each tile back to back.  After every MFMA comes one
                    // promotion FMA of the tile before (its chain has drained by
                    // then), with scheduling fences on both sides, so that each
                    // MFMA issues before the FMA and the compiler keeps the MFMAs
                    // spread among the vector instructions instead of bunching
                    // them.  The next row block's A fragment is read after tile 0,
                    // whose widening frees this one's registers, and lands during
                    // tiles 1..JT-1.
                    v8h ahq[4];
                    const float sav[4] = {sa4.x, sa4.y, sa4.z, sa4.w};
                    float rsc[4];   // sA sB of this lane's rows (128x128 B scales) or sA
#pragma unroll
                    for (int j = 0; j < JT; j++) {
                        v4f P;
#pragma unroll
                        for (int q = 0; q < 4; q++) {
                            if (j == 0)
                                ahq[q] = widen8(araw, q);
                            const v4f zero = {0.0f, 0.0f, 0.0f, 0.0f};
                            P = __builtin_amdgcn_mfma_f32_16x16x32_f16(ahq[q], bh[j].c[q], q ? P : zero, 0, 0, 0);
                            // the MFMA first, then the promotion of the tile before
                            __builtin_amdgcn_sched_barrier(0);
                            if (i > 0 || j > 0) {
                                // the tile before this one (compile-time indices)
                                const int pi = j > 0 ? i : i - 1, pj = j > 0 ? j - 1 : JT - 1;
                                acc[pi][pj][q] = fmaf(prev_s[q], prev_P[q], acc[pi][pj][q]);
                            }
                            if (j == 1 && q == 0 && i + 1 < IT)
                                araw = A_KMAJ ? fast_frag_k(ta, wrow + (i + 1) * 16, lane)
                                              : fast_frag_mn<TM>(ta, wrow + (i + 1) * 16, lane);
                            __builtin_amdgcn_sched_barrier(0);
                        }
                        prev_P = P;
                        if (j == 0) {
#pragma unroll
                            for (int r = 0; r < 4; r++)
                                rsc[r] = BGRAN ? sav[r] * sbv[0] : sav[r];
                        }
#pragma unroll
                        for (int r = 0; r < 4; r++)
                            prev_s[r] = BGRAN ? rsc[r] : rsc[r] * sbv[j];
                    }
                    if (i == IT - 1) {
#pragma unroll
                        for (int r = 0; r < 4; r++)
                            acc[IT - 1][JT - 1][r] = fmaf(prev_s[r], prev_P[r], acc[IT - 1][JT - 1][r]);
                    }
                }
            }
        }
    };
    // Blocks [b0, b1) of one run: the first is staged into stage 0, then each
    // is computed while the next is copied.
    auto run = [&](auto &&stg, int64_t b0, int64_t b1) {
        if (b0 < b1)
            stg(b0, lds0, lds_sc0);
        // the scaled-matrix-core form holds no widened fragments: it has the registers for
        // statically named stages in every configuration
        if constexpr (Cfg::STATIC_STAGES || DP != DP_F16) {
            // pairs of blocks, then an odd last block: no compute is
            // conditional inside the loop
            int64_t kb = b0;
            for (; kb + 2 <= b1; kb += 2) {
                kblock(stg, kb, b1, lds0, lds_sc0, lds1, lds_sc1);
                kblock(stg, kb + 1, b1, lds1, lds_sc1, lds0, lds_sc0);
            }
            if (kb < b1)
                kblock(stg, kb, b1, lds0, lds_sc0, lds1, lds_sc1);
        } else {
            // stage chosen at run time: every read of a stage waits for the copies in flight
            for (int64_t kb = b0; kb < b1; kb++) {
                const bool odd = ((kb - b0) & 1) != 0;
                kblock(stg, kb, b1, odd ? lds1 : lds0, odd ? lds_sc1 : lds_sc0, odd ? lds0 : lds1,
                       odd ? lds_sc0 : lds_sc1);
            }
        }
    };
    if constexpr (!MULTI) {
        run(stage, kb_lo, kb_hi);
    } else {
        // Several segments (the whole K range): one run per segment, so that the
        // K loop of each has its operands and scale source fixed.  A segment's
        // fields are picked with a constant index (they stay in scalar
        // registers); between runs every wave finishes the previous run's last
        // block before its stage is refilled.
        static_assert(kMaxKSeg == 4, "segment selection below");
        for (int si = 0; si < p.nseg; si++) {
            KSeg sg;
            switch (si) {
            case 0: sg = p.seg[0]; break;
            case 1: sg = p.seg[1]; break;
            case 2: sg = p.seg[2]; break;
            default: sg = p.seg[3]; break;
            }
            const float *scb;
            int64_t step;
            scale_source(sg, scb, step);
            auto stg = [&](int64_t kb, uint8_t *L, float *LSC) { stage_seg(sg, kb, scb + kb * step, L, LSC); };
            if (si > 0) {
                __builtin_amdgcn_s_waitcnt(0);   // the previous run's copies have all landed
                __syncthreads();
            }
            run(stg, 0, sg.KB);
        }
    }

    // Epilogue.  Each wave passes its results through a private LDS strip of
    // 16 rows x JT*16 columns so that every lane stores 16 contiguous bytes of
    // one row (the MFMA layout gives a lane one column of four rows).  The
    // strips live in stage 0, free once every wave has finished the last K
    // block (the barrier below); no copy is in flight by then.
    constexpr int CW = JT * 16;                              // strip width
    constexpr int SST = CW + 4;                              // row stride (floats): 4 row groups hit disjoint banks
    constexpr int CH = (CBF16 && !OUT_PARTIAL) ? 8 : 4;      // elements per 16-byte store
    constexpr int NCH = 16 * CW / CH;                        // 16-byte chunks per strip
    static_assert(NCH % 64 == 0, "whole chunks per lane");
    static_assert(16 * SST * 4 * NW <= A_BYTES + B_BYTES, "strips fit in one stage");
    __builtin_amdgcn_s_waitcnt(0);   // no copy is in flight (the idle copy of IDLE_COPY)
    __syncthreads();   // every wave is done with the last K block: stage 0 is free
    float *strip = reinterpret_cast<float *>(lds0) + wave * 16 * SST;
    const int wrow = wm * IT * 16, wcol = wn * JT * 16;
    void *const gC = p.C;
    const int64_t ldc = p.ldc, pM = p.M, pN = p.N;
    const bool accumulate = p.accumulate != 0;
#pragma unroll
    for (int i = 0; i < IT; i++) {
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
        for (int j = 0; j < JT; j++)
#pragma unroll
            for (int r = 0; r < 4; r++)
                strip[(4 * (lane >> 4) + r) * SST + j * 16 + (lane & 15)] = acc[i][j][r];
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
        for (int t = 0; t < NCH / 64; t++) {
            const int c = t * 64 + lane;
            const int row = c / (CW / CH), col = (c % (CW / CH)) * CH;
            const float *src = strip + row * SST + col;
            const float4 v0 = *reinterpret_cast<const float4 *>(src);
            const int64_t m = m0 + wrow + i * 16 + row, n = n0 + wcol + col;
            if (OUT_PARTIAL) {
                *reinterpret_cast<float4 *>(ws + ((int64_t)split * pM + m) * pN + n) = v0;
            } else if (CBF16) {
                float4 a = v0, b = *reinterpret_cast<const float4 *>(src + 4);
                uint4 *dst = reinterpret_cast<uint4 *>(reinterpret_cast<uint16_t *>(gC) + m * ldc + n);
                if (accumulate) {   // C + sum, rounded once
                    const uint4 c = *dst;
                    a.x += bf16_lo(c.x); a.y += bf16_hi(c.x); a.z += bf16_lo(c.y); a.w += bf16_hi(c.y);
                    b.x += bf16_lo(c.z); b.y += bf16_hi(c.z); b.z += bf16_lo(c.w); b.w += bf16_hi(c.w);
                }
                uint4 o;
                o.x = to_bf16x2(a.x, a.y);
                o.y = to_bf16x2(a.z, a.w);
                o.z = to_bf16x2(b.x, b.y);
                o.w = to_bf16x2(b.z, b.w);
                store_out_nt(dst, o);
            } else {
                float4 *dst = reinterpret_cast<float4 *>(reinterpret_cast<float *>(gC) + m * ldc + n);
                float4 o = v0;
                if (accumulate) {
                    const float4 c = *dst;
                    o.x += c.x; o.y += c.y; o.z += c.z; o.w += c.w;
                }
                store_out_nt(dst, o);
            }
        }
    }
}

// Split-K: workgroup b handles K blocks [kb_lo, kb_hi) of split s = b / tiles.
// Kernel arguments are read through the kernel-argument segment pointer (a
// constant-address-space pointer), so that indexing into them never makes the
// compiler copy the whole argument block into per-lane scratch memory.
typedef __attribute__((address_space(4))) const GemmArgs *KernargGemm;

__device__ __forceinline__ GemmArgs load_args(KernargGemm src)
{
    GemmArgs a;
#pragma unroll
    for (int i = 0; i < kMaxKSeg; i++) {
        a.seg[i].A = src->seg[i].A;
        a.seg[i].B = src->seg[i].B;
        a.seg[i].sA = src->seg[i].sA;
        a.seg[i].sB = src->seg[i].sB;
        a.seg[i].K = src->seg[i].K;
        a.seg[i].lda = src->seg[i].lda;
        a.seg[i].ldb = src->seg[i].ldb;
        a.seg[i].KB = src->seg[i].KB;
    }
    a.nseg = src->nseg;
    a.accumulate = src->accumulate;
    a.C = src->C;
    a.M = src->M;
    a.N = src->N;
    a.ldc = src->ldc;
    a.NB = src->NB;
    return a;
}

template <class Cfg, int LAYOUT, int BGRAN, bool CBF16, bool OUT_PARTIAL, int DP = DP_F16>
__global__ __launch_bounds__(Cfg::THREADS, 2) void gemm_fast_kernel(GemmArgs args, int tiles_m, int tiles_n,
                                                                 int splits, float *ws)
{
    (void)args;   // same bytes as *kargs
    const GemmArgs p = load_args((KernargGemm)__builtin_amdgcn_kernarg_segment_ptr());
    const int tiles = tiles_m * tiles_n;
    const int b = xcd_contiguous(blockIdx.x, tiles * splits);
    const int split = b / tiles;
    int tm, tn;
    tile_coords(b - split * tiles, tiles_m, tiles_n, tm, tn);
    // split K only for single-segment products
    const int64_t KB = p.seg[0].KB;
    const int64_t kb_lo = KB * split / splits, kb_hi = KB * (split + 1) / splits;
    fast_tile<Cfg, LAYOUT, BGRAN, CBF16, OUT_PARTIAL, false, DP>(p, (int64_t)tm * Cfg::TM, (int64_t)tn * Cfg::TN,
                                                             kb_lo, kb_hi, split, ws);
}

// Several independent problems in one launch: problem i owns tiles
// [first[i], first[i+1]) of the launch, walked as in gemm_fast_kernel.
// Workgroups reach the 8 XCDs round-robin.  With xcd_whole each XCD takes a
// contiguous eighth of the launch's tiles: one or two whole problems, or a
// contiguous part of one, so that the tiles resident together on an XCD share
// operand panels in its L2 (the host asks for it when every problem has the
// same number of K blocks, which keeps the eighths equal in work).  Otherwise
// each XCD takes a contiguous eighth of every problem's tiles.
constexpr int kGroupMax = 8;
struct GroupArgs {
    GemmArgs p[kGroupMax];
    int first[kGroupMax + 1];
    int count;
    int xcd_whole;
};

template <class Cfg, int LAYOUT, int BGRAN, bool CBF16, bool MULTI, int DP = DP_F16>
__global__ __launch_bounds__(Cfg::THREADS, 2) void gemm_group_kernel(GroupArgs args)
{
    (void)args;   // read through the argument segment pointer below
    typedef __attribute__((address_space(4))) const GroupArgs *KernargGroup;
    const KernargGroup gp = (KernargGroup)__builtin_amdgcn_kernarg_segment_ptr();
    const bool whole = gp->xcd_whole != 0;
    const int b = whole ? xcd_contiguous(blockIdx.x, gp->first[gp->count]) : blockIdx.x;
    int i = 0;
    while (i + 1 < gp->count && b >= gp->first[i + 1])
        i++;
    // i is the same in every lane: say so, so that the problem's fields are
    // read with scalar loads and kept in scalar registers
    i = __builtin_amdgcn_readfirstlane(i);
    const GemmArgs p = load_args(&gp->p[i]);
    const int first = gp->first[i];
    const int tiles_m = (int)(p.M / Cfg::TM), tiles_n = (int)(p.N / Cfg::TN);
    const int t = whole ? b - first : xcd_contiguous(b - first, tiles_m * tiles_n);
    int tm, tn;
    tile_coords(t, tiles_m, tiles_n, tm, tn);
    int64_t blocks = 0;
#pragma unroll
    for (int s = 0; s < kMaxKSeg; s++)
        if (s < p.nseg)
            blocks += p.seg[s].KB;
    fast_tile<Cfg, LAYOUT, BGRAN, CBF16, false, MULTI, DP>(p, (int64_t)tm * Cfg::TM, (int64_t)tn * Cfg::TN, 0, blocks,
                                                           0, nullptr);
}

// C[m][n] = sum over s = 0 .. splits-1, in that order, of ws[s][m][n]; four
// consecutive columns per thread (N % 4 == 0 on this path).
template <bool CBF16>
__global__ __launch_bounds__(256) void gemm_split_reduce(const float *__restrict__ ws, int splits, int64_t M,
                                                         int64_t N, void *__restrict__ C, int64_t ldc)
{
    const int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t n4 = N / 4;
    if (q >= M * n4)
        return;
    const int64_t m = q / n4, n = (q - m * n4) * 4;
    float4 sum = *reinterpret_cast<const float4 *>(ws + m * N + n);
    for (int s = 1; s < splits; s++) {
        const float4 v = *reinterpret_cast<const float4 *>(ws + ((int64_t)s * M + m) * N + n);
        sum.x += v.x;
        sum.y += v.y;
        sum.z += v.z;
        sum.w += v.w;
    }
    if (CBF16) {
        const uint32_t lo = to_bf16x2(sum.x, sum.y);
        const uint32_t hi = to_bf16x2(sum.z, sum.w);
        store_out_nt(reinterpret_cast<uint2 *>(reinterpret_cast<uint16_t *>(C) + m * ldc + n), make_uint2(lo, hi));
    } else {
        store_out_nt(reinterpret_cast<float4 *>(reinterpret_cast<float *>(C) + m * ldc + n), sum);
    }
}

// Launch plan for an aligned problem: tile configuration and number of K splits.
struct FastPlan {
    bool ok;       // aligned fast path applies
    int cfg;       // CFG_L or CFG_Q
    int splits;    // K splits (1 = none)
};

constexpr int kComputeUnits = 256;

// Per-tile cost of a tile configuration on one datapath, measured on gfx950
// with every CU busy (us): a tile takes `fixed + blocks * step`; 128 x 128
// tiles run two per CU (`step2`, `fixed2` each pair) and `step1`, `fixed1`
// when one is left alone.
struct TileCost {
    double step2, fixed2, step1, fixed1, launch;   // launch: once per launch
};

TileCost tile_cost(int cfg, int dp, bool bgran128)
{
    if (cfg == CFG_Q) {
        if (dp == DP_F16)
            return {1.96, 4.1, 1.4, 3.0, 0.0};
        if (dp == DP_MX)
            return {1.07, 5.6, 0.8, 4.0, 0.0};
        return {1.24, 2.2, 0.9, 2.0, 0.0};
    }
    if (dp == DP_F16)   // 1x128 B scales: one more product per promoted element
        return bgran128 ? TileCost{3.3, 8.0, 3.3, 8.0, 6.0} : TileCost{3.67, 8.0, 3.67, 8.0, 6.0};
    if (dp == DP_MX)
        return {2.13, 6.1, 2.13, 6.1, 0.0};
    return {2.24, 6.1, 2.24, 6.1, 0.0};
}

// Picks the candidate with the least estimated time.  Workgroups are spread
// evenly over the CUs, so the busiest CU sets the time.  Splitting K adds the
// partial sums, (splits + 1) M N 4 bytes moved at about 4 TB/s, and the
// reduction launch.  On the FP32-exact datapath the 256 x 256 tile is
// considered for NT products only (its K-major fragments).
FastPlan fast_plan(int64_t M, int64_t N, int64_t K, int dp, bool nt, bool bgran128)
{
    FastPlan best = {false, CFG_Q, 1};
    if (K <= 0 || K % 128 || M % CfgQ::TM || N % CfgQ::TN)
        return best;
    const int64_t KB = K / 128;
    double best_us = 1e300;
    for (int cfg : {(int)CFG_L, (int)CFG_Q}) {
        if (cfg == CFG_L && dp == DP_F16 && !nt)
            continue;
        const int T = cfg == CFG_Q ? CfgQ::TM : CfgL::TM;
        if (M % T || N % T)
            continue;
        const TileCost c = tile_cost(cfg, dp, bgran128);
        const int64_t tiles = (M / T) * (N / T);
        for (int sp = 1; sp <= 8; sp *= 2) {
            if (sp > 1 && KB / sp < 4)
                break;
            const double steps = (double)((KB + sp - 1) / sp);
            const int64_t per_cu = (tiles * sp + kComputeUnits - 1) / kComputeUnits;
            double us = cfg == CFG_Q ? (double)(per_cu / 2) * (steps * c.step2 + c.fixed2) +
                                           (double)(per_cu % 2) * (steps * c.step1 + c.fixed1)
                                     : (double)per_cu * (steps * c.step1 + c.fixed1) + c.launch;
            if (sp > 1)
                us += (double)(sp + 1) * (double)M * (double)N * 4.0 / 4e6 + 5.0;
            if (us < best_us) {
                best_us = us;
                best = {true, cfg, sp};
            }
        }
    }
    return best;
}

template <class Cfg, int LAYOUT, int BGRAN, bool CBF16, int DP>
hipError_t launch_fast_cfg(const GemmArgs &a, int splits, float *ws, hipStream_t st)
{
    const int tiles_m = (int)(a.M / Cfg::TM), tiles_n = (int)(a.N / Cfg::TN);
    const dim3 grid((unsigned)(tiles_m * tiles_n * splits));
    if (splits == 1) {
        hipLaunchKernelGGL((gemm_fast_kernel<Cfg, LAYOUT, BGRAN, CBF16, false, DP>), grid, dim3(Cfg::THREADS), 0,
                           st, a, tiles_m, tiles_n, 1, (float *)nullptr);
        return hipGetLastError();
    }
    hipLaunchKernelGGL((gemm_fast_kernel<Cfg, LAYOUT, BGRAN, CBF16, true, DP>), grid, dim3(Cfg::THREADS), 0, st,
                       a, tiles_m, tiles_n, splits, ws);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    const int64_t quads = a.M * (a.N / 4);
    hipLaunchKernelGGL((gemm_split_reduce<CBF16>), dim3((unsigned)((quads + 255) / 256)), dim3(256), 0, st, ws,
                       splits, a.M, a.N, a.C, a.ldc);
    return hipGetLastError();
}

// The tile kernels' copies take a 32-bit per-lane offset of up to 7 leading
// dimensions: every segment's leading dimensions must be below 2^28.
constexpr int64_t kFastLdLimit = (int64_t)1 << 28;
bool fast_ld_ok(const GemmArgs &a)
{
    bool ok = true;
    for (int i = 0; i < a.nseg; i++)
        ok = ok && a.seg[i].lda < kFastLdLimit && a.seg[i].ldb < kFastLdLimit;
    return ok;
}

template <int LAYOUT, int BGRAN, bool CBF16, int DP>
hipError_t launch_planned(const GemmArgs &a, const FastPlan &plan, float *ws, hipStream_t st)
{
    if (plan.cfg == CFG_L) {
        // the FP32-exact datapath plans 256 x 256 tiles for NT only
        if constexpr (DP != DP_F16 || LAYOUT == 0)
            return launch_fast_cfg<CfgL, LAYOUT, BGRAN, CBF16, DP>(a, plan.splits, ws, st);
        return hipErrorInvalidValue;
    }
    return launch_fast_cfg<CfgQ, LAYOUT, BGRAN, CBF16, DP>(a, plan.splits, ws, st);
}

// FP32-exact datapath: aligned shapes take the tile kernels, any other the
// bounds-checked general kernel.
template <int LAYOUT, int BGRAN, bool CBF16>
hipError_t launch_one(const GemmArgs &a, float *ws, hipStream_t st)
{
    const FastPlan plan = fast_plan(a.M, a.N, a.seg[0].K, DP_F16, LAYOUT == 0, BGRAN == 1);
    if (plan.ok && fast_ld_ok(a))
        return launch_planned<LAYOUT, BGRAN, CBF16, DP_F16>(a, plan, ws, st);
    const dim3 grid((unsigned)((a.N + BN - 1) / BN), (unsigned)((a.M + BM - 1) / BM));
    hipLaunchKernelGGL((gemm_kernel<LAYOUT, BGRAN, CBF16>), grid, dim3(256), 0, st, a);
    return hipGetLastError();
}

// Scaled (MX) and native FP8 datapaths: aligned shapes only (the API layer
// admits no others).
template <int LAYOUT, int BGRAN, bool CBF16, int DP>
hipError_t launch_aligned_t(const GemmArgs &a, float *ws, hipStream_t st)
{
    const FastPlan plan = fast_plan(a.M, a.N, a.seg[0].K, DP, LAYOUT == 0, BGRAN == 1);
    if (!plan.ok || !fast_ld_ok(a))
        return hipErrorInvalidValue;
    return launch_planned<LAYOUT, BGRAN, CBF16, DP>(a, plan, ws, st);
}

template <int LAYOUT, int DP>
hipError_t launch_aligned_layout(const GemmProblem &p, const GemmArgs &a, float *ws, hipStream_t st)
{
    if (p.bgran)
        return p.c_bf16 ? launch_aligned_t<LAYOUT, 1, true, DP>(a, ws, st) : launch_aligned_t<LAYOUT, 1, false, DP>(a, ws, st);
    return p.c_bf16 ? launch_aligned_t<LAYOUT, 0, true, DP>(a, ws, st) : launch_aligned_t<LAYOUT, 0, false, DP>(a, ws, st);
}

template <int LAYOUT>
hipError_t launch_layout(const GemmProblem &p, const GemmArgs &a, float *ws, hipStream_t st)
{
    if (p.bgran)
        return p.c_bf16 ? launch_one<LAYOUT, 1, true>(a, ws, st) : launch_one<LAYOUT, 1, false>(a, ws, st);
    return p.c_bf16 ? launch_one<LAYOUT, 0, true>(a, ws, st) : launch_one<LAYOUT, 0, false>(a, ws, st);
}

GemmArgs make_args(const GemmProblem &p)
{
    GemmArgs a;
    a.nseg = p.nseg;
    for (int i = 0; i < kMaxKSeg; i++) {
        KSeg &g = a.seg[i];
        if (i < p.nseg) {
            const GemmSegment &q = p.seg[i];
            g.A = q.A;
            g.B = q.B;
            g.sA = q.sA;
            g.sB = q.sB;
            g.K = q.K;
            g.lda = q.lda;
            g.ldb = q.ldb;
            g.KB = (q.K + 127) / 128;
        } else {
            g = KSeg{nullptr, nullptr, nullptr, nullptr, 0, 0, 0, 0};
        }
    }
    a.accumulate = p.accumulate ? 1 : 0;
    a.C = p.C;
    a.M = p.M;
    a.N = p.N;
    a.ldc = p.ldc;
    a.NB = (p.N + 127) / 128;
    return a;
}

// One or more grouped launches of problems sharing a tile size: T = 128 or
// 256 (fast_tile's two configurations).
template <int T, int LAYOUT, int BGRAN, bool CBF16, int DP>
hipError_t launch_group_tiles(const std::vector<GemmArgs> &ps, hipStream_t st)
{
    for (size_t lo = 0; lo < ps.size(); lo += kGroupMax) {
        GroupArgs g;
        g.count = (int)std::min(ps.size() - lo, (size_t)kGroupMax);
        g.first[0] = 0;
        bool same_k = true;
        for (int i = 0; i < g.count; i++) {
            g.p[i] = ps[lo + i];
            g.first[i + 1] = g.first[i] + (int)((g.p[i].M / T) * (g.p[i].N / T));
            int64_t kb = 0, kb0 = 0;
            for (int j = 0; j < g.p[i].nseg; j++)
                kb += g.p[i].seg[j].KB;
            for (int j = 0; j < g.p[0].nseg; j++)
                kb0 += g.p[0].seg[j].KB;
            same_k = same_k && kb == kb0;
        }
#ifndef PURO_XCD_WHOLE
#define PURO_XCD_WHOLE 1
#endif
        g.xcd_whole = PURO_XCD_WHOLE && g.count > 1 && same_k && g.first[g.count] % 8 == 0;
        // launches whose problems all have one K segment take the kernel
        // without the segment lookup
        bool multi = false;
        for (int i = 0; i < g.count; i++)
            multi = multi || g.p[i].nseg > 1;
        const dim3 grid((unsigned)g.first[g.count]);
        if constexpr (T == 256) {
            // single-segment problems only (the caller's choice): the 256 x 256
            // tile has no registers to spare for the segment lookup
            if (multi)
                return hipErrorInvalidValue;
            hipLaunchKernelGGL((gemm_group_kernel<CfgL, LAYOUT, BGRAN, CBF16, false, DP>), grid, dim3(CfgL::THREADS),
                               0, st, g);
        } else {
            if (multi)
                hipLaunchKernelGGL((gemm_group_kernel<CfgQ, LAYOUT, BGRAN, CBF16, true, DP>), grid,
                                   dim3(CfgQ::THREADS), 0, st, g);
            else
                hipLaunchKernelGGL((gemm_group_kernel<CfgQ, LAYOUT, BGRAN, CBF16, false, DP>), grid,
                                   dim3(CfgQ::THREADS), 0, st, g);
        }
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess)
            return e;
    }
    return hipSuccess;
}

// Estimated time of a group's problems on one tile configuration of a
// datapath (the per-tile costs of fast_plan, work spread evenly over the CUs).
double group_estimate(const std::vector<GemmArgs> &ps, int cfg, int dp, bool bgran128)
{
    const TileCost c = tile_cost(cfg, dp, bgran128);
    const int T = cfg == CFG_Q ? CfgQ::TM : CfgL::TM;
    double work = 0.0;
    for (const GemmArgs &x : ps) {
        int64_t blocks = 0;
        for (int j = 0; j < x.nseg; j++)
            blocks += x.seg[j].KB;
        const double tiles = (double)((x.M / T) * (x.N / T));
        work += cfg == CFG_Q ? tiles * ((double)blocks * c.step2 + c.fixed2) / 2.0
                             : tiles * ((double)blocks * c.step1 + c.fixed1);
    }
    return work / kComputeUnits + c.launch;
}

template <int LAYOUT, int BGRAN, bool CBF16, int DP>
hipError_t launch_group_t(const GemmProblem *probs, int count, hipStream_t st)
{
    // Problems whose extents are multiples of 128 share grouped launches
    // (longest K first, so that the longest tiles start first); on the
    // FP32-exact datapath any other non-empty problem runs on its own through
    // the bounds-checked kernel (the other datapaths admit aligned problems
    // only: the API layer checks).
    std::vector<GemmArgs> fast;
    for (int i = 0; i < count; i++) {
        const GemmProblem &p = probs[i];
        if (p.M == 0 || p.N == 0)
            continue;
        bool k_aligned = true;
        for (int j = 0; j < p.nseg; j++)
            k_aligned = k_aligned && p.seg[j].K % 128 == 0;
        if (k_aligned && p.M % CfgQ::TM == 0 && p.N % CfgQ::TN == 0 && fast_ld_ok(make_args(p))) {
            fast.push_back(make_args(p));
        } else if (DP != DP_F16) {
            return hipErrorInvalidValue;
        } else {
            const GemmArgs a = make_args(p);
            const dim3 grid((unsigned)((a.N + BN - 1) / BN), (unsigned)((a.M + BM - 1) / BM));
            hipLaunchKernelGGL((gemm_kernel<LAYOUT, BGRAN, CBF16>), grid, dim3(256), 0, st, a);
            const hipError_t e = hipGetLastError();
            if (e != hipSuccess)
                return e;
        }
    }
    if (fast.empty())
        return hipSuccess;
    auto blocks = [](const GemmArgs &x) {
        int64_t kb = 0;
        for (int j = 0; j < x.nseg; j++)
            kb += x.seg[j].KB;
        return kb;
    };
    std::stable_sort(fast.begin(), fast.end(),
                     [&](const GemmArgs &x, const GemmArgs &y) { return blocks(x) > blocks(y); });
    std::vector<GemmArgs> large, small;
    // 256 x 256 tiles: single-segment problems whose extents are multiples of
    // 256 (on the FP32-exact datapath NT products only, its K-major fragments)
    constexpr bool L_OK = DP != DP_F16 || LAYOUT == 0;
    for (const GemmArgs &x : fast) {
        if (L_OK && x.nseg == 1 && x.M % CfgL::TM == 0 && x.N % CfgL::TN == 0) {
            large.push_back(x);
        } else {
            small.push_back(x);
        }
    }
    // the 256 x 256 tiles take the eligible problems when the estimate favours them
    if (large.empty() ||
        group_estimate(large, CFG_L, DP, BGRAN == 1) >= group_estimate(large, CFG_Q, DP, BGRAN == 1)) {
        small = fast;
        large.clear();
    }
    if constexpr (L_OK) {
        if (!large.empty()) {
            const hipError_t e = launch_group_tiles<256, LAYOUT, BGRAN, CBF16, DP>(large, st);
            if (e != hipSuccess)
                return e;
        }
    }
    if (small.empty())
        return hipSuccess;
    return launch_group_tiles<128, LAYOUT, BGRAN, CBF16, DP>(small, st);
}

template <int LAYOUT, int DP>
hipError_t launch_group_layout(const GemmProblem *probs, int count, hipStream_t st)
{
    const GemmProblem &p = probs[0];
    if (p.bgran)
        return p.c_bf16 ? launch_group_t<LAYOUT, 1, true, DP>(probs, count, st)
                        : launch_group_t<LAYOUT, 1, false, DP>(probs, count, st);
    return p.c_bf16 ? launch_group_t<LAYOUT, 0, true, DP>(probs, count, st)
                    : launch_group_t<LAYOUT, 0, false, DP>(probs, count, st);
}

template <int DP>
hipError_t launch_group_dp(const GemmProblem *probs, int count, hipStream_t st)
{
    if (count <= 0)
        return hipSuccess;
    switch (probs[0].layout) {
    case 0: return launch_group_layout<0, DP>(probs, count, st);
    case 1: return launch_group_layout<1, DP>(probs, count, st);
    default: return launch_group_layout<2, DP>(probs, count, st);
    }
}

size_t plan_workspace(const GemmProblem &p, int dp)
{
    const FastPlan plan = fast_plan(p.M, p.N, p.seg[0].K, dp, p.layout == 0, p.bgran == 1);
    if (!plan.ok || plan.splits == 1)
        return 0;
    return (size_t)plan.splits * (size_t)p.M * (size_t)p.N * sizeof(float);
}

template <int DP>
hipError_t launch_aligned(const GemmProblem &p, void *workspace, hipStream_t st)
{
    if (p.M == 0 || p.N == 0)
        return hipSuccess;
    const GemmArgs a = make_args(p);
    float *ws = reinterpret_cast<float *>(workspace);
    switch (p.layout) {
    case 0: return launch_aligned_layout<0, DP>(p, a, ws, st);
    case 1: return launch_aligned_layout<1, DP>(p, a, ws, st);
    default: return launch_aligned_layout<2, DP>(p, a, ws, st);
    }
}

} // namespace

size_t gemm_workspace_bytes(const GemmProblem &p)
{
    return plan_workspace(p, DP_F16);
}

hipError_t launch_gemm(const GemmProblem &p, void *workspace, hipStream_t st)
{
    if (p.M == 0 || p.N == 0)
        return hipSuccess;
    const GemmArgs a = make_args(p);
    float *ws = reinterpret_cast<float *>(workspace);
    switch (p.layout) {
    case 0: return launch_layout<0>(p, a, ws, st);
    case 1: return launch_layout<1>(p, a, ws, st);
    default: return launch_layout<2>(p, a, ws, st);
    }
}

size_t gemm_mx_workspace_bytes(const GemmProblem &p)
{
    return plan_workspace(p, DP_MX);
}

hipError_t launch_gemm_mx(const GemmProblem &p, void *workspace, hipStream_t st)
{
    return launch_aligned<DP_MX>(p, workspace, st);
}

size_t gemm_native_workspace_bytes(const GemmProblem &p)
{
    return plan_workspace(p, DP_FP8);
}

hipError_t launch_gemm_native(const GemmProblem &p, void *workspace, hipStream_t st)
{
    return launch_aligned<DP_FP8>(p, workspace, st);
}

hipError_t launch_gemm_group(const GemmProblem *probs, int count, hipStream_t st)
{
    return launch_group_dp<DP_F16>(probs, count, st);
}

hipError_t launch_gemm_group_mx(const GemmProblem *probs, int count, hipStream_t st)
{
    return launch_group_dp<DP_MX>(probs, count, st);
}

hipError_t launch_gemm_group_native(const GemmProblem *probs, int count, hipStream_t st)
{
    return launch_group_dp<DP_FP8>(probs, count, st);
}

} // namespace puro
