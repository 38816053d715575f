// Device helpers shared by the quantiser and GEMM kernels (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace puro {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v2i __attribute__((ext_vector_type(2)));
typedef float v4f __attribute__((ext_vector_type(4)));

// Four floats -> four E4M3 codes packed little-endian into one dword.
// v_cvt_pk_fp8_f32 rounds to nearest even into the OCP E4M3 format; it was
// checked on gfx950 against an integer-only round-to-nearest-even,
// saturating encoder for every FP32 value with |y| <= 449, which covers every
// quotient x/s the quantisers form (|x/s| <= 448 * (1 + 2^-23)).
__device__ __forceinline__ uint32_t e4m3x4(float a, float b, float c, float d)
{
    uint32_t lo = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
    return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(c, d, (int)lo, true);
}

// Code of +-0 by the sign of x: 0x80 for negative values and -0.
__device__ __forceinline__ uint32_t sign_code(float x)
{
    return (__float_as_uint(x) >> 24) & 0x80u;
}

// Correctly rounded x / s for one block's scale s.
//
// With r = RN(1/s), y0 = RN(x r) is within an ulp of x/s; the residual
// e = x - y0 s is then exact (one FMA), and RN(y0 + e r) = RN(x/s)
// (Markstein's correction step).  The residual is exact only while it does
// not underflow, which holds for s >= 2^-80 over every quotient that can
// change an E4M3 code (|x/s| >= 2^-12); below that the kernel divides.  The
// sign is copied from x so that -0 stays -0.  Checked against IEEE division
// on 7e9 quotients (s in [2^-90, 2^30]) before use.
struct Divider {
    float s, r;
    bool fast;
};

__device__ __forceinline__ Divider make_divider(float s)
{
    Divider d;
    d.s = s;
    d.fast = s >= 0x1p-80f;
    d.r = d.fast ? 1.0f / s : 0.0f;
    return d;
}

__device__ __forceinline__ float quotient(const Divider &d, float x)
{
    if (!d.fast)
        return x / d.s;
    const float y0 = x * d.r;
    const float e = fmaf(-y0, d.s, x);
    return __builtin_copysignf(fmaf(e, d.r, y0), x);
}

// Power-of-two block scale: the smallest s = 2^k with 448 s >= amax, k kept
// in [-127, 127] (the E8M0 range of the scaled matrix cores; a zero block gets
// 2^-127).  With amax = m 2^e (m in [0.5, 1)), 448 2^(e-9) = 0.875 2^e, so k
// is e - 9 or e - 8; 448 2^k = 1.75 2^(k+8) is built exactly from its bits.
__device__ __forceinline__ float pow2_scale(float amax)
{
    int e = -300;
    if (amax > 0.0f)
        frexpf(amax, &e);
    int k = e - 9 < -127 ? -127 : e - 9;
    if (k <= 119 && amax > __uint_as_float(((uint32_t)(k + 135) << 23) | 0x600000u))
        k++;
    return __uint_as_float(k >= -126 ? (uint32_t)(k + 127) << 23 : 0x00400000u);
}

// Dequantisation scale of a block with largest magnitude amax: amax / 448
// (IEEE binary32 division), or the power-of-two rule.
__device__ __forceinline__ float block_scale(float amax, int pow2)
{
    return pow2 ? pow2_scale(amax) : amax / 448.0f;
}

// Quantise four values of a block with dequant scale d.s (> 0, or == 0 for a
// zero block: codes +-0 by sign).
__device__ __forceinline__ uint32_t quant4(float a, float b, float c, float d_, const Divider &d)
{
    if (d.s == 0.0f)
        return sign_code(a) | (sign_code(b) << 8) | (sign_code(c) << 16) | (sign_code(d_) << 24);
    return e4m3x4(quotient(d, a), quotient(d, b), quotient(d, c), quotient(d, d_));
}

__device__ __forceinline__ float bf16_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t u) { return __uint_as_float(u & 0xFFFF0000u); }

// Round to nearest even FP32 -> BF16, two at a time: a in the low half, b in
// the high half.  v_cvt_pk_bf16_f32 was checked on gfx950 against an integer
// round-to-nearest-even for every non-NaN FP32 bit pattern (no mismatch).
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t to_bf16x2(float a, float b)
{
    const f32x2_t v = {a, b};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

// One value: the low half of to_bf16x2.
__device__ __forceinline__ uint16_t to_bf16(float f)
{
    return (uint16_t)(to_bf16x2(f, 0.0f) & 0xFFFFu);
}

// Element loads widened to FP32.
template <typename T> struct Elem;
template <> struct Elem<float> {
    __device__ __forceinline__ static float load(const float *p) { return *p; }
    // 8 consecutive values from a 16-byte aligned address
    __device__ __forceinline__ static void load8(const float *p, float v[8])
    {
        const float4 a = *reinterpret_cast<const float4 *>(p);
        const float4 b = *reinterpret_cast<const float4 *>(p + 4);
        v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
        v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
    }
};
template <> struct Elem<uint16_t> {
    __device__ __forceinline__ static float load(const uint16_t *p) { return __uint_as_float((uint32_t)*p << 16); }
    __device__ __forceinline__ static void load8(const uint16_t *p, float v[8])
    {
        const uint4 a = *reinterpret_cast<const uint4 *>(p);
        v[0] = bf16_lo(a.x); v[1] = bf16_hi(a.x); v[2] = bf16_lo(a.y); v[3] = bf16_hi(a.y);
        v[4] = bf16_lo(a.z); v[5] = bf16_hi(a.z); v[6] = bf16_lo(a.w); v[7] = bf16_hi(a.w);
    }
};

} // namespace puro
