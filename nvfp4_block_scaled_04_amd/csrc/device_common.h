// device_common.h -- small gfx950 device helpers shared by the quantize and
// GEMM kernels: bf16 packing, the ue4m3 / e2m1 conversions through the
// hardware convert instructions, and the 128x4 swizzled scale offset.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nvfp4 {

typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

constexpr float kFp32Max = 3.40282346638528859812e+38f;

__device__ __forceinline__ float bits_f(uint32_t u) { return __builtin_bit_cast(float, u); }
__device__ __forceinline__ uint32_t f_bits(float f) { return __builtin_bit_cast(uint32_t, f); }

// Low / high bf16 of a packed pair, widened to fp32 (exact).
__device__ __forceinline__ float bf16_lo(uint32_t w) { return bits_f(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return bits_f(w & 0xFFFF0000u); }

// fp32 -> bf16, round to nearest even; NaN stays NaN.
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
    uint32_t u = f_bits(f);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return 0x7FC0u;
    u += 0x7FFFu + ((u >> 16) & 1u);
    return u >> 16;
}

// Two fp32 values to a packed bf16 pair (a low, b high) with one hardware
// conversion, round to nearest even (NaN stays NaN).
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    typedef float f32x2_t __attribute__((ext_vector_type(2)));
    typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{a, b}, bf16x2_t));
}

// Largest |x| over 8 packed bf16 values, as the bf16 bit pattern of |x|
// (for non-negative values integer order is value order; NaN and inf patterns
// compare above every finite one).
__device__ __forceinline__ uint32_t absmax_bits_bf16x8(const uint32_t w[4]) {
    u16x2 a0 = __builtin_bit_cast(u16x2, w[0] & 0x7FFF7FFFu);
    u16x2 a1 = __builtin_bit_cast(u16x2, w[1] & 0x7FFF7FFFu);
    u16x2 a2 = __builtin_bit_cast(u16x2, w[2] & 0x7FFF7FFFu);
    u16x2 a3 = __builtin_bit_cast(u16x2, w[3] & 0x7FFF7FFFu);
    u16x2 m = __builtin_elementwise_max(__builtin_elementwise_max(a0, a1), __builtin_elementwise_max(a2, a3));
    return m[0] > m[1] ? m[0] : m[1];
}

// nan_to_num: NaN -> 0, +-inf -> +-FLT_MAX.
__device__ __forceinline__ float nan_to_num(float v) {
    if (v != v) return 0.0f;
    if (v == __builtin_inff()) return kFp32Max;
    if (v == -__builtin_inff()) return -kFp32Max;
    return v;
}

// Exchange with the neighbouring lane (lane ^ 1) through DPP quad_perm [1,0,3,2].
__device__ __forceinline__ float xor1(float v) {
    return bits_f((uint32_t)__builtin_amdgcn_mov_dpp((int)f_bits(v), 0xB1, 0xF, 0xF, true));
}

// fp32(x / 6) for x >= 0, correctly rounded, without the division sequence:
// q0 = x * RN(1/6), then one correction step with the exact FMA residual
// r = x - q0 * 6 (Markstein's correction for division by a constant).
// Compared with the IEEE quotient over every non-negative finite fp32: equal
// for all x >= 2^-120; below that, where the quotient is subnormal, the
// division itself is used.
__device__ __forceinline__ float div6(float x) {
    const float c = 0.16666667163372039794921875f;  // RN(1/6)
    const float q0 = x * c;
    const float q1 = __builtin_fmaf(__builtin_fmaf(-q0, 6.0f, x), c, q0);
    if (__builtin_expect(x < 0x1p-120f, 0)) return x / 6.0f;
    return q1;
}

// ue4m3 code of a non-negative fp32 value: round to nearest even, saturating
// at 448.  The hardware e4m3 conversion rounds to nearest even but overflows
// to NaN above 464, so the value is clamped to 448 first.
__device__ __forceinline__ uint32_t ue4m3_encode(float v) {
    v = __builtin_fminf(v, 448.0f);
    return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(v, 0.0f, 0, false) & 0xFFu;
}

__device__ __forceinline__ float ue4m3_decode(uint32_t code) {
    return __builtin_amdgcn_cvt_f32_fp8((int)code, 0);
}

// Two fp32 values to two e2m1 codes (a -> low nibble, b -> high nibble)
// written into byte `sel` of `old`: round to nearest even, saturating at 6,
// sign kept.  A scale of 1.0 leaves the values unscaled.
#define NVFP4_PACK_FP4(old, a, b, sel) \
    __builtin_amdgcn_cvt_scalef32_pk_fp4_f32((old), (a), (b), 1.0f, (sel))

// Byte offset of scale (r, c) in the 128x4 swizzled layout with cp4 =
// pad_up(k/16,4)/4 column groups.
__device__ __forceinline__ int64_t sf_offset(int64_t r, int64_t c, int64_t cp4) {
    return ((r >> 7) * cp4 + (c >> 2)) * 512 + (r & 31) * 16 + ((r & 127) >> 5) * 4 + (c & 3);
}

__device__ __forceinline__ int clamp_rows(const int32_t* mask, int e, int m) {
    if (!mask) return m;
    int v = mask[e];
    return v < 0 ? 0 : (v > m ? m : v);
}

}  // namespace nvfp4
