// quant_block.h -- the per-block arithmetic of NVFP4 quantization shared by
// the quantize kernels and the GEMM epilogue that quantizes its own output:
// the silu_and_mul prologue, the block's values after the prologue with their
// largest magnitude, and the e2m1 packing of a block.
#pragma once

#include "device_common.h"

namespace nvfp4 {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

enum Variant { V_BF16 = 0, V_F32 = 1, V_BF16_SMOOTH = 2, V_F32_SMOOTH = 3, V_SILU = 4 };

// silu(g) = g / (1 + e^-g), evaluated in fp64 and rounded once to fp32.
__device__ __forceinline__ float silu_f32(float g) {
    double x = (double)g;
    return (float)(x / (1.0 + exp(-x)));
}

// h = bf16(fp32(S * u)) with S = silu(g) correctly rounded to fp32, for the
// two bf16 pairs packed in a gate word and an up word: the fast path and its
// exactness test.  Returns the two h as a packed bf16 pair; bit i of `bad`
// (i = 0 low, 1 high) is set where the result must come from the exact path.
//
// y = g * rcp(1 + 2^(-g * log2 e)) in fp32.  For |g| < 16 the product
// -g * log2(e) is off by at most |g| * 2^-23 * log2(e) in absolute terms
// (two roundings), which moves 2^t by at most |g| * 2^-23 relative; with
// the hardware exp2 and reciprocal (at most 2 ulp and 1 ulp) and the three
// fp32 roundings, y is within 21 * 2^-23 of S relative.  So fp32(S * u) and
// p = fp32(y * u) differ by at most 43 ulp of p (a relative bound is worth at
// most twice its size in ulp).  bf16 rounding changes its result only where
// the low 16 bits of the pattern cross 0x8000, which no interval of that
// width does when they sit more than 64 away from it (a binade change inside
// the interval puts them next to 0 or 0xFFFF), so then bf16(p) is the exact
// h.  The test also requires |g| >= 2^-77 (so |y| > 2^-101, far from the
// subnormals) and |p| in [2^-100, 2^100).  Elements that fail it (about 1 in
// 500 for N(0,1) data, and every |g| >= 16, inf and NaN) take the exact fp64
// path.
//
// The two failure kinds are reported apart: `rng` (an operand or the product
// outside the ranges above, inf, NaN: nothing is known of h) and `win` (in
// range, but the low half of p within 64 of 0x8000: h is bf16(p) or its
// neighbour on the other side of p, i.e. |h| is at most the magnitude bits
// of bf16(p) plus one).
// p = fp32(y * u) of the fast path for one element (the same operations,
// so the same bits, as silu_mul_fast2s).
__device__ __forceinline__ float silu_fast_p(float g, float u) {
    constexpr float kLog2e = 1.44269504088896340736f;
    const float y = g * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(g * -kLog2e));
    return y * u;
}

__device__ __forceinline__ uint32_t silu_mul_fast2s(uint32_t gw, uint32_t uw, uint32_t& rng, uint32_t& win) {
    const float p0 = silu_fast_p(bf16_lo(gw), bf16_lo(uw)), p1 = silu_fast_p(bf16_hi(gw), bf16_hi(uw));
    const float g0 = bf16_lo(gw), g1 = bf16_hi(gw);
    // (bitwise, not short-circuit, so the test stays branch-free)
    auto out_of_range = [](float g, float p) -> uint32_t {
        const uint32_t ga = f_bits(g) & 0x7FFFFFFFu, pa = f_bits(p) & 0x7FFFFFFFu;
        return (uint32_t)(ga - 0x19000000u >= 0x41800000u - 0x19000000u) |  // not 2^-77 <= |g| < 16
               (uint32_t)(pa - 0x0D800000u >= 0x64000000u);                  // not 2^-100 <= |p| < 2^100
    };
    auto near_tie = [](float p) -> uint32_t {
        return (uint32_t)((f_bits(p) & 0xFFFFu) - 0x7FC0u <= 0x80u);  // low half within 64 of 0x8000
    };
    rng = out_of_range(g0, p0) | (out_of_range(g1, p1) << 1);
    win = near_tie(p0) | (near_tie(p1) << 1);
    typedef float f32x2 __attribute__((ext_vector_type(2)));
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{p0, p1}, bf16x2));  // RNE
}

__device__ __forceinline__ uint32_t silu_mul_fast2(uint32_t gw, uint32_t uw, uint32_t& bad) {
    uint32_t rng, win;
    const uint32_t h = silu_mul_fast2s(gw, uw, rng, win);
    bad = rng | win;
    return h;
}

__device__ __forceinline__ uint32_t silu_mul_exact(float g, float u) {
    return f32_to_bf16_rne(silu_f32(g) * u);
}

// Element `bit` (2j + half) of a silu block's gate / up words r[0..3] through
// the exact path, written into its bf16 half of w[j]: a single inlined copy
// of the exact path for every flagged element of the block, one at a time.
__device__ __forceinline__ void silu_exact_into(const u32x4 (&r)[4], int bit, uint32_t (&w)[8]) {
    const int j = bit >> 1, sh = (bit & 1) * 16;
    uint32_t gw = 0, uw = 0;
#pragma unroll
    for (int jj = 0; jj < 8; jj++) {
        if (jj == j) {
            gw = jj < 4 ? r[0][jj] : r[1][jj - 4];
            uw = jj < 4 ? r[2][jj] : r[3][jj - 4];
        }
    }
    const uint32_t h = silu_mul_exact(bits_f((gw >> sh) << 16), bits_f((uw >> sh) << 16));
#pragma unroll
    for (int jj = 0; jj < 8; jj++)
        if (jj == j) w[jj] = (w[jj] & ~(0xFFFFu << sh)) | (h << sh);
}

// h = silu(g) * u (bf16) of a block's 16 elements, as 8 words of bf16 pairs:
// the fast path for all of them, then the exact path for the flagged ones
// (rare: one divergent branch per block).
__device__ __forceinline__ void silu_block_words(const u32x4 (&r)[4], uint32_t (&w)[8]) {
    uint32_t need = 0;
#pragma unroll
    for (int j = 0; j < 8; j++) {
        const uint32_t gw = j < 4 ? r[0][j] : r[1][j - 4];
        const uint32_t uw = j < 4 ? r[2][j] : r[3][j - 4];
        uint32_t bad;
        w[j] = silu_mul_fast2(gw, uw, bad);
        need |= bad << (2 * j);
    }
    // The flagged elements one at a time through a single inlined copy of
    // the exact path (a call would make the wave wait for every load it has
    // in flight).
    while (need) {
        const int bit = __builtin_ctz(need);
        need &= need - 1;
        silu_exact_into(r, bit, w);
    }
}

// Largest |nan_to_num(v)| over the 16 bf16 values of 8 words.
__device__ __forceinline__ float bf16_words_amax(const uint32_t (&w)[8]) {
    const uint32_t mb = __builtin_elementwise_max(absmax_bits_bf16x8(w), absmax_bits_bf16x8(w + 4));
    if (mb < 0x7F80u) return bits_f(mb << 16);
    float a = 0.0f;  // inf or NaN present
#pragma unroll
    for (int j = 0; j < 16; j++) {
        const float v = nan_to_num((j & 1) ? bf16_hi(w[j >> 1]) : bf16_lo(w[j >> 1]));
        a = __builtin_fmaxf(a, __builtin_fabsf(v));
    }
    return a;
}

// 16-byte loads behind one 16-element block of a row.
template <int V>
constexpr int loads_per_block() {
    return V == V_BF16 || V == V_BF16_SMOOTH ? 2 : 4;  // fp32: 64 bytes; silu: gate 32 + up 32
}

// The block's 16 values after the prologue and nan_to_num, and their largest
// magnitude.
template <int V>
__device__ __forceinline__ float process_block(const u32x4 (&r)[loads_per_block<V>()], const u32x4 (&pq)[2],
                                               float (&f)[16]) {
    if constexpr (V == V_BF16 || V == V_SILU) {
        uint32_t w[8];
        if constexpr (V == V_BF16) {
#pragma unroll
            for (int j = 0; j < 4; j++) { w[j] = r[0][j]; w[4 + j] = r[1][j]; }
        } else {
            silu_block_words(r, w);
        }
        // bf16 magnitudes compare as integers; inf / NaN patterns sort above
        // every finite one
        const uint32_t mb = __builtin_elementwise_max(absmax_bits_bf16x8(w), absmax_bits_bf16x8(w + 4));
#pragma unroll
        for (int j = 0; j < 8; j++) {
            f[2 * j] = bf16_lo(w[j]);
            f[2 * j + 1] = bf16_hi(w[j]);
        }
        if (mb < 0x7F80u) return bits_f(mb << 16);
    } else {
        if constexpr (V == V_F32 || V == V_F32_SMOOTH) {
#pragma unroll
            for (int j = 0; j < 16; j++) f[j] = bits_f(r[j >> 2][j & 3]);
        } else {
#pragma unroll
            for (int j = 0; j < 8; j++) {
                const uint32_t xw = r[j >> 2][j & 3];
                f[2 * j] = bf16_lo(xw);
                f[2 * j + 1] = bf16_hi(xw);
            }
        }
        if constexpr (V == V_BF16_SMOOTH || V == V_F32_SMOOTH) {
#pragma unroll
            for (int j = 0; j < 8; j++) {
                const uint32_t pw = pq[j >> 2][j & 3];
                f[2 * j] = f[2 * j] * bf16_lo(pw);
                f[2 * j + 1] = f[2 * j + 1] * bf16_hi(pw);
            }
        }
        float a = 0.0f;
        uint32_t bad = 0;
#pragma unroll
        for (int j = 0; j < 16; j++) {
            a = __builtin_fmaxf(a, __builtin_fabsf(f[j]));
            bad |= (f_bits(f[j]) & 0x7FFFFFFFu) >= 0x7F800000u;
        }
        if (!bad) return a;
    }
    // inf or NaN present: the exact nan_to_num path
    float a = 0.0f;
#pragma unroll
    for (int j = 0; j < 16; j++) {
        f[j] = nan_to_num(f[j]);
        a = __builtin_fmaxf(a, __builtin_fabsf(f[j]));
    }
    return a;
}

// Largest |h| of a silu block (nan_to_num applied), given that `thr` (>= 0,
// a value already attained) is a lower bound of the result: as
// process_block<V_SILU> for the maximum, except that an element flagged only
// for being near a bf16 tie skips the exact path when even the larger of its
// two possible values, |bf16(p)| + 1 ulp, cannot exceed max(thr, the block's
// unflagged magnitudes) -- it cannot change the maximum then.
__device__ __forceinline__ float silu_block_amax(const u32x4 (&r)[4], float thr) {
    uint32_t w[8];
    uint32_t rng = 0, win = 0;
#pragma unroll
    for (int j = 0; j < 8; j++) {
        const uint32_t gw = j < 4 ? r[0][j] : r[1][j - 4];
        const uint32_t uw = j < 4 ? r[2][j] : r[3][j - 4];
        uint32_t rb, wb;
        w[j] = silu_mul_fast2s(gw, uw, rb, wb);
        rng |= rb << (2 * j);
        win |= wb << (2 * j);
    }
    uint32_t need = rng;
    uint32_t tie = win & ~rng;
    if (tie) {
        // bound from thr and the unflagged elements (their bf16 h is exact)
        uint32_t tb = f_bits(thr) >> 16;
        const uint32_t flagged = rng | win;
#pragma unroll
        for (int j = 0; j < 8; j++) {
            const uint32_t m0 = (flagged >> (2 * j)) & 1u ? 0u : w[j] & 0x7FFFu;
            const uint32_t m1 = (flagged >> (2 * j + 1)) & 1u ? 0u : (w[j] >> 16) & 0x7FFFu;
            tb = __builtin_elementwise_max(tb, __builtin_elementwise_max(m0, m1));
        }
        while (tie) {
            const int bit = __builtin_ctz(tie);
            tie &= tie - 1;
            uint32_t hw = 0;
#pragma unroll
            for (int jj = 0; jj < 8; jj++)
                if (jj == (bit >> 1)) hw = w[jj];
            if (((hw >> ((bit & 1) * 16)) & 0x7FFFu) + 1u > tb) need |= 1u << bit;
        }
    }
    while (need) {
        const int bit = __builtin_ctz(need);
        need &= need - 1;
        silu_exact_into(r, bit, w);
    }
    return bf16_words_amax(w);
}

// The 16 values of a block times the element factor r = gs / dec(s), as 16
// e2m1 codes in two dwords (element 2i in the low nibble of byte i).
__device__ __forceinline__ void pack_block(const float (&f)[16], float r, uint32_t& w0, uint32_t& w1) {
    w0 = 0;
    w1 = 0;
    w0 = NVFP4_PACK_FP4(w0, f[0] * r, f[1] * r, 0);
    w0 = NVFP4_PACK_FP4(w0, f[2] * r, f[3] * r, 1);
    w0 = NVFP4_PACK_FP4(w0, f[4] * r, f[5] * r, 2);
    w0 = NVFP4_PACK_FP4(w0, f[6] * r, f[7] * r, 3);
    w1 = NVFP4_PACK_FP4(w1, f[8] * r, f[9] * r, 0);
    w1 = NVFP4_PACK_FP4(w1, f[10] * r, f[11] * r, 1);
    w1 = NVFP4_PACK_FP4(w1, f[12] * r, f[13] * r, 2);
    w1 = NVFP4_PACK_FP4(w1, f[14] * r, f[15] * r, 3);
}

}  // namespace nvfp4
