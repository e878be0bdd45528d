// mx.hip -- the MX setting of the quantizer and the GEMM for gfx950: MXFP4,
// i.e. 32-element blocks with one ue8m0 (power-of-two) scale each, e2m1
// elements and no global scale.
//
// What is computed (flashinfer PR #1774: fp4_quantize takes the block width
// and a ue8m0 flag as positional arguments, set there to 16 / off; the other
// setting is read as the OCP Microscaling Formats v1.0 conversion):
//   x'  = nan_to_num(x)
//   X   = 2^(floor(log2 amax32) - 2)   clamped to [2^-127, 2^127]; code = exponent + 127
//   q   = e2m1(x' / X)                 nearest even, saturating at 6
//   out = bf16(alpha * sum_k dq(a) dq(b) (+ bias)),  dq = e2m1 * 2^(code - 127)
// Scales use the same 128x4 swizzled, zero-padded layout as NVFP4, over k/32
// scale columns, so one 128-element K step of a row has one scale dword.
//
// The GEMM feeds gfx950's block-scaled MFMA directly (v_mfma_scale_f32_32x32x64
// with FP4 operands): lane (row l%32, half h = l/32) of a fragment holds the
// 32 consecutive elements 64q+32h.. of its row for half step q -- exactly one
// MX block -- and supplies that block's scale byte, so no element is ever
// dequantized.  The staging pipeline (FP4 rows and scale dwords straight into
// LDS, three stages) and the epilogue are those of the NVFP4 GEMM.
#include "device_common.h"
#include "gemm_common.h"
#include "internal.h"

namespace nvfp4 {

typedef int i32x8 __attribute__((ext_vector_type(8)));

// ---------------------------------------------------------------------------
// Quantization.  A workgroup of 256 threads owns a 128-row x 128*CT column
// tile (CT whole 512-byte tiles of the scale layout); a lane owns whole
// 32-element blocks: BPR = 4*CT lanes cover one row segment, all of a lane's
// loads are issued before any is used, and the scale bytes are gathered in
// LDS and written with 16-byte stores.
// ---------------------------------------------------------------------------
struct MxQParams {
    const void* x;       // [m, k] bf16 or fp32
    uint8_t* out_fp4;    // [m, k/2]
    uint8_t* out_sf;     // [pad_up(m,128) * pad_up(k/32,4)]
    int64_t m, k;
    int nct;             // 128-column scale tiles = ceil(k/128)
};

// Shared exponent of a block from the bit pattern of its largest magnitude
// (non-negative, finite): floor(log2 amax) - 2, at least -127; amax = 0
// gives -127 (code 0).
__device__ __forceinline__ int mx_shared_exp(uint32_t abits) {
    if (abits == 0) return -127;
    const int e = abits >= 0x00800000u ? (int)(abits >> 23) - 127          // normal
                                       : (31 - __builtin_clz(abits)) - 149;  // subnormal: abits * 2^-149
    return e - 2 < -127 ? -127 : e - 2;  // at most 125 for a finite amax
}

template <bool F32, int CT>
__global__ __launch_bounds__(256) void k_quantize_mx(MxQParams p) {
#if defined(__HIP_DEVICE_COMPILE__)
    constexpr int BPR = 4 * CT, RPP = 256 / BPR, NP = 128 / RPP;
    constexpr int NL = F32 ? 8 : 4;  // 16-byte loads per block
    const int wct = blockIdx.x, rt = blockIdx.y;
    const int t = threadIdx.x;
    const int rsub = t / BPR, lb = t % BPR;
    const int c = lb >> 2, blk = lb & 3;  // scale tile within the workgroup, block column within it
    int64_t col = (int64_t)wct * 128 * CT + lb * 32;
    const bool col_ok = col < p.k;
    col = col_ok ? col : p.k - 32;
    __shared__ __align__(16) uint8_t sbuf[512 * CT];
    const int ntile_here = (p.nct - wct * CT) < CT ? (p.nct - wct * CT) : CT;
    uint8_t* sf_dst = p.out_sf + ((int64_t)rt * p.nct + (int64_t)wct * CT) * 512;

    u32x4 raw[NP][NL];
#pragma unroll
    for (int i = 0; i < NP; i++) {
        int64_t row = (int64_t)rt * 128 + rsub + RPP * i;
        row = row < p.m ? row : p.m - 1;
        const u32x4* src = F32 ? (const u32x4*)((const float*)p.x + row * p.k + col)
                               : (const u32x4*)((const uint16_t*)p.x + row * p.k + col);
#pragma unroll
        for (int j = 0; j < NL; j++) raw[i][j] = src[j];
    }
#pragma unroll
    for (int i = 0; i < NP; i++) {
        const int rl = rsub + RPP * i;
        const int64_t row = (int64_t)rt * 128 + rl;
        const bool active = col_ok && row < p.m;
        float f[32];
        if constexpr (F32) {
#pragma unroll
            for (int j = 0; j < 32; j++) f[j] = bits_f(raw[i][j >> 2][j & 3]);
        } else {
#pragma unroll
            for (int j = 0; j < 16; j++) {
                f[2 * j] = bf16_lo(raw[i][j >> 2][j & 3]);
                f[2 * j + 1] = bf16_hi(raw[i][j >> 2][j & 3]);
            }
        }
        uint32_t mb = 0;
#pragma unroll
        for (int j = 0; j < 32; j++) mb = __builtin_elementwise_max(mb, f_bits(f[j]) & 0x7FFFFFFFu);
        if (mb >= 0x7F800000u) {  // inf or NaN present: nan_to_num, then the maximum again
            mb = 0;
#pragma unroll
            for (int j = 0; j < 32; j++) {
                f[j] = nan_to_num(f[j]);
                mb = __builtin_elementwise_max(mb, f_bits(f[j]) & 0x7FFFFFFFu);
            }
        }
        const int se = mx_shared_exp(mb);
        const float mul = bits_f((uint32_t)(127 - se) << 23);  // 2^-se, a normal fp32 for se in [-127, 125]
        u32x4 w;
#pragma unroll
        for (int d = 0; d < 4; d++) {
            uint32_t v = 0;
            v = NVFP4_PACK_FP4(v, f[8 * d + 0] * mul, f[8 * d + 1] * mul, 0);
            v = NVFP4_PACK_FP4(v, f[8 * d + 2] * mul, f[8 * d + 3] * mul, 1);
            v = NVFP4_PACK_FP4(v, f[8 * d + 4] * mul, f[8 * d + 5] * mul, 2);
            v = NVFP4_PACK_FP4(v, f[8 * d + 6] * mul, f[8 * d + 7] * mul, 3);
            w[d] = v;
        }
        if (active) *(u32x4*)(p.out_fp4 + row * (p.k / 2) + col / 2) = w;
        sbuf[c * 512 + (rl & 31) * 16 + (rl >> 5) * 4 + blk] = active ? (uint8_t)(se + 127) : (uint8_t)0;
    }
    __syncthreads();
    for (int i = t; i < ntile_here * 32; i += 256) *(u32x4*)(sf_dst + i * 16) = *(const u32x4*)(sbuf + i * 16);
#endif
}

hipError_t launch_quantize_mx(const MxQuantizeArgs& a, hipStream_t st) {
    MxQParams p{};
    p.x = a.x; p.out_fp4 = a.out_fp4; p.out_sf = a.out_sf;
    p.m = a.m; p.k = a.k;
    p.nct = (int)((a.k + 127) / 128);
    const int nrt = (int)((a.m + 127) / 128);
    if (a.x_dtype == 1) {
        k_quantize_mx<true, 1><<<dim3(p.nct, nrt), 256, 0, st>>>(p);
    } else {
        k_quantize_mx<false, 2><<<dim3((p.nct + 1) / 2, nrt), 256, 0, st>>>(p);
    }
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// GEMM.  A workgroup computes a BM x BN tile with WGM x WGN waves; each K
// step (128 elements) takes two half steps of FM x FN block-scaled MFMAs.
// ---------------------------------------------------------------------------
template <int WM, int WN>
constexpr int kMxWavesPerEU = WM * WN >= 16384 ? 1 : 2;

__device__ __forceinline__ i32x8 mx_operand(const u32x4& v) {
    return i32x8{(int)v.x, (int)v.y, (int)v.z, (int)v.w, 0, 0, 0, 0};
}

template <int BM, int BN, int WGM, int WGN, int NST, bool ALIGNED>
__global__ __launch_bounds__(64 * WGM * WGN, (kMxWavesPerEU<BM / WGM, BN / WGN>)) void k_gemm_mx(GParams p) {
#if defined(__HIP_DEVICE_COMPILE__)
    constexpr int NW = WGM * WGN;
    constexpr int WM = BM / WGM, WN = BN / WGN;
    constexpr int FM = WM / 32, FN = WN / 32;
    // one LDS stage: FP4 A rows, FP4 B rows, one scale dword per tile row
    // (padded to whole wave loads of 64 dwords per wave)
    constexpr int OFF_B = BM * 64, OFF_S = OFF_B + BN * 64;
    constexpr int SC_DW = (BM + BN + 64 * NW - 1) / (64 * NW) * (64 * NW);
    constexpr int STAGE = OFF_S + SC_DW * 4;
    constexpr int NFA = BM / (16 * NW), NFB = BN / (16 * NW), NSC = SC_DW / (64 * NW);
    constexpr int ND = NFA + NFB + NSC;
    static_assert(BM % (16 * NW) == 0 && BN % (16 * NW) == 0 && BM % 64 == 0, "whole rows per wave load");
    static_assert(NST >= 2 && NST <= 4, "two to four LDS stages");
    __shared__ __align__(16) uint8_t smem[NST * STAGE];

    const int t = threadIdx.x;
    const int lane = t & 63;
    const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
    const int wm = wave % WGM, wn = wave / WGM;
    int tm, tn;
    tile_coords(p, tm, tn);
    const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN;

    const int64_t rowb = p.K / 2;
    const __amdgpu_buffer_rsrc_t rA = make_rsrc(p.a, (uint32_t)(p.M * rowb));
    const __amdgpu_buffer_rsrc_t rB = make_rsrc(p.b, (uint32_t)(p.N * rowb));
    const __amdgpu_buffer_rsrc_t rSA = make_rsrc(p.a_sf, (uint32_t)p.sfa);
    const __amdgpu_buffer_rsrc_t rSB = make_rsrc(p.b_sf, (uint32_t)p.sfb);

    // staging offsets, as in the NVFP4 GEMM (a K step adds 64 bytes of FP4
    // and 512 bytes -- one scale column group -- of scales)
    uint32_t voA[NFA], voB[NFB], voS[NSC];
#pragma unroll
    for (int i = 0; i < NFA; i++) {
        const int r = (i * NW + wave) * 16 + (lane >> 2);
        const int64_t row = m0 + r < p.M ? m0 + r : p.M - 1;
        voA[i] = (uint32_t)(row * rowb) + (uint32_t)((((lane & 3) ^ swz(r)) << 4));
    }
#pragma unroll
    for (int i = 0; i < NFB; i++) {
        const int r = (i * NW + wave) * 16 + (lane >> 2);
        const int64_t row = n0 + r < p.N ? n0 + r : p.N - 1;
        voB[i] = (uint32_t)(row * rowb) + (uint32_t)((((lane & 3) ^ swz(r)) << 4));
    }
#pragma unroll
    for (int i = 0; i < NSC; i++) {
        const int tr = (i * NW + wave) * 64 + lane;  // tile row of this scale dword
        if (tr < BM) {
            const int64_t row = m0 + tr < p.rpa ? m0 + tr : p.rpa - 1;
            voS[i] = scale_dword_off(row, 0, p.cpa4);
        } else if (tr < BM + BN) {
            const int64_t row = n0 + (tr - BM) < p.rpb ? n0 + (tr - BM) : p.rpb - 1;
            voS[i] = scale_dword_off(row, 0, p.cpa4);
        } else {
            voS[i] = 0;  // padding dwords: any in-bounds source
        }
    }
    lds_u8* const sm = (lds_u8*)smem;
    auto issue = [&](int step, lds_u8* st) {
#pragma unroll
        for (int i = 0; i < NFA; i++)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rA, (__attribute__((address_space(3))) void*)(st + (i * NW + wave) * 1024),
                                                     16, voA[i], step * 64, 0, 0);
#pragma unroll
        for (int i = 0; i < NFB; i++)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rB, (__attribute__((address_space(3))) void*)(st + OFF_B + (i * NW + wave) * 1024),
                                                     16, voB[i], step * 64, 0, 0);
#pragma unroll
        for (int i = 0; i < NSC; i++) {
            const bool isA = (i * NW + wave) * 64 < BM;  // a wave load covers 64 tile rows: all A or all B
            __builtin_amdgcn_raw_ptr_buffer_load_lds(isA ? rSA : rSB,
                                                     (__attribute__((address_space(3))) void*)(st + OFF_S + (i * NW + wave) * 256),
                                                     4, voS[i], step * 512, 0, 0);
        }
    };

    f32x16 acc[FN][FM];
#pragma unroll
    for (int i = 0; i < FN; i++)
#pragma unroll
        for (int j = 0; j < FM; j++)
#pragma unroll
            for (int v = 0; v < 16; v++) acc[i][j][v] = 0.0f;

    const int nkt = (int)((p.K + 127) / 128);
    const int h = lane >> 5, l32 = lane & 31;
    const int ra_off = (wm * WM + l32) * 64, rb_off = OFF_B + (wn * WN + l32) * 64;
    const int xr = swz(l32);
    const int cq0 = ((h ^ xr) << 4), cq1 = (((2 + h) ^ xr) << 4);
    const int sa_off = OFF_S + (wm * WM + l32) * 4;
    const int sb_off = OFF_S + (BM + wn * WN + l32) * 4;

    // fragments of half step q and the scale dwords of a step (shifted so the
    // lane's block of half step q sits in byte 2q, selected by the MFMA's
    // opsel); blocks past K (only when K % 128 != 0) get zero elements
    u32x4 fa[2][FM], fb[2][FN];
    auto load_scales = [&](const lds_u8* st, int (&sa)[FM], int (&sb)[FN]) {
#pragma unroll
        for (int i = 0; i < FM; i++)
            sa[i] = (int)(*(const __attribute__((address_space(3))) uint32_t*)(st + sa_off + i * 128) >> (8 * h));
#pragma unroll
        for (int i = 0; i < FN; i++)
            sb[i] = (int)(*(const __attribute__((address_space(3))) uint32_t*)(st + sb_off + i * 128) >> (8 * h));
    };
    auto load_half = [&](const lds_u8* st, int step, int q) {
        const int cq = q ? cq1 : cq0;
#pragma unroll
        for (int i = 0; i < FM; i++) fa[q][i] = *(const __attribute__((address_space(3))) u32x4*)(st + ra_off + i * 2048 + cq);
#pragma unroll
        for (int i = 0; i < FN; i++) fb[q][i] = *(const __attribute__((address_space(3))) u32x4*)(st + rb_off + i * 2048 + cq);
        if constexpr (!ALIGNED) {
            if (step * 4 + 2 * q + h >= p.nblk) {
#pragma unroll
                for (int i = 0; i < FM; i++) fa[q][i] = u32x4{0u, 0u, 0u, 0u};
#pragma unroll
                for (int i = 0; i < FN; i++) fb[q][i] = u32x4{0u, 0u, 0u, 0u};
            }
        }
    };
    // B is the MFMA's first operand (4 consecutive output columns per lane)
    auto mfma_half0 = [&](const int (&sa)[FM], const int (&sb)[FN]) {
#pragma unroll
        for (int in = 0; in < FN; in++)
#pragma unroll
            for (int im = 0; im < FM; im++)
                acc[in][im] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                    mx_operand(fb[0][in]), mx_operand(fa[0][im]), acc[in][im], 4, 4, 0, sb[in], 0, sa[im]);
    };
    auto mfma_half1 = [&](const int (&sa)[FM], const int (&sb)[FN]) {
#pragma unroll
        for (int in = 0; in < FN; in++)
#pragma unroll
            for (int im = 0; im < FM; im++)
                acc[in][im] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                    mx_operand(fb[1][in]), mx_operand(fa[1][im]), acc[in][im], 4, 4, 2, sb[in], 2, sa[im]);
    };
    auto barrier = [&]() {
        __builtin_amdgcn_s_waitcnt((0x3F & 0xF) | (0x3 << 14) | (0x7 << 4) | (0x0 << 8));  // lgkmcnt(0)
        asm volatile("s_barrier" ::: "memory");
    };

    // Step kt lives in stage kt % NST; its loads are issued NST-1 steps ahead
    // into the stage step kt-1 used, which every wave has finished reading
    // (its reads complete before the barrier in the middle of step kt-1's
    // MFMAs).  The LDS reads of each half step are in flight during the
    // other half's MFMAs: q = 1 of step kt beside q = 0, and after the
    // barrier the scales and q = 0 of step kt+1 beside q = 1 of step kt
    // (measured: 2-3% over letting the compiler place the reads; a fourth
    // stage, two K steps per barrier and 128 x 128 wave tiles at one wave per
    // SIMD were no faster).  The last step's read of the next stage finds a
    // reloaded copy of the final step, unused.
#pragma unroll
    for (int j = 0; j < NST - 1; j++) issue(j < nkt ? j : nkt - 1, sm + j * STAGE);
    wait_vmcnt<ND * (NST - 2)>();
    barrier();
    int sa[FM], sb[FN];
    load_scales(sm, sa, sb);
    load_half(sm, 0, 0);
    int sc = 0;
    for (int kt = 0; kt < nkt; kt++) {
        const int s1 = sc == NST - 1 ? 0 : sc + 1;
        const int sl = sc == 0 ? NST - 1 : sc - 1;  // stage of step kt+NST-1 (= that of step kt-1)
        issue(kt + NST - 1 < nkt ? kt + NST - 1 : nkt - 1, sm + sl * STAGE);
        load_half(sm + sc * STAGE, kt, 1);
        mfma_half0(sa, sb);
        // staging loads, then the q = 1 reads, then the q = 0 MFMAs
        __builtin_amdgcn_sched_group_barrier(0x020, ND, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, FM + FN, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, FM * FN, 0);
        __builtin_amdgcn_sched_barrier(0);
        wait_vmcnt<ND * (NST - 2)>();  // step kt+1 has landed (this wave's part)
        barrier();
        __builtin_amdgcn_sched_barrier(0);
        int na[FM], nb[FN];
        load_scales(sm + s1 * STAGE, na, nb);
        load_half(sm + s1 * STAGE, kt + 1, 0);
        mfma_half1(sa, sb);
        // the next step's scale and q = 0 reads, then the q = 1 MFMAs
        __builtin_amdgcn_sched_group_barrier(0x100, 2 * (FM + FN), 0);
        __builtin_amdgcn_sched_group_barrier(0x008, FM * FN, 0);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < FM; i++) sa[i] = na[i];
#pragma unroll
        for (int i = 0; i < FN; i++) sb[i] = nb[i];
        sc = s1;
    }
    wait_vmcnt<0>();  // this wave's staging loads have landed

    // ---- epilogue: alpha, bias, bf16, staged through LDS one 32-row
    // fragment row at a time so every output row leaves as 16-byte pieces.
    // The staging region overlaps the pipeline stages: the barrier holds it
    // until every wave's last staging loads have landed.
    constexpr int PITCH = WN * 2 + 16;
    static_assert(NW * 32 * PITCH <= NST * STAGE, "epilogue staging fits in the pipeline's LDS");
    barrier();
    lds_u8* const ep = sm + wave * 32 * PITCH;
    const float alpha = p.alpha ? p.alpha[0] : 1.0f;
    constexpr int CPR = WN / 8, RPI = 64 / CPR;
#pragma unroll
    for (int im = 0; im < FM; im++) {
#pragma unroll
        for (int in = 0; in < FN; in++) {
#pragma unroll
            for (int g = 0; g < 4; g++) {
                const int cl = in * 32 + g * 8 + h * 4;
                const int64_t n = n0 + wn * WN + cl;
                float y[4];
#pragma unroll
                for (int u = 0; u < 4; u++) {
                    y[u] = alpha * acc[in][im][g * 4 + u];
                    if (p.bias && n + u < p.N) y[u] += bf16_lo((uint32_t)p.bias[n + u]);
                }
                *(__attribute__((address_space(3))) u32x2*)(ep + l32 * PITCH + cl * 2) =
                    u32x2{pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3])};
            }
        }
        __builtin_amdgcn_s_waitcnt((0x3F & 0xF) | (0x3 << 14) | (0x7 << 4) | (0x0 << 8));  // lgkmcnt(0)
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int it = 0; it < 32 / RPI; it++) {
            const int rl = it * RPI + lane / CPR, c = lane % CPR;
            const u32x4 v = *(const __attribute__((address_space(3))) u32x4*)(ep + rl * PITCH + c * 16);
            const int64_t m = m0 + wm * WM + im * 32 + rl;
            const int64_t n = n0 + wn * WN + c * 8;
            if (m >= p.M) continue;
            if (n + 8 <= p.N && (p.N & 7) == 0) {
                *(u32x4*)(p.out + m * p.N + n) = v;
            } else {
#pragma unroll
                for (int u = 0; u < 8; u++)
                    if (n + u < p.N) p.out[m * p.N + n + u] = (uint16_t)(v[u >> 1] >> (16 * (u & 1)));
            }
        }
        __builtin_amdgcn_s_waitcnt((0x3F & 0xF) | (0x3 << 14) | (0x7 << 4) | (0x0 << 8));  // reads done before the region is rewritten
        __builtin_amdgcn_sched_barrier(0);
    }
#endif
}

template <int BM, int BN, int WGM, int WGN, int NST>
static hipError_t launch_mx_tile(GParams p, hipStream_t st) {
    p.tiles_m = (int)((p.M + BM - 1) / BM);
    p.tiles_n = (int)((p.N + BN - 1) / BN);
    const int tiles = p.tiles_m * p.tiles_n;
    p.xcd_chunk = tiles % 8 == 0 ? tiles / 8 : 0;
    if (p.K % 128 == 0) k_gemm_mx<BM, BN, WGM, WGN, NST, true><<<tiles, 64 * WGM * WGN, 0, st>>>(p);
    else k_gemm_mx<BM, BN, WGM, WGN, NST, false><<<tiles, 64 * WGM * WGN, 0, st>>>(p);
    return hipGetLastError();
}

hipError_t launch_gemm_mx(const GemmArgs& g, hipStream_t st) {
    GParams p{};
    p.a = g.a; p.b = g.b; p.a_sf = g.a_sf; p.b_sf = g.b_sf;
    p.alpha = g.alpha; p.bias = g.bias; p.out = g.out;
    p.M = g.m; p.N = g.n; p.K = g.k; p.E = 1;
    const int64_t cp = ((g.k / 32) + 3) / 4 * 4;
    p.cpa4 = (int)(cp / 4);
    p.nblk = (int)(g.k / 32);
    p.rpa = (int)((g.m + 127) / 128 * 128);
    p.rpb = (int)((g.n + 127) / 128 * 128);
    p.sfa = (int64_t)p.rpa * cp;
    p.sfb = (int64_t)p.rpb * cp;
    const int64_t t256 = ((g.m + 255) / 256) * ((g.n + 255) / 256);
    if (t256 >= 256) return launch_mx_tile<256, 256, 4, 2, 3>(p, st);
    return launch_mx_tile<128, 128, 2, 2, 2>(p, st);
}

}  // namespace nvfp4
