// gemm.hip -- block-scaled NVFP4 GEMM for gfx950 (dense, grouped-masked and
// SVDQuant forms).
//
// What is computed (flashinfer mm_nvfp4_svdquant: out = alpha*(a@b^T) +
// d@l1^T [+bias], the rank-r term entering the same accumulator after the
// NVFP4 K loop; flashinfer PR #1774: grouped_gemm_nt_masked over experts;
// NVIDIA/Fuser PR #5737: eager meaning = dequantize, then linear):
//   acc[m,n] = sum_k dq(a)[m,k] * dq(b)[n,k]  (+ sum_p d[m,p] * l1[n,p])
//   out[m,n] = bf16(alpha * acc (+ bias[n]))
// with dq(x) = e2m1(x) * ue4m3(scale of x's 16-element block).
//
// How the 16-element e4m3 block scales meet CDNA4 MFMA: each operand element
// is dequantized in registers to fp16, exactly (e2m1 has 2 significant bits,
// ue4m3 4, so the product has at most 6; its range 2^-10 .. 2688 is inside
// fp16's normal range), and fed to v_mfma_f32_32x32x16_f16, which
// accumulates in fp32.  The hardware FP4 converts apply only the exponent of
// their fp32 scale operand, so the conversion runs with scale 1.0 and the
// block scale is applied with one packed fp16 multiply per element pair.
// gfx950's native scaled MFMA takes one power-of-two (e8m0) scale per 32
// elements and cannot carry a 16-element e4m3 scale exactly.
//
// Tiling: a 256-thread workgroup computes a BM x BN tile, 2 x 2 waves of
// (BM/2) x (BN/2), each wave a grid of 32 x 32 MFMA fragments.  K advances
// 128 elements (64 bytes of a row) per step; the FP4 tiles and their scales
// are staged in LDS.  Within a 64-element half-step, lane l of a fragment
// (row l%32, half h = l/32) owns the 32 consecutive elements 32h.. of its
// row: one 16-byte LDS read, two block scales, four MFMA K-slices.  The same
// K permutation is used for both operands, so the contraction is unchanged.
// The MFMA's first operand is the B fragment and its second the A fragment,
// which puts 4 consecutive output columns of one output row in each lane.
#include "device_common.h"
#include "internal.h"

namespace nvfp4 {

struct GParams {
    const uint8_t* a;
    const uint8_t* b;
    const uint8_t* a_sf;
    const uint8_t* b_sf;
    const float* alpha;
    const int32_t* mask;
    const uint16_t* bias;
    const uint16_t* d;
    const uint16_t* l1;
    uint16_t* out;
    int64_t M, N, K, r, E;
    int64_t sfa, sfb;    // per-expert scale buffer bytes
    int cpa4;            // column groups of the scale layout = pad_up(K/16,4)/4
    int rpa, rpb;        // padded rows of the scale buffers
    int tiles_m, tiles_n;
};

constexpr int kPitch = 80;  // LDS row pitch of a 64-byte FP4 row (+16 avoids bank conflicts)

__device__ __forceinline__ f16x2 dup_scale_f16(uint32_t code) {
    _Float16 h = (_Float16)ue4m3_decode(code);
    return f16x2{h, h};
}

// 8 FP4 codes of one dword times one block scale -> 8 fp16 (exact).
__device__ __forceinline__ f16x8 dequant8(uint32_t w, f16x2 s) {
    f16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0) * s;
    f16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1) * s;
    f16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2) * s;
    f16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3) * s;
    return f16x8{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
}

// Global -> register staging of one K step (128 elements) of the A and B
// tiles and their scales.  Addresses are clamped into the buffers so every
// load is issued unconditionally (all of them stay in flight together);
// values from rows or K blocks outside the matrix are zeroed when stored.
template <int BM, int BN, bool ALIGNED>
struct Stage {
    static constexpr int CH = ALIGNED ? 16 : 8;          // bytes per chunk
    static constexpr int CPR = 64 / CH;                  // chunks per row
    static constexpr int NA = (BM * CPR + 255) / 256;    // A chunks per thread
    static constexpr int NB = (BN * CPR + 255) / 256;
    static constexpr int NSA = (BM * 2 + 255) / 256;     // A scale dwords per thread
    static constexpr int NSB = (BN * 2 + 255) / 256;
    uint4 ra[NA], rb[NB];
    uint32_t sa[NSA], sb[NSB];
};

template <int BM, int BN, bool ALIGNED>
__device__ __forceinline__ void stage_load(Stage<BM, BN, ALIGNED>& st, const GParams& p,
                                           const uint8_t* A, const uint8_t* B,
                                           const uint8_t* SA, const uint8_t* SB,
                                           int64_t m0, int64_t n0, int kt, int t) {
    using S = Stage<BM, BN, ALIGNED>;
    const int64_t rowb = p.K / 2;
#pragma unroll
    for (int i = 0; i < S::NA; i++) {
        const int idx = t + 256 * i;
        const int r = idx / S::CPR, c = idx % S::CPR;
        int64_t row = m0 + r;
        row = row < p.M ? row : p.M - 1;
        if constexpr (ALIGNED) {
            st.ra[i] = *(const uint4*)(A + row * rowb + kt * 64 + c * 16);
        } else {
            int64_t kb = (int64_t)kt * 64 + c * 8;
            kb = kb < rowb ? kb : rowb - 8;
            uint2 v = *(const uint2*)(A + row * rowb + kb);
            st.ra[i] = uint4{v.x, v.y, 0u, 0u};
        }
    }
#pragma unroll
    for (int i = 0; i < S::NB; i++) {
        const int idx = t + 256 * i;
        const int r = idx / S::CPR, c = idx % S::CPR;
        int64_t row = n0 + r;
        row = row < p.N ? row : p.N - 1;
        if constexpr (ALIGNED) {
            st.rb[i] = *(const uint4*)(B + row * rowb + kt * 64 + c * 16);
        } else {
            int64_t kb = (int64_t)kt * 64 + c * 8;
            kb = kb < rowb ? kb : rowb - 8;
            uint2 v = *(const uint2*)(B + row * rowb + kb);
            st.rb[i] = uint4{v.x, v.y, 0u, 0u};
        }
    }
#pragma unroll
    for (int i = 0; i < S::NSA; i++) {
        const int idx = (t + 256 * i) % (BM * 2);
        const int r = idx >> 1, g = idx & 1;
        int64_t row = m0 + r;
        row = row < p.rpa ? row : p.rpa - 1;
        int cg = kt * 2 + g;
        cg = cg < p.cpa4 ? cg : p.cpa4 - 1;
        st.sa[i] = *(const uint32_t*)(SA + ((row >> 7) * p.cpa4 + cg) * 512 + (row & 31) * 16 + ((row & 127) >> 5) * 4);
    }
#pragma unroll
    for (int i = 0; i < S::NSB; i++) {
        const int idx = (t + 256 * i) % (BN * 2);
        const int r = idx >> 1, g = idx & 1;
        int64_t row = n0 + r;
        row = row < p.rpb ? row : p.rpb - 1;
        int cg = kt * 2 + g;
        cg = cg < p.cpa4 ? cg : p.cpa4 - 1;
        st.sb[i] = *(const uint32_t*)(SB + ((row >> 7) * p.cpa4 + cg) * 512 + (row & 31) * 16 + ((row & 127) >> 5) * 4);
    }
}

template <int BM, int BN, bool ALIGNED>
__device__ __forceinline__ void stage_store(const Stage<BM, BN, ALIGNED>& st, const GParams& p,
                                            uint8_t* sA, uint8_t* sB, uint8_t* sSA, uint8_t* sSB,
                                            int64_t m0, int64_t n0, int kt, int t) {
    using S = Stage<BM, BN, ALIGNED>;
#pragma unroll
    for (int i = 0; i < S::NA; i++) {
        const int idx = t + 256 * i;
        if (S::NA * 256 > BM * S::CPR && idx >= BM * S::CPR) break;
        const int r = idx / S::CPR, c = idx % S::CPR;
        bool ok = m0 + r < p.M;
        if constexpr (ALIGNED) {
            uint4 v = st.ra[i];
            if (!ok) v = uint4{0u, 0u, 0u, 0u};
            *(uint4*)(sA + r * kPitch + c * 16) = v;
        } else {
            ok = ok && (int64_t)kt * 128 + c * 16 < p.K;
            uint2 v = uint2{st.ra[i].x, st.ra[i].y};
            if (!ok) v = uint2{0u, 0u};
            *(uint2*)(sA + r * kPitch + c * 8) = v;
        }
    }
#pragma unroll
    for (int i = 0; i < S::NB; i++) {
        const int idx = t + 256 * i;
        if (S::NB * 256 > BN * S::CPR && idx >= BN * S::CPR) break;
        const int r = idx / S::CPR, c = idx % S::CPR;
        bool ok = n0 + r < p.N;
        if constexpr (ALIGNED) {
            uint4 v = st.rb[i];
            if (!ok) v = uint4{0u, 0u, 0u, 0u};
            *(uint4*)(sB + r * kPitch + c * 16) = v;
        } else {
            ok = ok && (int64_t)kt * 128 + c * 16 < p.K;
            uint2 v = uint2{st.rb[i].x, st.rb[i].y};
            if (!ok) v = uint2{0u, 0u};
            *(uint2*)(sB + r * kPitch + c * 8) = v;
        }
    }
#pragma unroll
    for (int i = 0; i < S::NSA; i++) {
        const int idx = t + 256 * i;
        if (idx >= BM * 2) break;
        const int r = idx >> 1, g = idx & 1;
        const bool ok = m0 + r < p.rpa && kt * 2 + g < p.cpa4;
        *(uint32_t*)(sSA + r * 8 + g * 4) = ok ? st.sa[i] : 0u;
    }
#pragma unroll
    for (int i = 0; i < S::NSB; i++) {
        const int idx = t + 256 * i;
        if (idx >= BN * 2) break;
        const int r = idx >> 1, g = idx & 1;
        const bool ok = n0 + r < p.rpb && kt * 2 + g < p.cpa4;
        *(uint32_t*)(sSB + r * 8 + g * 4) = ok ? st.sb[i] : 0u;
    }
}

template <int BM, int BN, bool ALIGNED, bool LORA>
__global__ __launch_bounds__(256) void k_gemm(GParams p) {
    constexpr int WM = BM / 2, WN = BN / 2;
    constexpr int FM = WM / 32, FN = WN / 32;
    constexpr int OFF_B = BM * kPitch, OFF_SA = OFF_B + BN * kPitch, OFF_SB = OFF_SA + BM * 8;
    constexpr int STAGE = OFF_SB + BN * 8;
    __shared__ __align__(16) uint8_t smem[2 * STAGE];

    const int t = threadIdx.x;
    const int lane = t & 63, wave = t >> 6;
    const int wm = wave & 1, wn = wave >> 1;
    const int e = blockIdx.z;
    const int tile = blockIdx.x;
    const int tm = tile / p.tiles_n, tn = tile - tm * p.tiles_n;
    const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN;
    const int valid = clamp_rows(p.mask, e, (int)p.M);
    if (m0 >= valid) return;  // whole tile past this expert's valid rows

    const int64_t rowb = p.K / 2;
    const uint8_t* A = p.a + (int64_t)e * p.M * rowb;
    const uint8_t* B = p.b + (int64_t)e * p.N * rowb;
    const uint8_t* SA = p.a_sf + (int64_t)e * p.sfa;
    const uint8_t* SB = p.b_sf + (int64_t)e * p.sfb;

    f32x16 acc[FN][FM];
#pragma unroll
    for (int i = 0; i < FN; i++)
#pragma unroll
        for (int j = 0; j < FM; j++)
#pragma unroll
            for (int v = 0; v < 16; v++) acc[i][j][v] = 0.0f;

    const int nkt = (int)((p.K + 127) / 128);
    const int h = lane >> 5, l32 = lane & 31;

    Stage<BM, BN, ALIGNED> st;
    stage_load<BM, BN, ALIGNED>(st, p, A, B, SA, SB, m0, n0, 0, t);
    stage_store<BM, BN, ALIGNED>(st, p, smem, smem + OFF_B, smem + OFF_SA, smem + OFF_SB, m0, n0, 0, t);
    __syncthreads();

    for (int kt = 0; kt < nkt; kt++) {
        const bool more = kt + 1 < nkt;
        if (more) stage_load<BM, BN, ALIGNED>(st, p, A, B, SA, SB, m0, n0, kt + 1, t);
        const uint8_t* cur = smem + (kt & 1) * STAGE;
        const uint8_t* sA = cur;
        const uint8_t* sB = cur + OFF_B;
        const uint8_t* sSA = cur + OFF_SA;
        const uint8_t* sSB = cur + OFF_SB;

        // ---- compute: two 64-element halves, four 16-element K-slices each
#pragma unroll
        for (int q = 0; q < 2; q++) {
            uint4 fa[FM], fb[FN];
            f16x2 ca[FM][2], cb[FN][2];
#pragma unroll
            for (int i = 0; i < FM; i++) {
                const int r = wm * WM + i * 32 + l32;
                fa[i] = *(const uint4*)(sA + r * kPitch + q * 32 + h * 16);
                const uint32_t s2 = *(const uint16_t*)(sSA + r * 8 + q * 4 + h * 2);
                ca[i][0] = dup_scale_f16(s2 & 0xFFu);
                ca[i][1] = dup_scale_f16(s2 >> 8);
            }
#pragma unroll
            for (int i = 0; i < FN; i++) {
                const int r = wn * WN + i * 32 + l32;
                fb[i] = *(const uint4*)(sB + r * kPitch + q * 32 + h * 16);
                const uint32_t s2 = *(const uint16_t*)(sSB + r * 8 + q * 4 + h * 2);
                cb[i][0] = dup_scale_f16(s2 & 0xFFu);
                cb[i][1] = dup_scale_f16(s2 >> 8);
            }
#pragma unroll
            for (int j = 0; j < 4; j++) {
                f16x8 oa[FM], ob[FN];
#pragma unroll
                for (int i = 0; i < FM; i++) {
                    const uint32_t w = j == 0 ? fa[i].x : j == 1 ? fa[i].y : j == 2 ? fa[i].z : fa[i].w;
                    oa[i] = dequant8(w, ca[i][j >> 1]);
                }
#pragma unroll
                for (int i = 0; i < FN; i++) {
                    const uint32_t w = j == 0 ? fb[i].x : j == 1 ? fb[i].y : j == 2 ? fb[i].z : fb[i].w;
                    ob[i] = dequant8(w, cb[i][j >> 1]);
                }
#pragma unroll
                for (int in = 0; in < FN; in++)
#pragma unroll
                    for (int im = 0; im < FM; im++)
                        acc[in][im] = __builtin_amdgcn_mfma_f32_32x32x16_f16(ob[in], oa[im], acc[in][im], 0, 0, 0);
            }
        }
        if (more) {
            uint8_t* nxt = smem + ((kt + 1) & 1) * STAGE;
            stage_store<BM, BN, ALIGNED>(st, p, nxt, nxt + OFF_B, nxt + OFF_SA, nxt + OFF_SB, m0, n0, kt + 1, t);
        }
        __syncthreads();
    }

    if constexpr (LORA) {
        // rank-r bf16 correction into the same accumulator
        for (int kr = 0; kr < p.r; kr += 16) {
            bf16x8 od[FM], ol[FN];
#pragma unroll
            for (int i = 0; i < FM; i++) {
                int64_t row = m0 + wm * WM + i * 32 + l32;
                row = row < p.M ? row : p.M - 1;
                uint4 v = *(const uint4*)(p.d + row * p.r + kr + h * 8);
                od[i] = __builtin_bit_cast(bf16x8, v);
            }
#pragma unroll
            for (int i = 0; i < FN; i++) {
                int64_t row = n0 + wn * WN + i * 32 + l32;
                row = row < p.N ? row : p.N - 1;
                uint4 v = *(const uint4*)(p.l1 + row * p.r + kr + h * 8);
                ol[i] = __builtin_bit_cast(bf16x8, v);
            }
#pragma unroll
            for (int in = 0; in < FN; in++)
#pragma unroll
                for (int im = 0; im < FM; im++)
                    acc[in][im] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ol[in], od[im], acc[in][im], 0, 0, 0);
        }
    }

    // ---- epilogue: alpha, bias, bf16, store rows < valid
    const float alpha = p.alpha[e];
    uint16_t* O = p.out + (int64_t)e * p.M * p.N;
    const bool vec_ok = (p.N & 3) == 0;
#pragma unroll
    for (int in = 0; in < FN; in++) {
#pragma unroll
        for (int im = 0; im < FM; im++) {
            const int64_t m = m0 + wm * WM + im * 32 + l32;
            if (m >= valid) continue;
#pragma unroll
            for (int g = 0; g < 4; g++) {
                const int64_t n = n0 + wn * WN + in * 32 + g * 8 + h * 4;
                float y[4];
#pragma unroll
                for (int u = 0; u < 4; u++) {
                    y[u] = alpha * acc[in][im][g * 4 + u];
                    if (p.bias && n + u < p.N) y[u] += bf16_lo((uint32_t)p.bias[n + u]);
                }
                if (vec_ok && n + 3 < p.N) {
                    uint2 v;
                    v.x = f32_to_bf16_rne(y[0]) | (f32_to_bf16_rne(y[1]) << 16);
                    v.y = f32_to_bf16_rne(y[2]) | (f32_to_bf16_rne(y[3]) << 16);
                    *(uint2*)(O + m * p.N + n) = v;
                } else {
#pragma unroll
                    for (int u = 0; u < 4; u++)
                        if (n + u < p.N) O[m * p.N + n + u] = (uint16_t)f32_to_bf16_rne(y[u]);
                }
            }
        }
    }
}

template <int BM, int BN>
static hipError_t launch_tile(GParams p, bool lora, hipStream_t st) {
    p.tiles_m = (int)((p.M + BM - 1) / BM);
    p.tiles_n = (int)((p.N + BN - 1) / BN);
    dim3 grid(p.tiles_m * p.tiles_n, 1, (unsigned)p.E ? (unsigned)p.E : 1u);
    const bool aligned = (p.K % 128) == 0;
    if (lora) {
        if (aligned) k_gemm<BM, BN, true, true><<<grid, 256, 0, st>>>(p);
        else k_gemm<BM, BN, false, true><<<grid, 256, 0, st>>>(p);
    } else {
        if (aligned) k_gemm<BM, BN, true, false><<<grid, 256, 0, st>>>(p);
        else k_gemm<BM, BN, false, false><<<grid, 256, 0, st>>>(p);
    }
    return hipGetLastError();
}

hipError_t launch_gemm(const GemmArgs& g, hipStream_t st) {
    GParams p{};
    p.a = g.a; p.b = g.b; p.a_sf = g.a_sf; p.b_sf = g.b_sf;
    p.alpha = g.alpha; p.mask = g.mask; p.bias = g.bias; p.d = g.d; p.l1 = g.l1;
    p.out = g.out;
    p.M = g.m; p.N = g.n; p.K = g.k; p.r = g.r;
    p.E = g.E;
    const int64_t cp = ((g.k / 16) + 3) / 4 * 4;
    p.cpa4 = (int)(cp / 4);
    p.rpa = (int)((g.m + 127) / 128 * 128);
    p.rpb = (int)((g.n + 127) / 128 * 128);
    p.sfa = (int64_t)p.rpa * cp;
    p.sfb = (int64_t)p.rpb * cp;
    const bool lora = g.d != nullptr;
    const int64_t work = g.m * g.n;
    if (g.m >= 2048 && g.n >= 2048 && work >= (int64_t)4096 * 4096)
        return launch_tile<256, 256>(p, lora, st);
    if (g.m <= 64)
        return launch_tile<64, 128>(p, lora, st);
    return launch_tile<128, 128>(p, lora, st);
}

}  // namespace nvfp4
