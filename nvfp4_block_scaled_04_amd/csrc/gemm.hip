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
// Tiling: a workgroup computes a BM x BN tile with WGM x WGN waves of
// (BM/WGM) x (BN/WGN), each wave a grid of 32 x 32 MFMA fragments: 4 x 2
// waves of 64 x 128 for the 256 x 256 tile (two waves per SIMD, so one
// wave's dequantization and LDS waits overlap the other's MFMAs; measured
// 2% faster than 2 x 2 waves of 128 x 128 with one wave per SIMD), 4 x 2
// waves of 64 x 96 for the 256 x 192 tile, 2 x 2 waves for the smaller
// tiles.  K advances
// 128 elements (64 bytes of a row) per step.  A step's FP4 rows and raw scale
// bytes go from global memory straight into LDS (buffer loads with the LDS
// bit: no registers), two or three stages deep, so a step's loads are issued
// one or two steps before it is consumed (the 256 x 256 tile runs a step of
// about 3 us, which covers the load latency with two stages: measured 1.5%
// faster than three; the quantizing epilogue's launch keeps three, measured
// faster there).  Within a 64-element half step q, lane l of a
// fragment (row l%32, half h = l/32) owns the 32 consecutive elements
// 64q+32h.. of its row: one 16-byte LDS read, two block scales, four MFMA
// K-slices.  The same K permutation is used for both operands, so the
// contraction is unchanged.  The dequantization of slice s+1 is issued
// between the MFMAs of slice s, and the MFMAs of a step's last slice run
// after the step barrier, next to the next step's first LDS reads.  The
// MFMA's first operand is the B fragment and its second the A fragment, which
// puts 4 consecutive output columns of one output row in each lane.
#include "device_common.h"
#include "gemm_common.h"
#include "internal.h"
#include "quant_block.h"

namespace nvfp4 {

typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));

// Epilogues of k_gemm: bf16 output; bf16 output after the rank-r LoRA-up
// term; or silu_and_mul of the gate | up output quantized to NVFP4.
enum Epilogue { EPI_PLAIN = 0, EPI_LORA = 1, EPI_SILUQ = 2 };

// Waves per SIMD each configuration is compiled for: a 128x128 wave tile
// takes the whole register file (256 accumulators per lane); smaller wave
// tiles are held to 256 registers so two waves share a SIMD.
template <int WM, int WN>
constexpr int kWavesPerEU = WM * WN >= 16384 ? 1 : 2;

// Split-tail schedule over rounds of G = p.sk_grid workgroups (one per CU;
// the workgroups of a round start as those of the previous one finish).  The
// T live tiles (experts in order; within an expert, bands
// of 8 tile rows walked column by column, as tile_coords does) are cut into
// D = floor(T/G)*G whole tiles, dealt G per round (XCD x taking the x-th
// eighth of a round, so tiles that share panels share an L2), and R = T - D
// tail tiles.  The K steps of a tail tile are split into S = min(G/R, steps
// per K group / 4) parts of whole groups of KS steps, one part per
// workgroup, so every CU receives the same work to within one part.  With
// S > 1 each part leaves an fp32 partial tile in workspace slot (r*S + j)
// and a second launch (k_gemm_fixup) adds a tail tile's S partials in part
// order: deterministic, and no workgroup ever waits for another.  Without a
// workspace, S = 1 (the tail tiles run whole).  Every workgroup of both
// launches derives the schedule from the mask itself.
struct SkPlan {
    int T, D, R, S;
};

// Live tile rows of expert `lane` (0 for lanes >= E; E <= 64): the mask is
// read once per wave, one expert per lane, all loads in flight together.
__device__ __forceinline__ int sk_lane_rows(const GParams& p, int bm) {
    const int lane = (int)(threadIdx.x & 63);
    const int v = lane < (int)p.E ? clamp_rows(p.mask, lane, (int)p.M) : 0;
    return (v + bm - 1) / bm;
}

__device__ __forceinline__ SkPlan sk_plan(const GParams& p, int tme_lane, int nkt, int ks) {
    int T = tme_lane * p.tiles_n;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) T += __shfl_xor(T, off);
    const int G = p.sk_grid;
    SkPlan s;
    s.T = T;
    s.D = T / G * G;
    s.R = T - s.D;
    // parts of at least 4 K-step pairs (of KS steps): shorter ones cost
    // more in pipeline fill and partial-tile traffic than they balance
    int S = s.R ? G / s.R : 0;
    const int smax = nkt / ks / 4 > 1 ? nkt / ks / 4 : 1;
    if (S > smax) S = smax;
    if (!p.part && S > 1) S = 1;
    s.S = S;
    return s;
}

// Expert and tile coordinates of live tile idx (0 <= idx < T); tme_lane
// from sk_lane_rows (every lane of the wave active).
__device__ __forceinline__ void sk_tile(const GParams& p, int tme_lane, int idx, int& e, int& tm, int& tn) {
    int tme = 0;
    for (e = 0; e < (int)p.E; e++) {
        tme = __shfl(tme_lane, e);
        const int cnt = tme * p.tiles_n;
        if (idx < cnt || e == (int)p.E - 1) break;
        idx -= cnt;
    }
    constexpr int G8 = 8;
    const int per = G8 * p.tiles_n;
    const int band = idx / per, first = band * G8;
    const int rows = tme - first < G8 ? tme - first : G8;
    const int in = idx - band * per;
    tm = first + in % rows;
    tn = in / rows;
}

// KS = 2 splits the K loop inside the workgroup: two groups of WGM x WGN
// waves each run half of the K steps through their own LDS pipeline over the
// same tile, then swap halves of their partial sums through LDS, so that
// every SIMD holds two waves (one of each group) when the tile count alone
// would leave one: one wave's dequantization then overlaps the other's MFMAs.
// Requires an even number of K steps.
//
// EPI_SILUQ (routed-expert SwiGLU front half): B holds 2H rows, gate rows
// [0, H) then up rows [H, 2H).  A tile covers BN/2 columns j of h, and each
// wave's WN columns are its WN/2 gate columns followed by the up columns of
// the same j, so the epilogue finds g and u of one output element in the
// same wave's staged rows and quantizes silu(g)*u per 16-column block, with
// the same arithmetic as the silu_and_mul quantize kernel.
//
// SK (split-tail schedule, plain and LoRA epilogues): rounds of p.sk_grid
// workgroups, one per CU, find their work from the mask (see sk_plan): a
// whole tile, or one K range of a tail tile, whose fp32 partial sums go to
// the workspace when the tile is split.
template <int BM, int BN, int WGM, int WGN, int NST, int KS, bool ALIGNED, int EPI, bool SK = false>
__global__ __launch_bounds__(64 * WGM * WGN * KS, (KS == 2 ? 2 : kWavesPerEU<BM / WGM, BN / WGN>)) void k_gemm(GParams p) {
#if defined(__HIP_DEVICE_COMPILE__)  // the host pass only needs the launch stub
    static_assert(KS == 1 || (KS == 2 && BM / WGM == 64), "the K split swaps 32-row fragment rows of 64-row wave tiles");
    static_assert(EPI != EPI_SILUQ || KS == 1, "the quantizing epilogue runs on whole-K tiles");
    constexpr bool LORA = EPI == EPI_LORA;
    constexpr int NW = WGM * WGN;  // waves of one K group, WGM along M x WGN along N
    constexpr int WM = BM / WGM, WN = BN / WGN;
    constexpr int FM = WM / 32, FN = WN / 32;
    // Scale staging.  Banded (the K-split tile, whose two K groups stage
    // their own steps): the swizzled layout keeps a 128-row band's 8 scales
    // per row of one K step (its two column groups of 4) in 1 KB of
    // contiguous memory, which one 16-byte load per lane copies as is (a
    // quarter of the load instructions of the dword path; measured 1-2%
    // faster there, 1% slower on the 256 x 256 tile, whose reads of it meet
    // two-way bank conflicts).  Otherwise: one dword per (row, column group),
    // two per row at 8t.
    constexpr bool BANDED = KS == 2 && EPI != EPI_SILUQ && BM % 128 == 0 && BN % 128 == 0;
    constexpr int NBAND = (BM + BN) / 128;
    // one LDS stage: FP4 A rows, FP4 B rows, scales (padded to whole wave
    // loads)
    constexpr int OFF_B = BM * 64, OFF_S = OFF_B + BN * 64;
    constexpr int SC_BYTES = BANDED ? NBAND * 1024 : ((BM + BN) * 2 + 64 * NW - 1) / (64 * NW) * (64 * NW) * 4;
    constexpr int STAGE = OFF_S + SC_BYTES;
    // loads per wave per step (FP4: 16 rows each; when a kind of load does
    // not divide evenly over the waves, its last round falls to the first
    // waves only, and the step waits count nothing: two stages)
    constexpr int NFA = (BM + 16 * NW - 1) / (16 * NW), NFB = (BN + 16 * NW - 1) / (16 * NW);
    constexpr int NSC = BANDED ? (NBAND + NW - 1) / NW : SC_BYTES / 4 / (64 * NW);
    constexpr bool EVEN_F = BM % (16 * NW) == 0 && BN % (16 * NW) == 0;
    constexpr bool EVEN = EVEN_F && (!BANDED || NBAND % NW == 0);
    constexpr int ND = NFA + NFB + NSC;
    static_assert(BM % 32 == 0 && BN % 32 == 0 && (EVEN || NST == 2), "whole fragments; uneven loads need two stages");
    static_assert(NST == 2 || NST == 3, "two or three LDS stages");
    __shared__ __align__(16) uint8_t smem[KS * NST * STAGE];

    const int t = threadIdx.x;
    const int lane = t & 63;
    const int wave_wg = __builtin_amdgcn_readfirstlane(t >> 6);
    const int grp = KS == 1 ? 0 : wave_wg / NW;          // K group
    const int wave = KS == 1 ? wave_wg : wave_wg % NW;   // wave within the group
    const int wm = wave % WGM, wn = wave / WGM;
    const int nkt = (int)((p.K + 127) / 128);  // K steps of a whole tile

    // One tile (expert e, tile row tm, tile column tn) over K steps
    // [ks0, ks1): stored as bf16, or with slot >= 0 left as an fp32 partial
    // tile in workspace slot `slot`.  lora: add the rank-r term (EPI_LORA).
    auto tile = [&](const int e, const int tm, const int tn, const int ks0, const int ks1, const int slot,
                    const bool lora) {
    const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN;
    const int64_t hc0 = (int64_t)tn * (BN / 2);  // first h column of the tile (EPI_SILUQ)
    const int valid = clamp_rows(p.mask, e, (int)p.M);
    if (m0 >= valid) {  // whole tile past this expert's valid rows
        if constexpr (EPI == EPI_SILUQ) {
            // its rows of the output scale buffer are zero
            constexpr int BC = BN / 32;  // 16-column blocks of the tile
            uint8_t* sf = p.q_sf + (int64_t)e * p.q_sfsz;
            for (int i = (int)threadIdx.x; i < BM * BC; i += 64 * WGM * WGN * KS) {
                const int64_t m = m0 + i / BC, c = hc0 / 16 + i % BC;
                if (m < p.q_rpad && c < 4 * (int64_t)p.q_cp4) sf[sf_offset(m, c, p.q_cp4)] = 0;
            }
        }
        return;
    }
    // B matrix row behind tile column c (0 <= c < BN): row n0 + c, or for
    // EPI_SILUQ the gate or up row of h column j (clamped rows feed outputs
    // that are never stored)
    auto b_row = [&](int c) -> int64_t {
        if constexpr (EPI == EPI_SILUQ) {
            constexpr int WNl = BN / WGN, HW = WNl / 2;
            const int cw = c % WNl;
            int64_t j = hc0 + (c / WNl) * HW + cw % HW;
            j = j < p.H ? j : p.H - 1;
            return cw < HW ? j : p.H + j;
        } else {
            return n0 + c < p.N ? n0 + c : p.N - 1;
        }
    };

    const int64_t rowb = p.K / 2;
    const __amdgpu_buffer_rsrc_t rA = make_rsrc(p.a + (int64_t)e * p.M * rowb, (uint32_t)(p.M * rowb));
    const __amdgpu_buffer_rsrc_t rB = make_rsrc(p.b + (int64_t)e * p.N * rowb, (uint32_t)(p.N * rowb));
    const __amdgpu_buffer_rsrc_t rSA = make_rsrc(p.a_sf + (int64_t)e * p.sfa, (uint32_t)p.sfa);
    const __amdgpu_buffer_rsrc_t rSB = make_rsrc(p.b_sf + (int64_t)e * p.sfb, (uint32_t)p.sfb);

    // Per-lane source offsets of this wave's staging loads (the step adds a
    // uniform 64 bytes of FP4 or 1024 bytes of scales per K step).  Lane l of
    // a 16-row FP4 load lands at byte 16*l of its 1 KB block: row l/4, slot
    // l%4, so it fetches chunk slot ^ swz(row).  Rows past the matrix read its
    // last row; they feed only outputs that are never stored.
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
        const int64_t row = b_row(r);
        voB[i] = (uint32_t)(row * rowb) + (uint32_t)((((lane & 3) ^ swz(r)) << 4));
    }
#pragma unroll
    for (int i = 0; i < NSC; i++) {
        if constexpr (BANDED) {
            // band bi: lanes 0-31 the first column group's 512 bytes, 32-63 the
            // second's (bands past the matrix's padded rows read its last band;
            // they feed only outputs that are never stored)
            const int bi = i * NW + wave;
            if (bi < BM / 128) {
                const int64_t r0 = m0 + 128 * bi < p.rpa ? m0 + 128 * bi : p.rpa - 128;
                voS[i] = (uint32_t)(((r0 >> 7) * p.cpa4) * 512) + lane * 16;
            } else {
                const int64_t r0 = n0 + 128 * (bi - BM / 128) < p.rpb ? n0 + 128 * (bi - BM / 128) : p.rpb - 128;
                voS[i] = (uint32_t)(((r0 >> 7) * p.cpa4) * 512) + lane * 16;
            }
            continue;
        }
        const int dw = (i * NW + wave) * 64 + lane;  // scale dword of the stage
        const int tr = dw >> 1, g = dw & 1;         // tile row, column group of the step
        if (tr < BM) {
            const int64_t row = m0 + tr < p.rpa ? m0 + tr : p.rpa - 1;
            voS[i] = scale_dword_off(row, g, p.cpa4);
        } else if (tr < BM + BN) {
            int64_t row;
            if constexpr (EPI == EPI_SILUQ) row = b_row(tr - BM);
            else row = n0 + (tr - BM) < p.rpb ? n0 + (tr - BM) : p.rpb - 1;
            voS[i] = scale_dword_off(row, g, p.cpa4);
        } else {
            voS[i] = 0;  // padding dwords: any in-bounds source
        }
    }
    lds_u8* const sm = (lds_u8*)smem + grp * (NST * STAGE);
    auto issue = [&](int step, lds_u8* st) {
#pragma unroll
        for (int i = 0; i < NFA; i++)
            if (EVEN_F || (i * NW + wave) * 16 < BM)  // (wave-uniform)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rA, (__attribute__((address_space(3))) void*)(st + (i * NW + wave) * 1024),
                                                         16, voA[i], step * 64, 0, 0);
#pragma unroll
        for (int i = 0; i < NFB; i++)
            if (EVEN_F || (i * NW + wave) * 16 < BN)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rB, (__attribute__((address_space(3))) void*)(st + OFF_B + (i * NW + wave) * 1024),
                                                         16, voB[i], step * 64, 0, 0);
#pragma unroll
        for (int i = 0; i < NSC; i++) {
            if constexpr (BANDED) {
                const int bi = i * NW + wave;
                if (NBAND % NW == 0 || bi < NBAND)
                    __builtin_amdgcn_raw_ptr_buffer_load_lds(bi < BM / 128 ? rSA : rSB,
                                                             (__attribute__((address_space(3))) void*)(st + OFF_S + bi * 1024),
                                                             16, voS[i], step * 1024, 0, 0);
            } else {
                const bool isA = (i * NW + wave) * 32 < BM;  // a wave load covers 32 tile rows: all A or all B
                __builtin_amdgcn_raw_ptr_buffer_load_lds(isA ? rSA : rSB,
                                                         (__attribute__((address_space(3))) void*)(st + OFF_S + (i * NW + wave) * 256),
                                                         4, voS[i], step * 1024, 0, 0);
            }
        }
    };

    f32x16 acc[FN][FM];
#pragma unroll
    for (int i = 0; i < FN; i++)
#pragma unroll
        for (int j = 0; j < FM; j++)
#pragma unroll
            for (int v = 0; v < 16; v++) acc[i][j][v] = 0.0f;

    const int kb = ks0 + grp * ((ks1 - ks0) / KS), ke = KS == 1 ? ks1 : kb + (ks1 - ks0) / KS;  // this group's K steps
    const int h = lane >> 5, l32 = lane & 31;
    // per-lane LDS offsets, fixed for the whole K loop (fragment i adds i*32 rows)
    const int ra_off = (wm * WM + l32) * 64, rb_off = OFF_B + (wn * WN + l32) * 64;
    const int xr = swz(l32);
    const int cq0 = ((h ^ xr) << 4), cq1 = (((2 + h) ^ xr) << 4);
    // this lane's first scale dword (fragment 0); banded: column group x of
    // tile row t at byte 1024 * (t >> 7) + 16 * (t & 31) + 4 * ((t >> 5) & 3)
    // of the region, y 512 bytes further
    auto band_off = [&](int f) { return OFF_S + (f >> 2) * 1024 + (f & 3) * 4 + l32 * 16; };  // fragment row f
    const int sa_off = BANDED ? 0 : OFF_S + (wm * WM + l32) * 8;
    const int sb_off = BANDED ? 0 : OFF_S + (BM + wn * WN + l32) * 8;
    const int hsh = 16 * h;  // this lane's blocks sit in the high half of each scale dword when h = 1

    // fragment registers of one half step q (lane: 32 elements = 4 dwords per
    // fragment row) and the fp16 scales of the whole K step
    u32x4 fa[FM], fb[FN];
    f16x2 sa2[FM][2], sb2[FN][2];
    // Scales of step `step` from stage st: blocks 2h, 2h+1 (q = 0) and
    // 4+2h, 5+2h (q = 1) of the step, converted to fp16 (exact).  Blocks past
    // K (only when K % 128 != 0) are zeroed: their FP4 bytes are the next
    // row's or zeros, and must not contribute.
    auto load_scales = [&](const lds_u8* st, int step) {
        u32x2 ra[FM], rb[FN];
        if constexpr (BANDED) {
#pragma unroll
            for (int i = 0; i < FM; i++) {
                const int o = band_off(wm * FM + i);
                ra[i] = u32x2{*(const __attribute__((address_space(3))) uint32_t*)(st + o),
                              *(const __attribute__((address_space(3))) uint32_t*)(st + o + 512)};
            }
#pragma unroll
            for (int i = 0; i < FN; i++) {
                const int o = band_off(BM / 32 + wn * FN + i);
                rb[i] = u32x2{*(const __attribute__((address_space(3))) uint32_t*)(st + o),
                              *(const __attribute__((address_space(3))) uint32_t*)(st + o + 512)};
            }
        } else {
#pragma unroll
            for (int i = 0; i < FM; i++) ra[i] = *(const __attribute__((address_space(3))) u32x2*)(st + sa_off + i * 256);
#pragma unroll
            for (int i = 0; i < FN; i++) rb[i] = *(const __attribute__((address_space(3))) u32x2*)(st + sb_off + i * 256);
        }
        uint32_t m0w = 0xFFFFFFFFu, m1w = 0xFFFFFFFFu;
        if constexpr (!ALIGNED) {
            const int left = p.nblk - step * 8;  // valid blocks in this step (<= 0 past the end)
            const int l0 = left < 0 ? 0 : left > 4 ? 4 : left, l1 = left < 4 ? 0 : left > 8 ? 4 : left - 4;
            m0w = (uint32_t)(((uint64_t)1 << (8 * l0)) - 1);
            m1w = (uint32_t)(((uint64_t)1 << (8 * l1)) - 1);
        }
#pragma unroll
        for (int i = 0; i < FM; i++) {
            sa2[i][0] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((ra[i].x & m0w) >> hsh, 1.0f, false);
            sa2[i][1] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((ra[i].y & m1w) >> hsh, 1.0f, false);
        }
#pragma unroll
        for (int i = 0; i < FN; i++) {
            sb2[i][0] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((rb[i].x & m0w) >> hsh, 1.0f, false);
            sb2[i][1] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((rb[i].y & m1w) >> hsh, 1.0f, false);
        }
    };
    auto load_half = [&](const lds_u8* st, int cq) {
#pragma unroll
        for (int i = 0; i < FM; i++) fa[i] = *(const __attribute__((address_space(3))) u32x4*)(st + ra_off + i * 2048 + cq);
#pragma unroll
        for (int i = 0; i < FN; i++) fb[i] = *(const __attribute__((address_space(3))) u32x4*)(st + rb_off + i * 2048 + cq);
    };
    // K slice s = 4q + j of the current step, dequantized into buffer s & 1
    f16x8 oa[2][FM], ob[2][FN];
    auto dequant_slice = [&](int s) {
        const int q = s >> 2, j = s & 3;
#pragma unroll
        for (int i = 0; i < FM; i++) oa[s & 1][i] = dequant8(word(fa[i], j), sa2[i][q][j >> 1]);
#pragma unroll
        for (int i = 0; i < FN; i++) ob[s & 1][i] = dequant8(word(fb[i], j), sb2[i][q][j >> 1]);
    };
    auto mfma_slice = [&](int s) {
#pragma unroll
        for (int in = 0; in < FN; in++)
#pragma unroll
            for (int im = 0; im < FM; im++)
                acc[in][im] = __builtin_amdgcn_mfma_f32_32x32x16_f16(ob[s & 1][in], oa[s & 1][im], acc[in][im],
                                                                     0, 0, 0);
    };
    // one MFMA, then its share of the dequantization VALU work, repeated
    constexpr int VPM = (8 * (FM + FN) + FM * FN - 1) / (FM * FN);
    constexpr int kLead = FM * FN >= 8 ? 4 : 1;  // MFMAs issued while a step's first LDS reads land
    constexpr int VPT = (8 * (FM + FN) + 4 * (FM + FN) + (FM * FN - kLead) - 1) /
                        (FM * FN - kLead > 0 ? FM * FN - kLead : 1);
    auto interleave = [&]() {
#pragma unroll
        for (int k = 0; k < FM * FN; k++) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x002, VPM, 0);
        }
    };
    // Workgroup barrier of the LDS pipeline: the waits that matter are
    // explicit (this wave's loads into the next stage, its LDS reads), and the
    // "memory" clobber keeps the compiler from moving LDS accesses across it.
    auto barrier = [&]() {
        __builtin_amdgcn_s_waitcnt((0x3F & 0xF) | (0x3 << 14) | (0x7 << 4) | (0x0 << 8));  // lgkmcnt(0)
        asm volatile("s_barrier" ::: "memory");
    };

    // Step kt lives in stage (kt - kb) % NST; its loads are issued NST-1 steps
    // ahead.  Both K groups run the same number of steps, so the workgroup
    // barriers pair up.
    issue(kb, sm);
    if constexpr (NST == 3) issue(kb + 1 < ke ? kb + 1 : kb, sm + STAGE);
    wait_vmcnt<ND * (NST - 2)>();  // step kb has landed (this wave's part)
    barrier();
    load_scales(sm, kb);
    load_half(sm, cq0);
    dequant_slice(0);

    int sc = 0;  // stage of step kt
    for (int kt = kb; kt < ke; kt++) {
        const int s1 = sc == NST - 1 ? 0 : sc + 1;
        const int sl = NST == 2 ? s1 : (s1 == 2 ? 0 : s1 + 1);  // stage of step kt+NST-1
        const lds_u8* cur = sm + sc * STAGE;
        // step kt+NST-1 into the stage that step kt-1 used (the last steps
        // reload the final K step into a stage nobody reads again, keeping the
        // loop branch-free)
        issue(kt + NST - 1 < ke ? kt + NST - 1 : ke - 1, sm + sl * STAGE);
#pragma unroll
        for (int s = 0; s < 7; s++) {
            dequant_slice(s + 1);
            if (s == 2) load_half(cur, cq1);  // the q = 0 words are dead after slice 3
            mfma_slice(s);
            interleave();
            if (s == 2) __builtin_amdgcn_sched_group_barrier(0x100, FM + FN, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
        wait_vmcnt<ND * (NST - 2)>();  // step kt+1 has landed; later steps may be in flight
        barrier();
        __builtin_amdgcn_sched_barrier(0);
        const lds_u8* nx = sm + s1 * STAGE;
        load_scales(nx, kt + 1);
        load_half(nx, cq0);
        dequant_slice(0);  // buffer 0: slice 7 lives in buffer 1
        mfma_slice(7);
        // LDS reads first, a few MFMAs while they are in flight, then the
        // scale conversion and slice-0 dequantization of step kt+1
        __builtin_amdgcn_sched_group_barrier(0x100, 2 * (FM + FN), 0);
        __builtin_amdgcn_sched_group_barrier(0x008, kLead, 0);
#pragma unroll
        for (int k = kLead; k < FM * FN; k++) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x002, VPT, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
        sc = s1;
    }
    wait_vmcnt<0>();  // nothing may land in LDS after the workgroup ends

    if constexpr (KS == 2) {
        // Group g keeps fragment row im = g of its wave tile and takes the
        // other group's partial sums of it: each wave writes the fragments it
        // gives away to its partner's LDS slot, then adds what its partner
        // wrote (FN / 2 fragment columns per round, so a round fits in the
        // pipeline's LDS).
        constexpr int FRAG = 64 * 16 * 4;  // one fragment of one wave, bytes
        constexpr int HALF = FN / 2;
        static_assert(FM == 2 && FN % 2 == 0 && NW * HALF * 2 * FRAG <= KS * NST * STAGE, "swap rounds fit in LDS");
        lds_u8* const xb = (lds_u8*)smem;
#pragma unroll
        for (int rd = 0; rd < 2; rd++) {
            barrier();  // every wave is done with the LDS it is about to overwrite
#pragma unroll
            for (int i = 0; i < HALF; i++) {
                const int in = rd * HALF + i;
                // slot (wave, i, destination group)
                lds_u8* dst = xb + ((wave * HALF + i) * 2 + (1 - grp)) * FRAG;
                auto put = [&](const f32x16& a) {
#pragma unroll
                    for (int g4 = 0; g4 < 4; g4++)
                        *(__attribute__((address_space(3))) f32x4*)(dst + (g4 * 64 + lane) * 16) =
                            f32x4{a[4 * g4], a[4 * g4 + 1], a[4 * g4 + 2], a[4 * g4 + 3]};
                };
                if (grp == 0) put(acc[in][1]);
                else put(acc[in][0]);
            }
            barrier();
#pragma unroll
            for (int i = 0; i < HALF; i++) {
                const int in = rd * HALF + i;
                const lds_u8* src = xb + ((wave * HALF + i) * 2 + grp) * FRAG;
                auto take = [&](f32x16& a) {
#pragma unroll
                    for (int g4 = 0; g4 < 4; g4++) {
                        const f32x4 v = *(const __attribute__((address_space(3))) f32x4*)(src + (g4 * 64 + lane) * 16);
#pragma unroll
                        for (int u = 0; u < 4; u++) a[4 * g4 + u] += v[u];
                    }
                };
                if (grp == 0) take(acc[in][0]);
                else take(acc[in][1]);
            }
        }
    }

    if (LORA && lora) {
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
                    if (KS == 1 || im == grp)
                    acc[in][im] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ol[in], od[im], acc[in][im], 0, 0, 0);
        }
    }

    if (SK && slot >= 0) {
        // fp32 partial tile, fragment-major: the v-th 4 floats of every lane
        // of fragment f (32-row block f / (BN/32), 32-column block f % (BN/32))
        // form one contiguous 1 KB piece at float offset (4f + v) * 256
        float* const P = p.part + (int64_t)slot * (BM * BN);
#pragma unroll
        for (int im = 0; im < FM; im++) {
            if (KS == 2 && im != grp) continue;  // the other K group holds this fragment row
#pragma unroll
            for (int in = 0; in < FN; in++) {
                const int f = (wm * FM + im) * (BN / 32) + wn * FN + in;
#pragma unroll
                for (int v = 0; v < 4; v++)
                    *(f32x4*)(P + ((f * 4 + v) * 64 + lane) * 4) =
                        f32x4{acc[in][im][4 * v], acc[in][im][4 * v + 1], acc[in][im][4 * v + 2], acc[in][im][4 * v + 3]};
            }
        }
        return;
    }

    // ---- epilogue: alpha, bias, bf16; staged through LDS (each wave its own
    // region, one 32-row fragment row at a time) so that every output row
    // leaves as whole 16-byte pieces covering the wave's WN columns, rows
    // >= valid skipped.  The pipeline stages are free once every wave is past
    // its last LDS read.
    constexpr int PITCH = WN * 2 + 16;  // bytes per staged row (16-byte aligned, banks spread)
    static_assert(NW * 32 * PITCH <= NST * STAGE, "epilogue staging fits in the pipeline's LDS");
    barrier();
    lds_u8* const ep = sm + wave * 32 * PITCH;
    const float alpha = p.alpha[e];
    uint16_t* O = p.out + (int64_t)e * p.M * p.N;
    constexpr int CPR = WN / 8;        // 16-byte pieces per staged row
    // the bias of this lane's columns (4 consecutive per fragment column and
    // group: one 8-byte load each, all in flight together; 0 past N)
    u32x2 bias_v[FN][4];
    if (EPI != EPI_SILUQ && p.bias) {
#pragma unroll
        for (int in = 0; in < FN; in++)
#pragma unroll
            for (int g = 0; g < 4; g++) {
                const int64_t n = n0 + wn * WN + in * 32 + g * 8 + h * 4;
                if ((p.N & 3) == 0 && n + 3 < p.N) {
                    bias_v[in][g] = *(const u32x2*)(p.bias + n);
                } else {
                    uint32_t b[4];
#pragma unroll
                    for (int u = 0; u < 4; u++) b[u] = n + u < p.N ? (uint32_t)p.bias[n + u] : 0u;
                    bias_v[in][g] = u32x2{b[0] | (b[1] << 16), b[2] | (b[3] << 16)};
                }
            }
    }
#pragma unroll
    for (int im = 0; im < FM; im++) {
        if (KS == 2 && im != grp) continue;  // the other K group stores this fragment row
        // lane (l32, h) of fragment in: row l32, columns in*32 + 8g + 4h .. +3
#pragma unroll
        for (int in = 0; in < FN; in++) {
#pragma unroll
            for (int g = 0; g < 4; g++) {
                const int cl = in * 32 + g * 8 + h * 4;  // column within the wave tile
                float y[4];
#pragma unroll
                for (int u = 0; u < 4; u++) {
                    y[u] = alpha * acc[in][im][g * 4 + u];
                    if (EPI != EPI_SILUQ && p.bias) {
                        const uint32_t bw = u < 2 ? bias_v[in][g].x : bias_v[in][g].y;
                        y[u] += (u & 1) ? bf16_hi(bw) : bf16_lo(bw);
                    }
                }
                *(__attribute__((address_space(3))) u32x2*)(ep + l32 * PITCH + cl * 2) =
                    u32x2{pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3])};
            }
        }
        __builtin_amdgcn_s_waitcnt((0x3F & 0xF) | (0x3 << 14) | (0x7 << 4) | (0x0 << 8));  // lgkmcnt(0)
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (EPI == EPI_SILUQ) {
            // 32 staged rows x NBW blocks of 16 h columns; lane -> (row, block)
            constexpr int NBW = WN / 32;
            const float gs = p.q_gs[e];
            uint8_t* const Q = p.q_fp4 + (int64_t)e * p.M * (p.H / 2);
            uint8_t* const SF = p.q_sf + (int64_t)e * p.q_sfsz;
#pragma unroll
            for (int it = 0; it < 32 * NBW / 64; it++) {
                const int bi = it * 64 + lane, rl = bi / NBW, bc = bi % NBW;
                const lds_u8* rowp = ep + rl * PITCH;
                u32x4 r[4];
                r[0] = *(const __attribute__((address_space(3))) u32x4*)(rowp + bc * 32);
                r[1] = *(const __attribute__((address_space(3))) u32x4*)(rowp + bc * 32 + 16);
                r[2] = *(const __attribute__((address_space(3))) u32x4*)(rowp + WN + bc * 32);
                r[3] = *(const __attribute__((address_space(3))) u32x4*)(rowp + WN + bc * 32 + 16);
                const int64_t m = m0 + wm * WM + im * 32 + rl;
                const int64_t hc = hc0 + wn * (WN / 2) + bc * 16;
                const bool active = m < valid && hc < p.H;
                // rows past the valid ones hold whatever A's padding rows gave
                // (often zeros, which the silu fast path sends to the exact
                // path): skip their arithmetic
                float f[16];
                float bamax = 0.0f;
                if (active) {
                    const u32x4 pq[2] = {u32x4{0u, 0u, 0u, 0u}, u32x4{0u, 0u, 0u, 0u}};
                    bamax = process_block<V_SILU>(r, pq, f);
                } else {
#pragma unroll
                    for (int j = 0; j < 16; j++) f[j] = 0.0f;
                }
                const uint32_t sc = active ? ue4m3_encode(div6(bamax) * gs) : 0u;
                const float dec = ue4m3_decode(sc);
                const float rr = dec == 0.0f ? 0.0f : gs / dec;
                uint32_t w0, w1;
                pack_block(f, rr, w0, w1);
                if (active) *(u32x2*)(Q + m * (p.H / 2) + hc / 2) = u32x2{w0, w1};
                if (m < p.q_rpad && hc / 16 < 4 * (int64_t)p.q_cp4) SF[sf_offset(m, hc / 16, p.q_cp4)] = (uint8_t)sc;
            }
        } else {
        // 32 staged rows x CPR pieces, 64 pieces per wave store instruction
#pragma unroll
        for (int it = 0; it < (32 * CPR + 63) / 64; it++) {
            const int pc = it * 64 + lane;
            if ((32 * CPR) % 64 != 0 && pc >= 32 * CPR) break;
            const int rl = pc / CPR, c = pc % CPR;
            const u32x4 v = *(const __attribute__((address_space(3))) u32x4*)(ep + rl * PITCH + c * 16);
            const int64_t m = m0 + wm * WM + im * 32 + rl;
            const int64_t n = n0 + wn * WN + c * 8;
            if (m >= valid) continue;
            if (n + 8 <= p.N && (p.N & 7) == 0) {
                *(u32x4*)(O + m * p.N + n) = v;
            } else {
#pragma unroll
                for (int u = 0; u < 8; u++)
                    if (n + u < p.N) O[m * p.N + n + u] = (uint16_t)(v[u >> 1] >> (16 * (u & 1)));
            }
        }
        }
        __builtin_amdgcn_s_waitcnt((0x3F & 0xF) | (0x3 << 14) | (0x7 << 4) | (0x0 << 8));  // reads done before the region is rewritten
        __builtin_amdgcn_sched_barrier(0);
    }
    };  // tile

    if constexpr (!SK) {
        int tm, tn;
        tile_coords(p, tm, tn);
        tile(blockIdx.z, tm, tn, 0, nkt, -1, true);
    } else {
        // workgroup w: round w / G, position b = w % G within the round (the
        // grid holds enough rounds for every live tile; workgroups past the
        // schedule exit at once)
        static_assert(EPI != EPI_SILUQ, "the split schedule stores plain or LoRA tiles");
        const int G = p.sk_grid, w = blockIdx.x, round = w / G, b = w % G;
        const int tme_lane = sk_lane_rows(p, BM);
        const SkPlan pl = sk_plan(p, tme_lane, nkt, KS);
        const int rounds = pl.D / G;
        int idx, ks0 = 0, ks1 = nkt, slot = -1, lora = 1;
        if (round < rounds) {
            idx = round * G + ((G & 7) == 0 ? (b & 7) * (G >> 3) + (b >> 3) : b);
        } else if (round == rounds && b < pl.R * pl.S) {
            const int r = b / pl.S, j = b % pl.S, np = nkt / KS;
            idx = pl.D + r;
            ks0 = KS * (j * np / pl.S);
            ks1 = KS * ((j + 1) * np / pl.S);
            if (pl.S > 1) {
                slot = b;
                lora = j == 0;
            }
        } else {
            return;
        }
        int e, tm, tn;
        sk_tile(p, tme_lane, idx, e, tm, tn);
        tile(__builtin_amdgcn_readfirstlane(e), __builtin_amdgcn_readfirstlane(tm),
             __builtin_amdgcn_readfirstlane(tn), __builtin_amdgcn_readfirstlane(ks0),
             __builtin_amdgcn_readfirstlane(ks1), __builtin_amdgcn_readfirstlane(slot),
             __builtin_amdgcn_readfirstlane(lora) != 0);
    }
#endif
}

// Second launch of a split-tail schedule: adds the S fp32 partial tiles of
// each tail tile r in part order (slots r*S .. r*S+S-1), applies alpha and
// bias and stores bf16, rows >= mask[e] untouched.  One item is 4 outputs
// (one float4 of every partial); a grid of one 1024-thread workgroup per CU
// walks the R * BM*BN/4 items, 1024 consecutive items (one tile) per
// workgroup and step, the loads of up to 8 parts of an item in flight
// together.  Exits at once when nothing was split.
constexpr int kFixupThreads = 1024;

template <int BM, int BN, int KS>
__global__ __launch_bounds__(kFixupThreads) void k_gemm_fixup(GParams p) {
    constexpr int ITEMS = BM * BN / 4;  // float4 items of one partial tile
    static_assert(ITEMS % kFixupThreads == 0, "a workgroup's items lie in one tile");
    const int nkt = (int)((p.K + 127) / 128);
    const int tme_lane = sk_lane_rows(p, BM);
    const SkPlan pl = sk_plan(p, tme_lane, nkt, KS);
    if (pl.S <= 1) return;
    const int total = pl.R * ITEMS;
    for (int g0 = blockIdx.x * kFixupThreads; g0 < total; g0 += gridDim.x * kFixupThreads) {
        const int r = g0 / ITEMS, i = g0 % ITEMS + (int)threadIdx.x;
        int e, tm, tn;
        sk_tile(p, tme_lane, pl.D + r, e, tm, tn);
        const int valid = clamp_rows(p.mask, e, (int)p.M);
        const int lane = i & 63, v = (i >> 6) & 3, f = i >> 8;
        const int64_t m = (int64_t)tm * BM + (f / (BN / 32)) * 32 + (lane & 31);
        const int64_t n = (int64_t)tn * BN + (f % (BN / 32)) * 32 + v * 8 + (lane >> 5) * 4;
        if (m >= valid) continue;
        const float* const P = p.part + (int64_t)r * pl.S * (BM * BN) + (int64_t)i * 4;
        f32x4 s = *(const f32x4*)P;
        for (int j0 = 1; j0 < pl.S; j0 += 8) {
            f32x4 t[8];
#pragma unroll
            for (int u = 0; u < 8; u++)
                if (j0 + u < pl.S) t[u] = *(const f32x4*)(P + (int64_t)(j0 + u) * (BM * BN));
#pragma unroll
            for (int u = 0; u < 8; u++)
                if (j0 + u < pl.S) s += t[u];
        }
        const float alpha = p.alpha[e];
        uint16_t* const O = p.out + (int64_t)e * p.M * p.N;
        float y[4];
#pragma unroll
        for (int u = 0; u < 4; u++) {
            y[u] = alpha * s[u];
            if (p.bias && n + u < p.N) y[u] += bf16_lo((uint32_t)p.bias[n + u]);
        }
        if ((p.N & 3) == 0 && n + 3 < p.N) {
            *(u32x2*)(O + m * p.N + n) = u32x2{pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3])};
        } else {
#pragma unroll
            for (int u = 0; u < 4; u++)
                if (n + u < p.N) O[m * p.N + n + u] = (uint16_t)pack_bf16x2(y[u], 0.0f);
        }
    }
}

template <int BM, int BN, int WGM, int WGN, int NST, int KS = 1>
static hipError_t launch_tile(GParams p, bool lora, hipStream_t st) {
    p.tiles_m = (int)((p.M + BM - 1) / BM);
    p.tiles_n = (int)((p.N + BN - 1) / BN);
    const int tiles = p.tiles_m * p.tiles_n;
    p.xcd_chunk = tiles % 8 == 0 ? tiles / 8 : 0;
    dim3 grid(tiles, 1, (unsigned)p.E ? (unsigned)p.E : 1u);
    constexpr int threads = 64 * WGM * WGN * KS;
    const bool aligned = (p.K % 128) == 0;
    if (lora) {
        if (aligned) k_gemm<BM, BN, WGM, WGN, NST, KS, true, EPI_LORA><<<grid, threads, 0, st>>>(p);
        else k_gemm<BM, BN, WGM, WGN, NST, KS, false, EPI_LORA><<<grid, threads, 0, st>>>(p);
    } else {
        if (aligned) k_gemm<BM, BN, WGM, WGN, NST, KS, true, EPI_PLAIN><<<grid, threads, 0, st>>>(p);
        else k_gemm<BM, BN, WGM, WGN, NST, KS, false, EPI_PLAIN><<<grid, threads, 0, st>>>(p);
    }
    return hipGetLastError();
}

// Split-tail launch (see sk_plan) and, with a workspace, the launch that
// adds the split tiles' partial sums.
template <int BM, int BN, int WGM, int WGN, int NST, int KS>
static hipError_t launch_tile_sk(GParams p, bool lora, float* ws, int G, hipStream_t st) {
    p.tiles_m = (int)((p.M + BM - 1) / BM);
    p.tiles_n = (int)((p.N + BN - 1) / BN);
    p.xcd_chunk = 0;
    p.part = ws;
    p.sk_grid = G;
    constexpr int threads = 64 * WGM * WGN * KS;
    const bool aligned = (p.K % 128) == 0;
    // rounds for every tile of every expert, plus the tail round
    const int64_t tmax = p.E * p.tiles_m * p.tiles_n;
    const dim3 grid((unsigned)(G * (tmax / G + 1)), 1, 1);
    if (lora) {
        if (aligned) k_gemm<BM, BN, WGM, WGN, NST, KS, true, EPI_LORA, true><<<grid, threads, 0, st>>>(p);
        else k_gemm<BM, BN, WGM, WGN, NST, KS, false, EPI_LORA, true><<<grid, threads, 0, st>>>(p);
    } else {
        if (aligned) k_gemm<BM, BN, WGM, WGN, NST, KS, true, EPI_PLAIN, true><<<grid, threads, 0, st>>>(p);
        else k_gemm<BM, BN, WGM, WGN, NST, KS, false, EPI_PLAIN, true><<<grid, threads, 0, st>>>(p);
    }
    if (ws) k_gemm_fixup<BM, BN, KS><<<dim3((unsigned)G), kFixupThreads, 0, st>>>(p);
    return hipGetLastError();
}

// Quantizing epilogue: a tile covers BN/2 columns of h (its gate and up
// columns), so the tile grid runs over H.
template <int BM, int BN, int WGM, int WGN, int NST>
static hipError_t launch_tile_siluq(GParams p, hipStream_t st) {
    p.tiles_m = (int)((p.M + BM - 1) / BM);
    p.tiles_n = (int)((p.H + BN / 2 - 1) / (BN / 2));
    const int tiles = p.tiles_m * p.tiles_n;
    p.xcd_chunk = tiles % 8 == 0 ? tiles / 8 : 0;
    dim3 grid(tiles, 1, (unsigned)p.E);
    constexpr int threads = 64 * WGM * WGN;
    if (p.K % 128 == 0) k_gemm<BM, BN, WGM, WGN, NST, 1, true, EPI_SILUQ><<<grid, threads, 0, st>>>(p);
    else k_gemm<BM, BN, WGM, WGN, NST, 1, false, EPI_SILUQ><<<grid, threads, 0, st>>>(p);
    return hipGetLastError();
}


// ---------------------------------------------------------------------------
// Skinny GEMM for small M (decode-shaped: M <= 64).  A workgroup computes a
// 16 x 16 output tile; its kSkinnyWaves waves split K into contiguous ranges and
// their fp32 partial tiles are summed through LDS.  Each lane loads its
// operand fragments straight from global memory (no reuse to stage for):
// lane (row r = l%16, group g = l/16) holds, per 128-element K chunk, the 32
// consecutive elements 32g.. of its A row and of its B row plus their two
// block scales, and feeds four v_mfma_f32_16x16x32_f16 K-slices from them
// (the same K permutation on both operands).  With N/16 x M/16 workgroups the
// weight is streamed once, spread over every CU.
// ---------------------------------------------------------------------------
constexpr int kSkinnyWaves = 8;  // K ranges of a workgroup (two waves per SIMD)

template <bool ALIGNED, bool LORA>
__global__ __launch_bounds__(64 * kSkinnyWaves) void k_gemm_skinny(GParams p) {
#if defined(__HIP_DEVICE_COMPILE__)  // the host pass only needs the launch stub
    const int t = threadIdx.x, lane = t & 63;
    const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
    const int e = blockIdx.z;
    const int64_t n0 = (int64_t)blockIdx.x * 16, m0 = (int64_t)blockIdx.y * 16;
    const int valid = clamp_rows(p.mask, e, (int)p.M);
    if (m0 >= valid) return;
    const int64_t rowb = p.K / 2;
    const int r = lane & 15, g = lane >> 4;
    const int64_t arow = m0 + r < p.M ? m0 + r : p.M - 1;
    const int64_t brow = n0 + r < p.N ? n0 + r : p.N - 1;
    const uint8_t* A = p.a + (int64_t)e * p.M * rowb + arow * rowb;
    const uint8_t* B = p.b + (int64_t)e * p.N * rowb + brow * rowb;
    const uint8_t* SA = p.a_sf + (int64_t)e * p.sfa;
    const uint8_t* SB = p.b_sf + (int64_t)e * p.sfb;

    const int nch = (int)((p.K + 127) / 128);
    const int per = (nch + kSkinnyWaves - 1) / kSkinnyWaves;
    const int c0 = wave * per, c1 = c0 + per < nch ? c0 + per : nch;
    f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
    constexpr int U = 4;  // chunks whose loads are in flight together
    for (int cb = c0; cb < c1; cb += U) {
        u32x4 fa[U], fb[U];
        uint32_t sa[U], sb[U];
#pragma unroll
        for (int u = 0; u < U; u++) {
            const int c = cb + u < c1 ? cb + u : c1 - 1;  // past the range: reload, never used
            const int64_t kb = (int64_t)c * 64 + g * 16;   // byte of this lane's 32 elements
            const int blk = c * 8 + 2 * g;                 // first of its two blocks
            if (ALIGNED) {
                fa[u] = *(const u32x4*)(A + kb);
                fb[u] = *(const u32x4*)(B + kb);
            } else {
                // 32, 16 or no valid elements in the group; the rest is zero
                const int64_t left = rowb - kb;
                const u32x2 za = left >= 8 ? *(const u32x2*)(A + kb) : u32x2{0u, 0u};
                const u32x2 zb = left >= 8 ? *(const u32x2*)(B + kb) : u32x2{0u, 0u};
                const u32x2 ya = left >= 16 ? *(const u32x2*)(A + kb + 8) : u32x2{0u, 0u};
                const u32x2 yb = left >= 16 ? *(const u32x2*)(B + kb + 8) : u32x2{0u, 0u};
                fa[u] = u32x4{za.x, za.y, ya.x, ya.y};
                fb[u] = u32x4{zb.x, zb.y, yb.x, yb.y};
            }
            const int bc = blk < p.nblk ? blk : 0;  // past K: any valid (even) block column, masked below
            uint32_t va = *(const uint16_t*)(SA + scale_byte_off(arow, bc, p.cpa4));
            uint32_t vb = *(const uint16_t*)(SB + scale_byte_off(brow, bc, p.cpa4));
            if (!ALIGNED) {  // blocks past K carry zero scales
                const uint32_t keep = blk + 1 < p.nblk ? 0xFFFFu : blk < p.nblk ? 0x00FFu : 0u;
                va &= keep;
                vb &= keep;
            }
            sa[u] = va;
            sb[u] = vb;
        }
#pragma unroll
        for (int u = 0; u < U; u++) {
            if (cb + u >= c1) break;
            const f16x2 ssa = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(sa[u], 1.0f, false);
            const f16x2 ssb = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(sb[u], 1.0f, false);
#pragma unroll
            for (int j = 0; j < 4; j++) {
                const f16x8 oa = dequant8(word(fa[u], j), ssa[j >> 1]);
                const f16x8 ob = dequant8(word(fb[u], j), ssb[j >> 1]);
                acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(ob, oa, acc, 0, 0, 0);
            }
        }
    }
    if constexpr (LORA) {
        if (wave == 0) {  // rank-r bf16 correction, once, into wave 0's partial
            const int64_t drow = arow, lrow = brow;
            for (int kr = 0; kr < p.r; kr += 32) {
                const bf16x8 od = __builtin_bit_cast(bf16x8, *(const u32x4*)(p.d + drow * p.r + kr + g * 8));
                const bf16x8 ol = __builtin_bit_cast(bf16x8, *(const u32x4*)(p.l1 + lrow * p.r + kr + g * 8));
                acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ol, od, acc, 0, 0, 0);
            }
        }
    }
    // sum the waves' partial tiles (in wave order)
    __shared__ f32x4 part[kSkinnyWaves - 1][64];
    if (wave > 0) part[wave - 1][lane] = acc;
    __syncthreads();
    if (wave != 0) return;
#pragma unroll
    for (int w = 0; w < kSkinnyWaves - 1; w++) acc += part[w][lane];
    // lane: output row m0 + r, columns n0 + 4g .. n0 + 4g + 3
    const int64_t m = m0 + r;
    if (m >= valid) return;
    const float alpha = p.alpha[e];
    uint16_t* O = p.out + (int64_t)e * p.M * p.N + m * p.N;
    const int64_t n = n0 + 4 * g;
    float y[4];
#pragma unroll
    for (int v = 0; v < 4; v++) {
        y[v] = alpha * acc[v];
        if (p.bias && n + v < p.N) y[v] += bf16_lo((uint32_t)p.bias[n + v]);
    }
    if ((p.N & 3) == 0 && n + 3 < p.N) {
        uint2 o;
        o.x = pack_bf16x2(y[0], y[1]);
        o.y = pack_bf16x2(y[2], y[3]);
        *(uint2*)(O + n) = o;
    } else {
#pragma unroll
        for (int v = 0; v < 4; v++)
            if (n + v < p.N) O[n + v] = (uint16_t)pack_bf16x2(y[v], 0.0f);
    }
#endif
}

// ---------------------------------------------------------------------------
// Weight-only GEMM (nvFuser page: f16a_nvfp4weight_scaled_mm, the bf16
// activation against the dequantized NVFP4 weight): out = bf16(alpha *
// (A @ Bdq^T) (+ bias)) with A bf16 [M, K] and alpha = 1 / the weight's
// global scale.  Built for decode, where the weight read bounds the time:
// the skinny kernel's layout (a 16 x 16 output tile per workgroup, the K
// loop split over its waves, partial tiles added through LDS, 16-byte
// weight loads covering 32 elements of a row per lane), with the weight
// dequantized exactly to bf16 (e2m1 times the block scale has at most 6
// significant bits) for v_mfma_f32_16x16x32_bf16.  The activation needs no
// conversion.  Any M works (grid y = M / 16); large M is better served by
// quantizing the activation and using the NVFP4 x NVFP4 kernels.
// ---------------------------------------------------------------------------

// 8 FP4 codes of one dword times one block scale -> 8 bf16 (exact).
__device__ __forceinline__ bf16x8 dequant8_bf16(uint32_t w, float s) {
    typedef float f32x2 __attribute__((ext_vector_type(2)));
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    const f32x2 v0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 0);
    const f32x2 v1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 1);
    const f32x2 v2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 2);
    const f32x2 v3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 3);
    const bf16x2 h0 = __builtin_convertvector(f32x2{v0[0] * s, v0[1] * s}, bf16x2);
    const bf16x2 h1 = __builtin_convertvector(f32x2{v1[0] * s, v1[1] * s}, bf16x2);
    const bf16x2 h2 = __builtin_convertvector(f32x2{v2[0] * s, v2[1] * s}, bf16x2);
    const bf16x2 h3 = __builtin_convertvector(f32x2{v3[0] * s, v3[1] * s}, bf16x2);
    return bf16x8{h0[0], h0[1], h1[0], h1[1], h2[0], h2[1], h3[0], h3[1]};
}

template <bool ALIGNED>
__global__ __launch_bounds__(64 * kSkinnyWaves) void k_gemm_w4a16(GParams p) {
#if defined(__HIP_DEVICE_COMPILE__)  // the host pass only needs the launch stub
    const int t = threadIdx.x, lane = t & 63;
    const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
    const int64_t n0 = (int64_t)blockIdx.x * 16, m0 = (int64_t)blockIdx.y * 16;
    const int64_t rowb = p.K / 2;
    const int r = lane & 15, g = lane >> 4;
    const int64_t arow = m0 + r < p.M ? m0 + r : p.M - 1;
    const int64_t brow = n0 + r < p.N ? n0 + r : p.N - 1;
    const uint16_t* A = (const uint16_t*)p.a + arow * p.K;
    const uint8_t* B = p.b + brow * rowb;

    const int nch = (int)((p.K + 127) / 128);
    const int per = (nch + kSkinnyWaves - 1) / kSkinnyWaves;
    const int c0 = wave * per, c1 = c0 + per < nch ? c0 + per : nch;
    f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
    constexpr int U = 4;  // chunks whose loads are in flight together
    for (int cb = c0; cb < c1; cb += U) {
        u32x4 fa[U][4], fb[U];
        uint32_t sb[U];
#pragma unroll
        for (int u = 0; u < U; u++) {
            const int c = cb + u < c1 ? cb + u : c1 - 1;  // past the range: reload, never used
            const int64_t ke = (int64_t)c * 128 + g * 32;  // first of this lane's 32 elements
            const int blk = c * 8 + 2 * g;                 // first of its two blocks
            if (ALIGNED) {
#pragma unroll
                for (int j = 0; j < 4; j++) fa[u][j] = *(const u32x4*)(A + ke + 8 * j);
                fb[u] = *(const u32x4*)(B + ke / 2);
            } else {
                // 32, 16 or no valid elements in the group; the rest is zero
                const int64_t left = p.K - ke;
#pragma unroll
                for (int j = 0; j < 4; j++)
                    fa[u][j] = left >= 8 * (j + 1) ? *(const u32x4*)(A + ke + 8 * j) : u32x4{0u, 0u, 0u, 0u};
                const u32x2 zb = left >= 16 ? *(const u32x2*)(B + ke / 2) : u32x2{0u, 0u};
                const u32x2 yb = left >= 32 ? *(const u32x2*)(B + ke / 2 + 8) : u32x2{0u, 0u};
                fb[u] = u32x4{zb.x, zb.y, yb.x, yb.y};
            }
            const int bc = blk < p.nblk ? blk : 0;  // past K: any valid (even) block column, masked below
            uint32_t vb = *(const uint16_t*)(p.b_sf + scale_byte_off(brow, bc, p.cpa4));
            if (!ALIGNED) vb &= blk + 1 < p.nblk ? 0xFFFFu : blk < p.nblk ? 0x00FFu : 0u;
            sb[u] = vb;
        }
#pragma unroll
        for (int u = 0; u < U; u++) {
            if (cb + u >= c1) break;
            const float s0 = __builtin_amdgcn_cvt_f32_fp8(sb[u], 0), s1 = __builtin_amdgcn_cvt_f32_fp8(sb[u], 1);
#pragma unroll
            for (int j = 0; j < 4; j++) {
                const bf16x8 ob = dequant8_bf16(word(fb[u], j), j < 2 ? s0 : s1);
                const bf16x8 oa = __builtin_bit_cast(bf16x8, fa[u][j]);
                acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ob, oa, acc, 0, 0, 0);
            }
        }
    }
    // sum the waves' partial tiles (in wave order)
    __shared__ f32x4 part[kSkinnyWaves - 1][64];
    if (wave > 0) part[wave - 1][lane] = acc;
    __syncthreads();
    if (wave != 0) return;
#pragma unroll
    for (int w = 0; w < kSkinnyWaves - 1; w++) acc += part[w][lane];
    // lane: output row m0 + r, columns n0 + 4g .. n0 + 4g + 3
    const int64_t m = m0 + r;
    if (m >= p.M) return;
    const float alpha = p.alpha[0];
    uint16_t* O = p.out + m * p.N;
    const int64_t n = n0 + 4 * g;
    float y[4];
#pragma unroll
    for (int v = 0; v < 4; v++) {
        y[v] = alpha * acc[v];
        if (p.bias && n + v < p.N) y[v] += bf16_lo((uint32_t)p.bias[n + v]);
    }
    if ((p.N & 3) == 0 && n + 3 < p.N) {
        uint2 o;
        o.x = pack_bf16x2(y[0], y[1]);
        o.y = pack_bf16x2(y[2], y[3]);
        *(uint2*)(O + n) = o;
    } else {
#pragma unroll
        for (int v = 0; v < 4; v++)
            if (n + v < p.N) O[n + v] = (uint16_t)pack_bf16x2(y[v], 0.0f);
    }
#endif
}

hipError_t launch_gemm_w4a16(const GemmArgs& g, hipStream_t st) {
    GParams p{};
    p.a = g.a; p.b = g.b; p.b_sf = g.b_sf;
    p.alpha = g.alpha; p.bias = g.bias; p.out = g.out;
    p.M = g.m; p.N = g.n; p.K = g.k; p.E = 1;
    const int64_t cp = ((g.k / 16) + 3) / 4 * 4;
    p.cpa4 = (int)(cp / 4);
    p.nblk = (int)(g.k / 16);
    dim3 grid((unsigned)((p.N + 15) / 16), (unsigned)((p.M + 15) / 16), 1u);
    if (p.K % 128 == 0) k_gemm_w4a16<true><<<grid, 64 * kSkinnyWaves, 0, st>>>(p);
    else k_gemm_w4a16<false><<<grid, 64 * kSkinnyWaves, 0, st>>>(p);
    return hipGetLastError();
}

static hipError_t launch_skinny(GParams p, bool lora, hipStream_t st) {
    dim3 grid((unsigned)((p.N + 15) / 16), (unsigned)((p.M + 15) / 16), (unsigned)p.E);
    const bool aligned = (p.K % 128) == 0;
    if (lora) {
        if (aligned) k_gemm_skinny<true, true><<<grid, 64 * kSkinnyWaves, 0, st>>>(p);
        else k_gemm_skinny<false, true><<<grid, 64 * kSkinnyWaves, 0, st>>>(p);
    } else {
        if (aligned) k_gemm_skinny<true, false><<<grid, 64 * kSkinnyWaves, 0, st>>>(p);
        else k_gemm_skinny<false, false><<<grid, 64 * kSkinnyWaves, 0, st>>>(p);
    }
    return hipGetLastError();
}

enum class Tile { T256x256, T256x192, T128x256, T128x256K2, T128x128, Skinny };

// Workgroup tile per problem.  Larger wave tiles need fewer dequantization
// instructions per MFMA (64x128 waves of the 256x256 and 128x256 tiles: 6,
// 64x96 waves of the 256x192 tile: 6.7, 64x64 waves of the 128x128 tile:
// 8), and two waves per SIMD hide one wave's dequantization behind the
// other's MFMAs, but the grid must still spread evenly over the 256 CUs
// (measured on the workload shapes: the 256x256 tile needs at least two
// tiles per CU; a single problem that makes one round of 256x192 tiles
// takes them; the 128x128 tile wins when it gives three per CU; with at most
// one 128x256 tile per CU the K loop is split over two wave groups so each
// SIMD still holds two waves).

static Tile pick_tile(int64_t m, int64_t n, int64_t k, int64_t E) {
    auto tiles = [&](int64_t bm, int64_t bn) { return E * ((m + bm - 1) / bm) * ((n + bn - 1) / bn); };
    const bool even_steps = ((k + 127) / 128) % 2 == 0;
    if (m <= 64) return Tile::Skinny;
    if (tiles(256, 256) >= 2 * 256) return Tile::T256x256;
    if (E == 1 && tiles(256, 192) <= 256 && tiles(256, 192) >= 224) return Tile::T256x192;
    if (E == 1 && tiles(128, 128) >= 3 * 256) return Tile::T128x128;
    if (tiles(128, 256) >= 128) return even_steps && tiles(128, 256) <= 256 ? Tile::T128x256K2 : Tile::T128x256;
    return Tile::T128x128;
}

// Workgroups of a persistent launch: one per CU, at most the workspace's
// slot count.
static int sk_grid_size() {
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        cus <= 0)
        return 0;
    return cus < kGemmWsSlots ? cus : kGemmWsSlots;
}

// The split-tail schedule on the K-split 128x256 tile replaces a 128x256
// tile choice that would leave one wave per SIMD or a mostly idle second
// round: for the grouped form (live tiles unknown on the host) always, and
// for a single problem (then more 128x256 tiles than CUs, but fewer than
// two 256x256 or three 128x128 tiles per CU) given a workspace.  K must make
// an even number of steps (the two K groups of the tile).
static bool use_split_schedule(const GemmArgs& g, Tile t) {
    if (((g.k + 127) / 128) % 2 != 0) return false;
    if (g.E > 1) return g.E <= kSkMaxExperts && (t == Tile::T128x256 || t == Tile::T128x256K2);
    return g.ws && t == Tile::T128x256;
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
    p.nblk = (int)(g.k / 16);
    p.rpa = (int)((g.m + 127) / 128 * 128);
    p.rpb = (int)((g.n + 127) / 128 * 128);
    p.sfa = (int64_t)p.rpa * cp;
    p.sfb = (int64_t)p.rpb * cp;
    const bool lora = g.d != nullptr;
    const Tile t = pick_tile(g.m, g.n, g.k, g.E);
    if (use_split_schedule(g, t)) {
        const int G = sk_grid_size();
        if (G <= 0) return hipErrorInvalidDevice;
        return launch_tile_sk<128, 256, 2, 2, 2, 2>(p, lora, g.ws, G, st);
    }
    switch (t) {
    case Tile::T256x256: return launch_tile<256, 256, 4, 2, 2>(p, lora, st);
    case Tile::T256x192: return launch_tile<256, 192, 4, 2, 2>(p, lora, st);
    case Tile::T128x256: return launch_tile<128, 256, 2, 2, 2>(p, lora, st);
    case Tile::T128x256K2: return launch_tile<128, 256, 2, 2, 2, 2>(p, lora, st);
    case Tile::Skinny: return launch_skinny(p, lora, st);
    default: return launch_tile<128, 128, 2, 2, 2>(p, lora, st);
    }
}

// Grouped masked GEMM whose epilogue applies silu_and_mul to the gate | up
// output and quantizes it to NVFP4 with a static per-expert global scale.
// Whole-K tiles only (the K-split tile would change the accumulation order
// and the skinny kernel has no staged epilogue); a tile covers BN/2 columns
// of h, so the tile counts are those of the plain GEMM over N = 2H.
hipError_t launch_gemm_silu_quantize(const GemmArgs& g, const SiluQuantOut& q, hipStream_t st) {
    GParams p{};
    p.a = g.a; p.b = g.b; p.a_sf = g.a_sf; p.b_sf = g.b_sf;
    p.alpha = g.alpha; p.mask = g.mask;
    p.M = g.m; p.N = g.n; p.K = g.k;
    p.E = g.E;
    const int64_t cp = ((g.k / 16) + 3) / 4 * 4;
    p.cpa4 = (int)(cp / 4);
    p.nblk = (int)(g.k / 16);
    p.rpa = (int)((g.m + 127) / 128 * 128);
    p.rpb = (int)((g.n + 127) / 128 * 128);
    p.sfa = (int64_t)p.rpa * cp;
    p.sfb = (int64_t)p.rpb * cp;
    p.H = g.n / 2;
    const int64_t qcp = ((p.H / 16) + 3) / 4 * 4;
    p.q_cp4 = (int)(qcp / 4);
    p.q_rpad = p.rpa;
    p.q_sfsz = (int64_t)p.q_rpad * qcp;
    p.q_fp4 = q.fp4; p.q_sf = q.sf; p.q_gs = q.gs;
    auto tiles = [&](int64_t bm, int64_t bn) { return g.E * ((g.m + bm - 1) / bm) * ((p.H + bn / 2 - 1) / (bn / 2)); };
    if (tiles(256, 256) >= 2 * 256) return launch_tile_siluq<256, 256, 4, 2, 3>(p, st);
    if (tiles(128, 256) >= 128) return launch_tile_siluq<128, 256, 2, 2, 2>(p, st);
    return launch_tile_siluq<128, 128, 2, 2, 2>(p, st);
}

}  // namespace nvfp4
