// gemm_common.h -- pieces shared by the block-scaled GEMM kernels (NVFP4 and
// MX): the kernel parameters, raw buffer resources for the direct-to-LDS
// staging loads, the wait-count helper, the LDS chunk swizzle of a staged FP4
// tile, the swizzled scale-dword offset and the XCD-aware tile order.
#pragma once

#include "device_common.h"

namespace nvfp4 {

// native vectors (not HIP's struct types) keep loaded values in registers
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) uint8_t lds_u8;

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
    int cpa4;            // column groups of the scale layout = pad_up(K/16,4)/4 (K/32 for MX)
    int nblk;            // scale blocks per row = K/16 (K/32 for MX)
    int rpa, rpb;        // padded rows of the scale buffers
    int tiles_m, tiles_n;
    int xcd_chunk;       // tiles per XCD when the tile count splits evenly over 8, else 0
    // quantizing epilogue (silu_and_mul + NVFP4 of the gate | up output)
    uint8_t* q_fp4;      // [E, M, H/2]
    uint8_t* q_sf;       // [E, q_sfsz]
    const float* q_gs;   // [E] static global scales of the quantized output
    int64_t H;           // gate (= up) width, N = 2H
    int64_t q_sfsz;      // per-expert scale bytes = pad_up(M,128) * pad_up(H/16,4)
    int q_cp4;           // pad_up(H/16,4)/4
    int q_rpad;          // pad_up(M,128)
    // split-tail schedule (persistent K-split launch)
    float* part;         // fp32 partial tiles of the split tail tiles, or null (no split)
    int sk_grid;         // workgroups of the persistent launch
};

// 8 FP4 codes of one dword times one block scale -> 8 fp16 (exact): the
// operand formation of the NVFP4 kernels.
__device__ __forceinline__ f16x8 dequant8(uint32_t w, _Float16 s) {
    const f16x2 ss = f16x2{s, s};
    const f16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0) * ss;
    const f16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1) * ss;
    const f16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2) * ss;
    const f16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3) * ss;
    return f16x8{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
}

__device__ __forceinline__ uint32_t word(const u32x4& v, int j) {
    return j == 0 ? v.x : j == 1 ? v.y : j == 2 ? v.z : v.w;
}

// Byte offset of scale (row, block column c) in the swizzled layout.
__device__ __forceinline__ int64_t scale_byte_off(int64_t row, int c, int cpa4) {
    return ((row >> 7) * cpa4 + (c >> 2)) * 512 + (row & 31) * 16 + ((row & 127) >> 5) * 4 + (c & 3);
}

// Raw buffer resource (gfx9 word 3: 32-bit untyped records).  Loads past
// `bytes` return zeros.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// s_waitcnt immediate waiting until at most N vector-memory operations are
// outstanding, other counters unconstrained (gfx9 encoding: vmcnt bits 3:0
// and 15:14, expcnt 6:4, lgkmcnt 11:8).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// LDS layout of a staged FP4 tile: rows of 64 bytes (the 128 elements of one
// K step); 16-byte chunk c of row r sits in slot c ^ swz(r).  A wave's staging
// load covers 16 whole rows (1 KB, contiguous), and a fragment read (32
// consecutive rows, one chunk each) touches every bank group once per 8 or 16
// lanes.  The scale region follows: row t of the tile (A rows, then B rows)
// holds its raw scale dwords of the step (NVFP4: two, blocks 0-3 and 4-7,
// at 8t; MX: one, blocks 0-3 of 32 elements, at 4t).
__device__ __forceinline__ int swz(int r) { return ((r >> 2) ^ (r & 2)) & 3; }

// Byte offset of scale dword (row, column group cg) in the swizzled layout.
__device__ __forceinline__ uint32_t scale_dword_off(int64_t row, int cg, int cpa4) {
    return (uint32_t)(((row >> 7) * cpa4 + cg) * 512 + (row & 31) * 16 + ((row & 127) >> 5) * 4);
}

// Tile coordinates of this workgroup.  Workgroups are dealt to the 8 XCDs
// round-robin; when the tile count splits evenly, XCD x is given the x-th
// contiguous eighth of the tile order, and within it tiles advance down
// groups of 8 tile rows, so the workgroups that run together on one XCD share
// A and B panels in that XCD's L2.
__device__ __forceinline__ void tile_coords(const GParams& p, int& tm, int& tn) {
    int L = blockIdx.x;
    if (p.xcd_chunk) L = (L & 7) * p.xcd_chunk + (L >> 3);
    constexpr int G = 8;
    const int per_group = G * p.tiles_n;
    const int grp = L / per_group;
    const int first = grp * G;
    const int rows = p.tiles_m - first < G ? p.tiles_m - first : G;
    const int in = L - grp * per_group;
    tm = first + in % rows;
    tn = in / rows;
}

}  // namespace nvfp4
