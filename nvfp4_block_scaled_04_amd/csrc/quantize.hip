// quantize.hip -- NVFP4 quantization kernels for gfx950.
//
// What is computed (FastVideo PR #1350 _global_sf; TensorRT-LLM
// NVFP4LinearMethod.create_weights; flashinfer PR #1774 batched / masked /
// silu_and_mul quantize; flashinfer mm_nvfp4_svdquant, parameters a and
// a_sf):
//   x'  = nan_to_num(prologue(x))     prologue: none | x*pqs | silu(g)*u -> bf16
//   gs  = 2688 / max(amax(x'), 1e-12)                   (DYNAMIC mode)
//   s   = ue4m3((block_amax / 6) * gs)                  per 16 elements of a row
//   q   = e2m1(x' * (gs / dec(s)))                      packed two per byte
//   scales in the 128x4 swizzled, zero-padded layout.
//
// Work decomposition: one workgroup of 256 threads owns a 128-row x 64*CT
// column tile, i.e. CT whole 512-byte tiles of the swizzled scale layout
// (CT per pass and shape, see quant_ct_for).
// A lane owns whole 16-element blocks: BPR = 4*CT consecutive lanes cover one
// row segment of the tile (a wave reads 64/BPR rows x 32*BPR contiguous bytes
// of bf16 per load pair), so the block scale is computed once per block with
// no cross-lane traffic, and every load of a lane is issued before any of it
// is used.  The element factor r = gs / dec(s) comes from a 128-entry
// per-workgroup LDS table (dec(s) takes only the ue4m3 code values), and
// bamax / 6 is the correctly rounded quotient computed with one FMA
// correction (div6).  The scale bytes are gathered in LDS and written with
// 16-byte stores.
//
// DYNAMIC mode is an amax pass that leaves partial maxima, then the quantize
// pass.  A single tensor (no row mask) is read by the amax pass as one flat
// stream (k_amax_flat: each workgroup walks contiguous 16 KB chunks, grid
// capped at 1024); masked and batched items are read tile by tile (k_amax).
// Where the partials go:
//   * with a caller workspace: into it, and every quantize workgroup reduces
//     them itself while its tile's loads are in flight (two launches);
//   * otherwise: into the call's own scale buffer (free until the quantize
//     pass overwrites it; it holds at least one float per partial), reduced
//     by a one-workgroup-per-item finish kernel before the quantize pass
//     (three launches).
// No atomics and no device-wide fences are involved: the kernel boundaries
// order every step.
#include <mutex>

#include "device_common.h"
#include "internal.h"
#include "quant_block.h"

namespace nvfp4 {

struct QParams {
    const void* x;
    const uint16_t* pqs;   // [K] bf16 or null
    const int32_t* mask;   // [b] or null
    float* gs;             // [b]
    uint8_t* out_fp4;      // [b, m, K/2]
    uint8_t* out_sf;       // [b, sfsz]
    int64_t m;             // rows per item
    int64_t K;             // quantized width
    int64_t k_in;          // input row stride in elements
    int64_t sfsz;          // per-item scale bytes
    int b;
    int nct;               // 64-column tiles = ceil(K/64) = Cp/4
    int nrt;               // row tiles = ceil(m/128)
    float* part;           // DYNAMIC: partial maxima, item e at part + e * part_stride
    int64_t part_stride;   // floats between items' partials
    int nparts;            // partials per item
    const float* gs_other; // [b] the GEMM partner's global scales, when alpha_out is set
    float* alpha_out;      // [b] or null: alpha = 1 / (gs * gs_other)
    uint16_t* hbuf;        // silu, DYNAMIC, large workspace: the amax pass's h [b, m, K] bf16 (valid rows)
};

// alpha of item e from its final global scale, with the arithmetic of k_alpha
__device__ __forceinline__ void write_alpha(const QParams& p, int e, float gs) {
    if (p.alpha_out) p.alpha_out[e] = 1.0f / (gs * p.gs_other[e]);
}

template <int V>
__device__ __forceinline__ void load_block(const QParams& p, int64_t e, int64_t row, int64_t col,
                                           u32x4 (&r)[loads_per_block<V>()]) {
    const int64_t roff = (e * p.m + row) * p.k_in;
    if constexpr (V == V_F32 || V == V_F32_SMOOTH) {
        const u32x4* src = (const u32x4*)((const float*)p.x + roff + col);
        r[0] = src[0]; r[1] = src[1]; r[2] = src[2]; r[3] = src[3];
    } else if constexpr (V == V_SILU) {
        const u32x4* g = (const u32x4*)((const uint16_t*)p.x + roff + col);
        const u32x4* u = (const u32x4*)((const uint16_t*)p.x + roff + p.K + col);
        r[0] = g[0]; r[1] = g[1]; r[2] = u[0]; r[3] = u[1];
    } else {
        const u32x4* src = (const u32x4*)((const uint16_t*)p.x + roff + col);
        r[0] = src[0]; r[1] = src[1];
    }
}

// pre_quant_scale of a block's 16 columns (bf16), smooth variants only.
template <int V>
__device__ __forceinline__ void load_pqs(const QParams& p, int64_t col, u32x4 (&pq)[2]) {
    if constexpr (V == V_BF16_SMOOTH || V == V_F32_SMOOTH) {
        const u32x4* src = (const u32x4*)(p.pqs + col);
        pq[0] = src[0]; pq[1] = src[1];
    } else {
        pq[0] = u32x4{0u, 0u, 0u, 0u};
        pq[1] = u32x4{0u, 0u, 0u, 0u};
    }
}

// Lane layout of a workgroup tile of 128 rows x 64*CT columns: BPR = 4*CT
// lanes own the blocks of one row segment, RPP = 256 / BPR rows are covered
// per pass, NP = 128 / RPP passes.
template <int CT>
struct TileMap {
    static constexpr int BPR = 4 * CT;
    static constexpr int RPP = 256 / BPR;
    static constexpr int NP = 128 / RPP;
};

// Partial maxima of item e.
__device__ __forceinline__ float* partials(const QParams& p, int e) {
    return p.part + (int64_t)e * p.part_stride;
}

// ---------------------------------------------------------------------------
// DYNAMIC mode: amax partials, finish, then quantize.
// ---------------------------------------------------------------------------

// HOUT (silu only): every block's exact h is also stored to p.hbuf, which
// the quantize pass then reads as a plain bf16 input (silu evaluated once).
template <int V, int CT, bool HOUT = false>
__global__ __launch_bounds__(256) void k_amax(QParams p) {
    static_assert(!HOUT || V == V_SILU, "h is stored by the silu pass");
    using TM = TileMap<CT>;
    constexpr int NL = loads_per_block<V>();
    const int tile = blockIdx.x, e = blockIdx.y;
    const int t = threadIdx.x;
    const int rsub = t / TM::BPR, lb = t % TM::BPR;
    const int valid = clamp_rows(p.mask, e, (int)p.m);
    const int nwct = (p.nct + CT - 1) / CT;
    const int rt = tile / nwct, wct = tile - rt * nwct;
    float amax = 0.0f;
    if ((int64_t)rt * 128 < valid) {  // tiles entirely past the valid rows contribute 0
        int64_t col = (int64_t)wct * 64 * CT + lb * 16;
        const bool col_ok = col < p.K;
        col = col_ok ? col : p.K - 16;
        u32x4 pq[2];
        load_pqs<V>(p, col, pq);
        u32x4 raw[TM::NP][NL];
#pragma unroll
        for (int i = 0; i < TM::NP; i++) {  // every load in flight before any use
            // rows past the valid ones read the last valid row again (a cache
            // hit; not processed): unconditional loads, so the compiler can
            // count them in flight
            const int64_t row = (int64_t)rt * 128 + rsub + TM::RPP * i;
            load_block<V>(p, e, row < valid ? row : valid - 1, col, raw[i]);
        }
#pragma unroll
        for (int i = 0; i < TM::NP; i++) {
            const int64_t row = (int64_t)rt * 128 + rsub + TM::RPP * i;
            if (col_ok && row < valid) {
                if constexpr (HOUT) {
                    uint32_t w[8];
                    silu_block_words(raw[i], w);
                    u32x4* hp = (u32x4*)(p.hbuf + ((int64_t)e * p.m + row) * p.K + col);
                    hp[0] = u32x4{w[0], w[1], w[2], w[3]};
                    hp[1] = u32x4{w[4], w[5], w[6], w[7]};
                    amax = __builtin_fmaxf(amax, bf16_words_amax(w));
                } else if constexpr (V == V_SILU) {
                    amax = __builtin_fmaxf(amax, silu_block_amax(raw[i], amax));
                } else {
                    float f[16];
                    amax = __builtin_fmaxf(amax, process_block<V>(raw[i], pq, f));
                }
            }
        }
    }
    // workgroup max: wave reduction through shuffles, then LDS across waves
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) amax = __builtin_fmaxf(amax, __shfl_xor(amax, off));
    __shared__ float wmax[4];
    if ((t & 63) == 0) wmax[t >> 6] = amax;
    __syncthreads();
    if (t == 0)
        partials(p, e)[tile] =
            __builtin_fmaxf(__builtin_fmaxf(wmax[0], wmax[1]), __builtin_fmaxf(wmax[2], wmax[3]));
}

// Running maximum of the bf16 magnitudes of 8 elements (one 16-byte load),
// compared as integers: NaN patterns are skipped and an infinity is noted
// (the caller takes it as FLT_MAX), which is max |nan_to_num(x)|.
__device__ __forceinline__ void bf16_amax8(const u32x4& v, uint32_t& mb, bool& inf) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
    const uint32_t b = absmax_bits_bf16x8(w);
    if (b < 0x7F80u) {
        mb = b > mb ? b : mb;
    } else {  // inf or NaN in these 8: one at a time
#pragma unroll
        for (int j = 0; j < 8; j++) {
            const uint32_t h = (w[j >> 1] >> (16 * (j & 1))) & 0x7FFFu;
            if (h == 0x7F80u) inf = true;
            else if (h < 0x7F80u) mb = h > mb ? h : mb;
        }
    }
}

// Amax pass over one item as a flat stream (b == 1, no row mask, no silu:
// the valid elements are x[0, m*K) in order).  Each workgroup walks chunks
// of 256 * U 16-byte loads (U in flight per thread), grid-strided; its
// partial maximum of |nan_to_num(x')| goes to part[blockIdx.x].
//   bf16: the maximum of the bf16 magnitudes compared as integers (NaN
//         patterns skipped, inf noted and taken as FLT_MAX);
//   fp32 / smooth: fmax over |x'| (fmax skips NaN) and inf clamped to
//         FLT_MAX at the end, which is the maximum of |nan_to_num(x')|.
template <int V>
__global__ __launch_bounds__(256) void k_amax_flat(QParams p) {
    constexpr bool F32 = V == V_F32 || V == V_F32_SMOOTH;
    constexpr bool SM = V == V_BF16_SMOOTH || V == V_F32_SMOOTH;
    constexpr int EPL = F32 ? 4 : 8;  // elements per 16-byte load
    constexpr int U = 4;
    const u32x4* src = (const u32x4*)p.x;
    const int64_t nl = p.m * p.K / EPL;  // K % 16 == 0: whole loads per row
    const int t = threadIdx.x;
    uint32_t mb = 0;   // bf16: largest finite magnitude pattern
    bool inf = false;  // bf16: an infinity was seen
    float a = 0.0f;    // other variants
    for (int64_t base = (int64_t)blockIdx.x * 256 * U; base < nl; base += (int64_t)gridDim.x * 256 * U) {
        u32x4 v[U];
#pragma unroll
        for (int u = 0; u < U; u++) {
            const int64_t i = base + u * 256 + t;
            v[u] = i < nl ? src[i] : u32x4{0u, 0u, 0u, 0u};
        }
        if constexpr (V == V_BF16) {
#pragma unroll
            for (int u = 0; u < U; u++) bf16_amax8(v[u], mb, inf);
        } else {
#pragma unroll
            for (int u = 0; u < U; u++) {
                const int64_t i = base + u * 256 + t;
                float f[EPL];
                if constexpr (F32) {
                    f[0] = bits_f(v[u].x); f[1] = bits_f(v[u].y); f[2] = bits_f(v[u].z); f[3] = bits_f(v[u].w);
                } else {
                    const uint32_t w[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
#pragma unroll
                    for (int j = 0; j < 4; j++) { f[2 * j] = bf16_lo(w[j]); f[2 * j + 1] = bf16_hi(w[j]); }
                }
                if constexpr (SM) {
                    // pre_quant_scale of these EPL columns (i * EPL is a multiple of EPL, K of 16)
                    const int64_t col = i < nl ? (i * EPL) % p.K : 0;
                    uint32_t pw[EPL / 2];
                    if constexpr (F32) {
                        const uint2 q = *(const uint2*)(p.pqs + col);
                        pw[0] = q.x; pw[1] = q.y;
                    } else {
                        const u32x4 q = *(const u32x4*)(p.pqs + col);
                        pw[0] = q.x; pw[1] = q.y; pw[2] = q.z; pw[3] = q.w;
                    }
#pragma unroll
                    for (int j = 0; j < EPL / 2; j++) {
                        f[2 * j] = f[2 * j] * bf16_lo(pw[j]);
                        f[2 * j + 1] = f[2 * j + 1] * bf16_hi(pw[j]);
                    }
                }
#pragma unroll
                for (int j = 0; j < EPL; j++) a = __builtin_fmaxf(a, __builtin_fabsf(f[j]));
            }
        }
    }
    if constexpr (V == V_BF16) a = inf ? kFp32Max : bits_f(mb << 16);
    else a = __builtin_fminf(a, kFp32Max);
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) a = __builtin_fmaxf(a, __shfl_xor(a, off));
    __shared__ float wmax[4];
    if ((t & 63) == 0) wmax[t >> 6] = a;
    __syncthreads();
    if (t == 0) p.part[blockIdx.x] = __builtin_fmaxf(__builtin_fmaxf(wmax[0], wmax[1]), __builtin_fmaxf(wmax[2], wmax[3]));
}

// gs = 2688 / max(amax, 1e-12) in fp32 (448 * 6 over the clamped amax).
__device__ __forceinline__ float gs_from_amax(float am) {
    const float lo = 1e-12f;
    return 2688.0f / (am < lo ? lo : am);
}

// Largest of item e's partial maxima, over the whole workgroup (every
// thread gets it); wmax: 4 floats of LDS.
__device__ __forceinline__ float reduce_partials(const QParams& p, int e, float* wmax) {
    const float* part = partials(p, e);
    const int t = threadIdx.x;
    float a = 0.0f;
    int i = t;
    for (; i + 768 < p.nparts; i += 1024)  // four independent loads in flight
        a = __builtin_fmaxf(__builtin_fmaxf(a, __builtin_fmaxf(part[i], part[i + 256])),
                            __builtin_fmaxf(part[i + 512], part[i + 768]));
    for (; i < p.nparts; i += 256) a = __builtin_fmaxf(a, part[i]);
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) a = __builtin_fmaxf(a, __shfl_xor(a, off));
    if ((t & 63) == 0) wmax[t >> 6] = a;
    __syncthreads();
    return __builtin_fmaxf(__builtin_fmaxf(wmax[0], wmax[1]), __builtin_fmaxf(wmax[2], wmax[3]));
}

// gs[e] = 2688 / max(amax_e, 1e-12) from item e's partial maxima.
__global__ __launch_bounds__(256) void k_finish_gs(QParams p) {
    __shared__ float wmax[4];
    const int e = blockIdx.x;
    const float am = reduce_partials(p, e, wmax);
    if (threadIdx.x == 0) p.gs[e] = gs_from_amax(am);
}

// One tile of the quantize pass; gs_of() gives the item's global scale (read
// while the tile's loads are in flight).
template <int V, int CT, typename GsFn>
__device__ __forceinline__ void quantize_tile(const QParams& p, int wct, int rt, int e, GsFn gs_of) {
    using TM = TileMap<CT>;
    constexpr int NL = loads_per_block<V>();
    const int t = threadIdx.x;
    const int rsub = t / TM::BPR, lb = t % TM::BPR;
    const int c = lb >> 2;   // swizzle tile within the workgroup
    const int blk = lb & 3;  // block column within that tile
    const int valid = clamp_rows(p.mask, e, (int)p.m);
    int64_t col = (int64_t)wct * 64 * CT + lb * 16;
    const bool col_ok = col < p.K;
    col = col_ok ? col : p.K - 16;
    __shared__ __align__(16) uint8_t sbuf[512 * CT];
    __shared__ float rtab[128];
    uint8_t* q = p.out_fp4 + (int64_t)e * p.m * (p.K / 2);
    // swizzle tiles this workgroup owns that exist in the buffer
    const int ntile_here = (p.nct - wct * CT) < CT ? (p.nct - wct * CT) : CT;
    uint8_t* sf_dst = p.out_sf + (int64_t)e * p.sfsz + ((int64_t)rt * p.nct + (int64_t)wct * CT) * 512;

    if ((int64_t)rt * 128 >= valid) {  // tile entirely past the valid rows: zero scales only
        for (int i = t; i < ntile_here * 32; i += 256) *(u32x4*)(sf_dst + i * 16) = u32x4{0u, 0u, 0u, 0u};
        return;
    }
    u32x4 pq[2];
    load_pqs<V>(p, col, pq);
    u32x4 raw[TM::NP][NL];
#pragma unroll
    for (int i = 0; i < TM::NP; i++) {  // every load in flight before any use
        // rows past the valid ones read the last valid row again (a cache
        // hit; not processed, below): unconditional loads, so the compiler
        // can count them in flight
        const int64_t row = (int64_t)rt * 128 + rsub + TM::RPP * i;
        load_block<V>(p, e, row < valid ? row : valid - 1, col, raw[i]);
    }
    // element factors r = gs / dec(s) for every scale code (0 for code 0),
    // computed while the loads are in flight
    const float gs = gs_of();
    if (t < 128) {
        const float dec = ue4m3_decode((uint32_t)t);
        rtab[t] = dec == 0.0f ? 0.0f : gs / dec;
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < TM::NP; i++) {
        const int rl = rsub + TM::RPP * i;  // row within the 128-row tile
        const int64_t row = (int64_t)rt * 128 + rl;
        const bool active = col_ok && row < valid;
        uint32_t sc = 0u;  // rows past the valid ones (and blocks past K): zero scale, no FP4 written
        if (active) {
            float f[16];
            const float bamax = process_block<V>(raw[i], pq, f);
            sc = ue4m3_encode(div6(bamax) * gs);
            const float r = rtab[sc];
            uint32_t w0 = 0, w1 = 0;
            w0 = NVFP4_PACK_FP4(w0, f[0] * r, f[1] * r, 0);
            w0 = NVFP4_PACK_FP4(w0, f[2] * r, f[3] * r, 1);
            w0 = NVFP4_PACK_FP4(w0, f[4] * r, f[5] * r, 2);
            w0 = NVFP4_PACK_FP4(w0, f[6] * r, f[7] * r, 3);
            w1 = NVFP4_PACK_FP4(w1, f[8] * r, f[9] * r, 0);
            w1 = NVFP4_PACK_FP4(w1, f[10] * r, f[11] * r, 1);
            w1 = NVFP4_PACK_FP4(w1, f[12] * r, f[13] * r, 2);
            w1 = NVFP4_PACK_FP4(w1, f[14] * r, f[15] * r, 3);
            *(uint2*)(q + row * (p.K / 2) + col / 2) = uint2{w0, w1};
        }
        sbuf[c * 512 + (rl & 31) * 16 + (rl >> 5) * 4 + blk] = (uint8_t)sc;
    }
    __syncthreads();
    for (int i = t; i < ntile_here * 32; i += 256) *(u32x4*)(sf_dst + i * 16) = *(const u32x4*)(sbuf + i * 16);
}

// FROM_PART: DYNAMIC mode with the partial maxima in a workspace: every
// workgroup reduces item e's partials itself (they are few and come from L2,
// while the tile's own loads are in flight) and the first workgroup of the
// item writes gs.  Otherwise gs[e] is final here (given, or written by the
// finish kernel before this pass).
template <int V, int CT, bool FROM_PART>
__global__ __launch_bounds__(256) void k_quantize(QParams p) {
    const int e = blockIdx.z;
    const bool first = blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x == 0;
    if constexpr (FROM_PART) {
        // an item without valid rows has only tiles that never ask for gs:
        // its amax is 0 (all its partials are)
        if (first && clamp_rows(p.mask, e, (int)p.m) == 0) {
            p.gs[e] = gs_from_amax(0.0f);
            write_alpha(p, e, p.gs[e]);
        }
        __shared__ float wmax[4];
        quantize_tile<V, CT>(p, blockIdx.x, blockIdx.y, e, [&] {
            const float gs = gs_from_amax(reduce_partials(p, e, wmax));
            if (first) {
                p.gs[e] = gs;
                write_alpha(p, e, gs);
            }
            return gs;
        });
    } else {
        if (p.alpha_out && first) write_alpha(p, e, p.gs[e]);
        quantize_tile<V, CT>(p, blockIdx.x, blockIdx.y, e, [&] { return p.gs[e]; });
    }
}

// ---------------------------------------------------------------------------
// Small items (at most 2^16 elements, 2^15 with the silu prologue) in
// DYNAMIC mode, in one launch: every workgroup of the tiled pass first
// recomputes the item's global amax over all of its valid blocks -- the item
// is small, so the redundant reads come from L2 and cost less than the amax
// and finish launches -- forms gs with the finish kernel's arithmetic, and
// quantizes its own tile.  The first workgroup of the item writes gs.  Same
// arithmetic and bytes as the three-kernel path.
// ---------------------------------------------------------------------------
template <int V>
constexpr int64_t fused_max_elems() { return V == V_SILU ? 32768 : 65536; }

template <int V>
__device__ __forceinline__ float item_amax(const QParams& p, int e, int valid) {
    if constexpr (V == V_BF16) {
        // plain bf16: the item's valid rows as one flat stream of 16-byte
        // loads, magnitudes compared as integers
        constexpr int UL = 32;  // loads per thread in flight together
        const u32x4* src = (const u32x4*)((const uint16_t*)p.x + (int64_t)e * p.m * p.k_in);
        const int64_t nl = (int64_t)valid * p.K / 8;
        uint32_t mb = 0;
        bool inf = false;
        for (int64_t b0 = threadIdx.x; b0 < nl; b0 += 256 * UL) {
            u32x4 v[UL];
#pragma unroll
            for (int u = 0; u < UL; u++) {
                const int64_t i = b0 + 256 * u;
                v[u] = i < nl ? src[i] : u32x4{0u, 0u, 0u, 0u};
            }
#pragma unroll
            for (int u = 0; u < UL; u++) bf16_amax8(v[u], mb, inf);
        }
        return inf ? kFp32Max : bits_f(mb << 16);
    }
    constexpr int NL = loads_per_block<V>();
    constexpr int U = V == V_BF16 ? 16 : 8;  // blocks per thread with loads in flight together
    const int64_t nblk = p.K / 16, nb = (int64_t)valid * nblk;
    float amax = 0.0f;
    for (int64_t b0 = threadIdx.x; b0 < nb; b0 += 256 * U) {
        u32x4 raw[U][NL], pq[U][2];
#pragma unroll
        for (int u = 0; u < U; u++) {
            const int64_t b = b0 + 256 * u < nb ? b0 + 256 * u : nb - 1;  // past the end: a repeat, same maximum
            const int64_t row = b / nblk, col = (b - row * nblk) * 16;
            load_block<V>(p, e, row, col, raw[u]);
            load_pqs<V>(p, col, pq[u]);
        }
#pragma unroll
        for (int u = 0; u < U; u++) {
            float f[16];
            amax = __builtin_fmaxf(amax, process_block<V>(raw[u], pq[u], f));
        }
    }
    return amax;
}

template <int V, int CT>
__global__ __launch_bounds__(256) void k_quantize_fused(QParams p) {
    const int wct = blockIdx.x, rt = blockIdx.y, e = blockIdx.z;
    const int t = threadIdx.x;
    const int valid = clamp_rows(p.mask, e, (int)p.m);
    const bool first = wct == 0 && rt == 0;
    __shared__ float wmax[4];
    // no valid rows: every tile only zeroes its scales, and gs comes from amax 0
    if (valid == 0 && first && t == 0) {
        p.gs[e] = gs_from_amax(0.0f);
        write_alpha(p, e, p.gs[e]);
    }
    // The amax pass runs where the tile asks for gs, after its own loads are
    // issued, so they land meanwhile (tiles past the valid rows never ask).
    quantize_tile<V, CT>(p, wct, rt, e, [&] {
        float a = item_amax<V>(p, e, valid);
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) a = __builtin_fmaxf(a, __shfl_xor(a, off));
        if ((t & 63) == 0) wmax[t >> 6] = a;
        __syncthreads();
        const float gs = gs_from_amax(__builtin_fmaxf(__builtin_fmaxf(wmax[0], wmax[1]),
                                                      __builtin_fmaxf(wmax[2], wmax[3])));
        if (first && t == 0) {
            p.gs[e] = gs;
            write_alpha(p, e, gs);
        }
        return gs;
    });
}


// ---------------------------------------------------------------------------
// Smooth quantize with the SVDQuant LoRA-down projection fused (flashinfer
// mm_nvfp4_svdquant: a is the NVFP4 quantization of x * pqs, and d = x @
// (pqs[:, None] * L2^T) is its rank-r projection): one read of x feeds both.
// A workgroup of 16 waves owns a 16-row band and walks K in chunks of
// kLoraChunk columns; in a chunk, wave w owns the band's 16 rows x 64
// columns 64w.. (lane l: row l/4, 16-element block l%4; each row's 128
// bytes read contiguously by four lanes), so a wave needs no other wave's
// data until the end: the block is quantized with the smooth pass's
// arithmetic, and the products x * pqs that the quantization forms (exact in
// fp32: two 8-bit significands) are split exactly into two bf16 halves, hi =
// bf16(x * pqs) and lo = x * pqs - hi (at most 8 significant bits, so exact
// in bf16), written to the wave's own LDS buffers and read back in the MFMA
// operand layout (the wave's LDS accesses execute in order; no workgroup
// barrier).  The wave then projects its two 32-column slices with
// v_mfma_f32_16x16x32_bf16: l2 as read (every workgroup reads the same rows,
// through the caches) as the A operand against hi and against lo, so every
// product is exact and only fp32 accumulation rounds.  The accumulators carry
// across chunks; the next two chunks' rows (ranks above 64: the next one's)
// are in flight while a chunk is worked on.  At the end the waves' partial projections are added through LDS (one
// barrier) and stored as bf16.  Any K with K % 16 == 0.
//
// PREP: the weight arrives prepared, w = pqs[:, None] * L2^T split exactly
// into hi + lo bf16 halves ([2, r, K], k_lora_split below), so x itself (bf16,
// exact) is the MFMA operand: nothing is split per element, and only x passes
// through the wave's LDS buffer (one buffer instead of two), against hi and
// against lo.  (A lane layout in which the registers x arrives in are
// already the MFMA operand, row = lane % 16, puts 16 rows in every 16-lane
// group of a load and measured 35% slower than the split it replaces.)
// ---------------------------------------------------------------------------

constexpr int kLoraWaves = 16;                 // = rows per band
constexpr int kLoraSlab = 64;                  // columns of a wave per chunk
constexpr int kLoraChunk = kLoraWaves * kLoraSlab;

template <int RT, bool PREP>  // rank tiles of 16; prepared (split) weight
__global__ __launch_bounds__(64 * kLoraWaves) void k_quantize_lora(QParams p, const uint16_t* l2, uint16_t* d_out,
                                                                  int rank) {
    constexpr int XP = kLoraSlab + 8;  // bf16 per LDS row of a wave's buffer (16 bytes of pad spread the banks)
    constexpr int WBUF = 16 * XP;      // bf16 per buffer (hi or lo of the wave's 16 x 64 slab)
    constexpr int SPW = kLoraSlab / 32;  // projection slices per wave per chunk
    // rank 32: the projection operands of the next chunk load with its rows;
    // larger ranks load each slice's operands just before its MFMAs (the
    // register file of a 16-wave workgroup holds no more)
    constexpr bool PREFETCH = RT <= 2 && !PREP;
    constexpr int PART = (kLoraWaves - 1) * RT * 64 * 8;  // bf16-sized slots of the waves' partial sums
    constexpr int XS = kLoraWaves * (PREP ? 1 : 2) * WBUF;
    constexpr int NH = PREP ? 2 : 1;  // weight operands per rank tile and slice (PREP: hi, lo)
    typedef float f32x2 __attribute__((ext_vector_type(2)));
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    __shared__ __align__(16) uint16_t xs[XS > PART ? XS : PART];
    __shared__ float rtab[128];
    const int t = threadIdx.x, lane = t & 63;
    const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
    const int64_t m0 = (int64_t)blockIdx.x * 16;
    const int lr = lane >> 2, lb = lane & 3;  // this lane's row of the band, block of the slab
    const int64_t row = m0 + lr;
    const bool row_ok = row < p.m;
    const uint16_t* xrow = (const uint16_t*)p.x + (row_ok ? row : p.m - 1) * p.k_in;
    const int nbk = (int)(p.K / 16);
    const int nch = (int)((p.K + kLoraChunk - 1) / kLoraChunk);
    const int r16 = lane & 15, kg = lane >> 4;
    const float gs = p.gs[0];
    if (t < 128) {
        const float dec = ue4m3_decode((uint32_t)t);
        rtab[t] = dec == 0.0f ? 0.0f : gs / dec;
    }
    uint16_t* const bhi = xs + wave * (PREP ? 1 : 2) * WBUF;  // PREP: x itself
    uint16_t* const blo = bhi + WBUF;

    // this lane's block of chunk c (past K: the last block, never stored)
    auto load_rows = [&](int c, u32x4 (&raw)[2], u32x4 (&pq)[2]) {
        int cb = c * (kLoraChunk / 16) + wave * (kLoraSlab / 16) + lb;
        cb = cb < nbk ? cb : nbk - 1;
        const u32x4* src = (const u32x4*)(xrow + (int64_t)cb * 16);
        raw[0] = src[0];
        raw[1] = src[1];
        load_pqs<V_BF16_SMOOTH>(p, (int64_t)cb * 16, pq);
    };
    // l2 operand of this wave's slice j of chunk c: ranks 16 i + r16 at this
    // lane's 8 columns (past K: column 0, and the operand is zeroed at its
    // use).  Every load here is issued on every path, so that the compiler
    // can count the loads in flight and wait only for the ones a use needs.
    auto slice_col = [&](int c, int j) {
        return (int64_t)c * kLoraChunk + wave * kLoraSlab + j * 32 + kg * 8;
    };
    // (PREP: the prepared weight is stored in this operand's order, one
    // 1024-byte fragment per half, rank tile and 32-column slice, so a wave
    // reads each contiguously; slices past the end read slice 0)
    const int64_t nsl = (p.K + 31) / 32;
    auto load_slice = [&](int c, int j, u32x4 (&b)[RT][NH]) {
        if constexpr (PREP) {
            int64_t sl = (int64_t)c * (kLoraChunk / 32) + wave * (kLoraSlab / 32) + j;
            sl = sl < nsl ? sl : 0;
#pragma unroll
            for (int i = 0; i < RT; i++)
#pragma unroll
                for (int h = 0; h < NH; h++)
                    b[i][h] = *(const u32x4*)(l2 + (((int64_t)(h * RT + i) * nsl + sl) * 64 + lane) * 8);
        } else {
            const int64_t col = slice_col(c, j);
            const int64_t cs = col < p.K ? col : 0;
#pragma unroll
            for (int i = 0; i < RT; i++) b[i][0] = *(const u32x4*)(l2 + (int64_t)(i * 16 + r16) * p.K + cs);
        }
    };
    auto load_proj = [&](int c, u32x4 (&b)[PREFETCH ? SPW : 1][RT][NH]) {
#pragma unroll
        for (int j = 0; j < SPW; j++) load_slice(c, j, b[j]);
    };

    f32x4 acc[RT];
#pragma unroll
    for (int i = 0; i < RT; i++) acc[i] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    // rows of chunks c, c + 1 and (rank 32 and 64) c + 2: one or two chunks in
    // flight while one is worked on (chunk indices past the end repeat the
    // last chunk); the larger ranks' registers hold one
    constexpr bool DEEP = RT <= 4;
    u32x4 raw[2], pqb[2], nraw[2], npqb[2], n2raw[2], n2pqb[2];
    u32x4 bf[PREFETCH ? SPW : 1][RT][NH];
    load_rows(0, raw, pqb);
    if constexpr (DEEP) load_rows(1 < nch ? 1 : 0, nraw, npqb);
    if constexpr (PREFETCH) load_proj(0, bf);
    __syncthreads();  // rtab

    uint8_t* const q = p.out_fp4;
    for (int c = 0; c < nch; c++) {
        // later chunks' rows, in flight while this chunk is worked on (past
        // the end: the last chunk again; unconditional, like every load here)
        if constexpr (DEEP) load_rows(c + 2 < nch ? c + 2 : nch - 1, n2raw, n2pqb);
        else load_rows(c + 1 < nch ? c + 1 : c, nraw, npqb);

        // ---- quantize this lane's block
        const int cb = c * (kLoraChunk / 16) + wave * (kLoraSlab / 16) + lb;  // block column
        const bool in_k = cb < nbk;
        const bool blk_ok = row_ok && in_k;
        float f[16];
        const float bamax = process_block<V_BF16_SMOOTH>(raw, pqb, f);
        const uint32_t sc = blk_ok ? ue4m3_encode(div6(bamax) * gs) : 0u;
        uint32_t w0, w1;
        pack_block(f, rtab[sc], w0, w1);
        if (blk_ok) *(uint2*)(q + row * (p.K / 2) + (int64_t)cb * 8) = uint2{w0, w1};
        // the 4 scale bytes of a swizzle dword sit in 4 neighbouring lanes
        // (blocks lb = 0..3 of the row's column group); rows past m (up to the
        // padded 128) and blocks past K write 0
        uint32_t v = sc << (8 * lb);
        v |= __shfl_xor(v, 1);
        v |= __shfl_xor(v, 2);
        if (lb == 0 && in_k)
            *(uint32_t*)(p.out_sf + ((row >> 7) * p.nct + (cb >> 2)) * 512 + (row & 31) * 16 +
                         ((row & 127) >> 5) * 4) = v;


        // ---- the projection's input, the plain products x * pqs (no
        // nan_to_num) as hi + lo, into the wave's buffers; rows past m and
        // columns past K are 0
        // (PREP: x itself, the smoothing being in the weight)
        uint32_t ph[8], pl[8];
#pragma unroll
        for (int jj = 0; jj < 8; jj++) {
            const uint32_t xw = raw[jj >> 2][jj & 3], pw = pqb[jj >> 2][jj & 3];
            if constexpr (PREP) {
                ph[jj] = blk_ok ? xw : 0u;
            } else {
                const f32x2 prod = {bf16_lo(xw) * bf16_lo(pw), bf16_hi(xw) * bf16_hi(pw)};
                const bf16x2 hv = __builtin_convertvector(prod, bf16x2);  // RNE
                const f32x2 rest = {prod[0] - (float)hv[0], prod[1] - (float)hv[1]};
                ph[jj] = blk_ok ? __builtin_bit_cast(uint32_t, hv) : 0u;
                pl[jj] = blk_ok ? __builtin_bit_cast(uint32_t, __builtin_convertvector(rest, bf16x2)) : 0u;
            }
        }
        u32x4* dh = (u32x4*)(bhi + lr * XP + lb * 16);
        dh[0] = u32x4{ph[0], ph[1], ph[2], ph[3]};
        dh[1] = u32x4{ph[4], ph[5], ph[6], ph[7]};
        if constexpr (!PREP) {
            u32x4* dl = (u32x4*)(blo + lr * XP + lb * 16);
            dl[0] = u32x4{pl[0], pl[1], pl[2], pl[3]};
            dl[1] = u32x4{pl[4], pl[5], pl[6], pl[7]};
        }
        // the wave's own writes, read back by other lanes of the wave: LDS
        // accesses of one wave execute in order; keep the compiler from
        // moving them across
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

        // ---- project this wave's slices of the chunk
#pragma unroll
        for (int j = 0; j < SPW; j++) {
            if ((int64_t)c * kLoraChunk + wave * kLoraSlab + j * 32 >= p.K) break;  // uniform in the wave
            const int js = PREFETCH ? j : 0;
            if constexpr (!PREFETCH) load_slice(c, j, bf[0]);
            const int off = r16 * XP + j * 32 + kg * 8;
            const bf16x8 xh = __builtin_bit_cast(bf16x8, *(const u32x4*)(bhi + off));
            if constexpr (PREP) {
                // x against hi and against lo (x past K is 0; the weight
                // read there is column 0, finite)
#pragma unroll
                for (int i = 0; i < RT; i++)
#pragma unroll
                    for (int h = 0; h < 2; h++)
                        acc[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, bf[js][i][h]),
                                                                         xh, acc[i], 0, 0, 0);
            } else {
                const bool ok = slice_col(c, j) < p.K;
                const bf16x8 xl = __builtin_bit_cast(bf16x8, *(const u32x4*)(blo + off));
#pragma unroll
                for (int i = 0; i < RT; i++) {
                    const bf16x8 w = __builtin_bit_cast(bf16x8, ok ? bf[js][i][0] : u32x4{0u, 0u, 0u, 0u});
                    acc[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(w, xh, acc[i], 0, 0, 0);
                    acc[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(w, xl, acc[i], 0, 0, 0);
                }
            }
        }
        // the buffers are rewritten next chunk only after these reads
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        if constexpr (PREFETCH) load_proj(c + 1 < nch ? c + 1 : c, bf);
        raw[0] = nraw[0]; raw[1] = nraw[1];
        pqb[0] = npqb[0]; pqb[1] = npqb[1];
        if constexpr (DEEP) {
            nraw[0] = n2raw[0]; nraw[1] = n2raw[1];
            npqb[0] = n2pqb[0]; npqb[1] = n2pqb[1];
        }
    }
    __syncthreads();  // every wave is done with its buffers: the LDS now holds the waves' partial sums
    f32x4* const part = (f32x4*)xs;
    if (wave > 0)
#pragma unroll
        for (int i = 0; i < RT; i++) part[((wave - 1) * RT + i) * 64 + lane] = acc[i];
    __syncthreads();
    if (wave != 0) return;
    // lane: row m0 + r16, ranks 16 i + 4 kg .. + 3
    const int64_t orow = m0 + r16;
    if (orow >= p.m) return;
#pragma unroll
    for (int i = 0; i < RT; i++) {
        f32x4 v = acc[i];
        for (int w = 0; w < kLoraWaves - 1; w++) v += part[(w * RT + i) * 64 + lane];
        *(uint2*)(d_out + orow * rank + i * 16 + kg * 4) =
            uint2{f32_to_bf16_rne(v[0]) | (f32_to_bf16_rne(v[1]) << 16),
                  f32_to_bf16_rne(v[2]) | (f32_to_bf16_rne(v[3]) << 16)};
    }
}

// The prepared LoRA-down weight (flashinfer mm_nvfp4_svdquant, parameter d:
// the factor pqs[:, None] * L2^T) as two bf16 halves, hi = bf16 of pqs[k] *
// l2[p, k] (round to nearest even; the fp32 product of two bf16 values is
// exact) and lo = bf16 of that product minus hi (exact: at most 8
// significant bits remain), stored in the order k_quantize_lora<RT, true>
// reads them as MFMA operands: fragment (h, t, s) = half h, rank tile t (16
// ranks), slice s (32 columns) is 64 lanes x 8 bf16, lane l holding rank
// 16 t + l % 16 at columns 32 s + 8 (l / 16) .. + 7 (zero past K).  One
// thread per lane of a (t, s) fragment pair (hi and lo).
__global__ void k_lora_split(const uint16_t* pqs, const uint16_t* l2, uint16_t* w, int64_t rank, int64_t K) {
    const int64_t nsl = (K + 31) / 32, rt = rank / 16;
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;  // (t, s, lane)
    if (i >= rt * nsl * 64) return;
    const int lane = (int)(i & 63);
    const int64_t ts = i >> 6, t = ts / nsl, sl = ts - t * nsl;
    const int64_t row = t * 16 + (lane & 15), col = sl * 32 + (lane >> 4) * 8;
    u32x4 hi = u32x4{0u, 0u, 0u, 0u}, lo = hi;
    if (col < K) {  // K % 16 == 0: the 8 columns are all in or all out
        const u32x4 a = *(const u32x4*)(l2 + row * K + col);
        const u32x4 sc = *(const u32x4*)(pqs + col);
#pragma unroll
        for (int j = 0; j < 4; j++) {
            const float p0 = bf16_lo(a[j]) * bf16_lo(sc[j]), p1 = bf16_hi(a[j]) * bf16_hi(sc[j]);
            const uint32_t h = pack_bf16x2(p0, p1);
            hi[j] = h;
            lo[j] = pack_bf16x2(p0 - bf16_lo(h), p1 - bf16_hi(h));
        }
    }
    *(u32x4*)(w + ((t * nsl + sl) * 64 + lane) * 8) = hi;
    *(u32x4*)(w + (((rt + t) * nsl + sl) * 64 + lane) * 8) = lo;
}

hipError_t launch_lora_split(const uint16_t* pqs, const uint16_t* l2, uint16_t* w, int rank, int64_t K,
                             hipStream_t st) {
    const int64_t n = (int64_t)(rank / 16) * ((K + 31) / 32) * 64;
    k_lora_split<<<(unsigned)((n + 255) / 256), 256, 0, st>>>(pqs, l2, w, rank, K);
    return hipGetLastError();
}

// The flat amax pass's grid: one workgroup per 256 x 4 loads of 16 bytes, at
// most kFlatAmaxGrid; its partials go to ws, or (ws null) to the scale
// buffer, which then also bounds their number.
constexpr int kFlatAmaxGrid = kQuantizeWsFloats;

template <int V>
static void launch_amax_flat(QParams& p, float* ws, hipStream_t st) {
    constexpr int EPL = V == V_F32 || V == V_F32_SMOOTH ? 4 : 8;
    int64_t g = (p.m * p.K / EPL + 1023) / 1024;
    g = g < kFlatAmaxGrid ? g : kFlatAmaxGrid;
    if (!ws && g > p.sfsz / 4) g = p.sfsz / 4;
    p.nparts = (int)g;
    p.part = ws ? ws : (float*)p.out_sf;
    p.part_stride = 0;
    k_amax_flat<V><<<(unsigned)g, 256, 0, st>>>(p);
}

hipError_t launch_quantize_lora(const QuantizeArgs& a, const uint16_t* l2, uint16_t* d, int rank, bool prepared,
                                hipStream_t st) {
    QParams p{};
    p.x = a.x;
    p.pqs = (const uint16_t*)a.pqs;
    p.gs = a.gs;
    p.out_fp4 = a.out_fp4;
    p.out_sf = a.out_sf;
    p.m = a.m;
    p.K = a.k_in;
    p.k_in = a.k_in;
    p.nct = (int)((p.K + 63) / 64);
    p.nrt = (int)((p.m + 127) / 128);
    p.sfsz = (int64_t)p.nrt * 128 * p.nct * 4;
    p.b = 1;
    if (a.dynamic) {
        launch_amax_flat<V_BF16_SMOOTH>(p, nullptr, st);
        k_finish_gs<<<1, 256, 0, st>>>(p);
    }
    const dim3 grid((unsigned)(p.nrt * 8));  // 16-row bands over the padded rows (their scales are zeroed)
    constexpr int nt = 64 * kLoraWaves;
    if (prepared) {
        switch (rank / 16) {
        case 2: k_quantize_lora<2, true><<<grid, nt, 0, st>>>(p, l2, d, rank); break;
        case 4: k_quantize_lora<4, true><<<grid, nt, 0, st>>>(p, l2, d, rank); break;
        case 6: k_quantize_lora<6, true><<<grid, nt, 0, st>>>(p, l2, d, rank); break;
        default: k_quantize_lora<8, true><<<grid, nt, 0, st>>>(p, l2, d, rank); break;
        }
        return hipGetLastError();
    }
    switch (rank / 16) {
    case 2: k_quantize_lora<2, false><<<grid, nt, 0, st>>>(p, l2, d, rank); break;
    case 4: k_quantize_lora<4, false><<<grid, nt, 0, st>>>(p, l2, d, rank); break;
    case 6: k_quantize_lora<6, false><<<grid, nt, 0, st>>>(p, l2, d, rank); break;
    default: k_quantize_lora<8, false><<<grid, nt, 0, st>>>(p, l2, d, rank); break;
    }
    return hipGetLastError();
}

__global__ void k_alpha(const float* ga, const float* gb, float* alpha, int64_t n) {
    int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) alpha[i] = 1.0f / (ga[i] * gb[i]);
}

// ---------------------------------------------------------------------------
// host-side launch
// ---------------------------------------------------------------------------

// 64-column swizzle tiles per workgroup (CT), picked per pass and shape
// (measured): the amax pass reads best from many small workgroups (CT = 2);
// the quantize pass writes whole 128-byte lines of FP4 per row with CT = 4,
// which pays when it still leaves at least 1024 workgroups.  The silu
// variant reads gate and up and carries the silu work, so it keeps CT = 1.
template <int V>
static int quant_ct_for(const QParams& p) {
    if (V == V_SILU) return 1;
    const int64_t wgs4 = (int64_t)p.nrt * ((p.nct + 3) / 4) * p.b;
    return wgs4 >= 1024 ? 4 : 2;
}

template <int V, int CT>
static void launch_quantize_pass(const QParams& p, bool from_part, hipStream_t st) {
    const dim3 grid((p.nct + CT - 1) / CT, p.nrt, p.b);
    if (from_part) k_quantize<V, CT, true><<<grid, 256, 0, st>>>(p);
    else k_quantize<V, CT, false><<<grid, 256, 0, st>>>(p);
}

// ws: DYNAMIC mode's partial maxima (a caller workspace of at least
// kFlatAmaxGrid floats), or null.
// hbuf (silu only, with ws): room for h [b, m, K] bf16: the amax pass
// stores h there and the quantize pass reads it as a bf16 input.
template <int V>
static hipError_t launch_variant(QParams p, bool dynamic, float* ws, uint16_t* hbuf, hipStream_t st) {
    constexpr int CTA = V == V_SILU ? 1 : 2;
    // DYNAMIC mode on small items: one launch instead of three (a STATIC pass
    // is one launch anyway, and spreads over more compute units)
    if (dynamic && p.m * p.K <= fused_max_elems<V>()) {
        if constexpr (V == V_SILU) {
            k_quantize_fused<V, 1><<<dim3(p.nct, p.nrt, p.b), 256, 0, st>>>(p);
        } else {
            k_quantize_fused<V, 2><<<dim3((p.nct + 1) / 2, p.nrt, p.b), 256, 0, st>>>(p);
        }
        return hipGetLastError();
    }
    bool from_part = false;
    int ct = quant_ct_for<V>(p);
    if (dynamic) {
        if (V != V_SILU && p.b == 1 && !p.mask) {
            // one item read as a flat stream; with a workspace the quantize
            // pass reduces the partials itself
            launch_amax_flat<V>(p, ws, st);
            from_part = ws != nullptr;
        } else {
            // one amax workgroup, and one partial maximum, per amax tile:
            // into the workspace (the quantize pass then reduces an item's
            // partials itself) or into each item's own scale buffer
            p.nparts = p.nrt * ((p.nct + CTA - 1) / CTA);
            if (ws) {
                p.part = ws;
                p.part_stride = p.nparts;
                from_part = true;
            } else {
                p.part = (float*)p.out_sf;
                p.part_stride = p.sfsz / 4;
            }
            if constexpr (V == V_SILU) {
                if (ws && hbuf) {
                    // silu once: the amax pass stores h, then a bf16 pass over h
                    p.hbuf = hbuf;
                    k_amax<V, CTA, true><<<dim3(p.nparts, p.b), 256, 0, st>>>(p);
                    QParams q = p;
                    q.x = hbuf;
                    q.k_in = p.K;
                    const int qct = q.b * q.m * q.K * 2 <= ((int64_t)128 << 20) ? 2 : quant_ct_for<V_BF16>(q);
                    if (qct == 4) launch_quantize_pass<V_BF16, 4>(q, true, st);
                    else launch_quantize_pass<V_BF16, 2>(q, true, st);
                    return hipGetLastError();
                }
            }
            k_amax<V, CTA><<<dim3(p.nparts, p.b), 256, 0, st>>>(p);
        }
        if (!from_part) k_finish_gs<<<p.b, 256, 0, st>>>(p);
        // the amax pass has just brought an input of this size into the
        // Infinity Cache, from which the two-tile pass reads faster (measured)
        constexpr int64_t kWarmBytes = (int64_t)128 << 20;
        const int64_t in_bytes = p.b * p.m * p.k_in * (V == V_F32 || V == V_F32_SMOOTH ? 4 : 2);
        if (in_bytes <= kWarmBytes) ct = 2;
    }
    if constexpr (V == V_SILU) {
        launch_quantize_pass<V, 1>(p, from_part, st);
    } else {
        if (ct == 4) launch_quantize_pass<V, 4>(p, from_part, st);
        else launch_quantize_pass<V, 2>(p, from_part, st);
    }
    return hipGetLastError();
}

hipError_t launch_quantize(const QuantizeArgs& a, hipStream_t st) {
    QParams p{};
    p.x = a.x;
    p.pqs = (const uint16_t*)a.pqs;
    p.mask = a.mask;
    p.gs = a.gs;
    p.out_fp4 = a.out_fp4;
    p.out_sf = a.out_sf;
    p.m = a.m;
    p.K = a.silu ? a.k_in / 2 : a.k_in;
    p.k_in = a.k_in;
    p.nct = (int)((p.K + 63) / 64);
    p.nrt = (int)((p.m + 127) / 128);
    p.sfsz = (int64_t)p.nrt * 128 * p.nct * 4;
    p.b = (int)a.b;
    p.gs_other = a.gs_other;
    p.alpha_out = a.alpha_out;
    const bool dyn = a.dynamic;
    float* ws = a.ws;
    if (a.silu) return launch_variant<V_SILU>(p, dyn, ws, a.hbuf, st);
    if (a.x_dtype == 0) {
        if (a.pqs) return launch_variant<V_BF16_SMOOTH>(p, dyn, ws, nullptr, st);
        return launch_variant<V_BF16>(p, dyn, ws, nullptr, st);
    }
    if (a.pqs) return launch_variant<V_F32_SMOOTH>(p, dyn, ws, nullptr, st);
    return launch_variant<V_F32>(p, dyn, ws, nullptr, st);
}

// ---------------------------------------------------------------------------
// Allocation-free DYNAMIC quantization: the partial maxima that
// nvfp4_quantize_ws keeps in a caller workspace live in this file-scope
// device array instead, one copy per GPU, held until the process ends.  Its
// device address is looked up once per device (first call with that device
// current) and only that address is handed to kernels.  Every partial is
// written by the amax pass before the quantize pass reads it, so nothing
// needs clearing; calls that overlap on one GPU share the array and race.
// ---------------------------------------------------------------------------
static __device__ __align__(256) float scratch[kQuantizeWsFloats];

constexpr int kMaxDevices = 64;
static float* g_scratch_ptr[kMaxDevices];
static hipError_t g_scratch_err[kMaxDevices];
static std::once_flag g_scratch_once[kMaxDevices];

hipError_t scratch_for_current_device(float** ptr) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::call_once(g_scratch_once[dev], [dev] {
        void* p = nullptr;
        g_scratch_err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        g_scratch_ptr[dev] = (float*)p;
    });
    if (g_scratch_err[dev] != hipSuccess) return g_scratch_err[dev];
    if (!g_scratch_ptr[dev]) return hipErrorInvalidSymbol;
    *ptr = g_scratch_ptr[dev];
    return hipSuccess;
}

hipError_t launch_alpha(const float* ga, const float* gb, float* alpha, int64_t n, hipStream_t st) {
    int blocks = (int)((n + 255) / 256);
    k_alpha<<<blocks, 256, 0, st>>>(ga, gb, alpha, n);
    return hipGetLastError();
}

}  // namespace nvfp4
