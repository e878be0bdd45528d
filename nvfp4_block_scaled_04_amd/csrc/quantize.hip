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
// per-workgroup LDS table (dec(s) takes only the ue4m3 code values), so the
// only division per block is bamax / 6.  The scale bytes are gathered in LDS
// and written with 16-byte stores.
//
// DYNAMIC mode runs three kernels on the caller's stream: the amax pass (one
// workgroup per quantize tile, each writing its partial maximum into the
// call's own scale buffer, which is free until the quantize pass overwrites
// it and holds at least one float per tile), a one-block-per-item finish that
// reduces the partials and writes gs, and the quantize pass.  No atomics and
// no device-wide fences are involved.
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
    int amax_blocks;       // amax workgroups per item (partials per item)
    const float* gs_other; // [b] the GEMM partner's global scales, when alpha_out is set
    float* alpha_out;      // [b] or null: alpha = 1 / (gs * gs_other)
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

// Partial maxima of item e live at the start of its scale buffer.
__device__ __forceinline__ float* partials(const QParams& p, int e) {
    return (float*)(p.out_sf + (int64_t)e * p.sfsz);
}

// ---------------------------------------------------------------------------
// DYNAMIC mode: amax partials, finish, then quantize.
// ---------------------------------------------------------------------------

template <int V, int CT>
__global__ __launch_bounds__(256) void k_amax(QParams p) {
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
            const int64_t row = (int64_t)rt * 128 + rsub + TM::RPP * i;
            load_block<V>(p, e, row < p.m ? row : p.m - 1, col, raw[i]);
        }
#pragma unroll
        for (int i = 0; i < TM::NP; i++) {
            const int64_t row = (int64_t)rt * 128 + rsub + TM::RPP * i;
            float f[16];
            const float a = process_block<V>(raw[i], pq, f);
            if (col_ok && row < valid) amax = __builtin_fmaxf(amax, a);
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

// gs = 2688 / max(amax, 1e-12) in fp32 (448 * 6 over the clamped amax).
__device__ __forceinline__ float gs_from_amax(float am) {
    const float lo = 1e-12f;
    return 2688.0f / (am < lo ? lo : am);
}

// gs[e] = 2688 / max(amax_e, 1e-12) from item e's partial maxima.
__global__ __launch_bounds__(256) void k_finish_gs(QParams p) {
    const int e = blockIdx.x, t = threadIdx.x;
    const float* part = partials(p, e);
    float a = 0.0f;
    int i = t;
    for (; i + 768 < p.amax_blocks; i += 1024)  // four independent loads in flight
        a = __builtin_fmaxf(__builtin_fmaxf(a, __builtin_fmaxf(part[i], part[i + 256])),
                            __builtin_fmaxf(part[i + 512], part[i + 768]));
    for (; i < p.amax_blocks; i += 256) a = __builtin_fmaxf(a, part[i]);
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) a = __builtin_fmaxf(a, __shfl_xor(a, off));
    __shared__ float wmax[4];
    if ((t & 63) == 0) wmax[t >> 6] = a;
    __syncthreads();
    if (t == 0) p.gs[e] = gs_from_amax(__builtin_fmaxf(__builtin_fmaxf(wmax[0], wmax[1]), __builtin_fmaxf(wmax[2], wmax[3])));
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
        const int64_t row = (int64_t)rt * 128 + rsub + TM::RPP * i;
        load_block<V>(p, e, row < p.m ? row : p.m - 1, col, raw[i]);
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
        float f[16];
        const float bamax = process_block<V>(raw[i], pq, f);
        const uint32_t sc = active ? ue4m3_encode((bamax / 6.0f) * gs) : 0u;
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
        if (active) *(uint2*)(q + row * (p.K / 2) + col / 2) = uint2{w0, w1};
        sbuf[c * 512 + (rl & 31) * 16 + (rl >> 5) * 4 + blk] = (uint8_t)sc;
    }
    __syncthreads();
    for (int i = t; i < ntile_here * 32; i += 256) *(u32x4*)(sf_dst + i * 16) = *(const u32x4*)(sbuf + i * 16);
}

template <int V, int CT>
__global__ __launch_bounds__(256) void k_quantize(QParams p) {
    const int e = blockIdx.z;
    // gs[e] is final here (given, or written by the finish kernel before this pass)
    if (p.alpha_out && blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x == 0) write_alpha(p, e, p.gs[e]);
    quantize_tile<V, CT>(p, blockIdx.x, blockIdx.y, e, [&] { return p.gs[e]; });
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
// A workgroup of 16 waves owns 16 rows across the whole K.  Phase 1: each
// thread takes one 16-element block per 256-column chunk of a row, for up
// to four chunks (all its loads in flight before any use), quantizes them
// exactly as the smooth pass does, and parks the raw bf16 rows in LDS.
// Phase 2 runs v_mfma_f32_16x16x32_bf16 over K with x from LDS as the A
// operand and l2 * pqs as the B operand, read through the caches (every
// workgroup reads the same L2 and pqs) and split exactly into two bf16
// halves: the product of two bf16 values has at most 16 significant bits,
// its bf16 rounding hi takes the top 8 and the remainder lo = product - hi
// at most 8 more, so x * hi + x * lo is x * l2 * pqs with every product
// exact and only fp32 accumulation rounding.  The waves take interleaved
// 32-column slices; their partial projections are added through LDS and
// stored as bf16.
// ---------------------------------------------------------------------------

constexpr int kLoraMaxK = 4096;   // columns of the LDS copy
constexpr int kLoraWaves = 16;
constexpr int kLoraPerThread = kLoraMaxK / 256 / (kLoraWaves / 4);  // chunks per thread

template <int RT>  // rank tiles of 16
__global__ __launch_bounds__(64 * kLoraWaves) void k_quantize_lora(QParams p, const uint16_t* l2, uint16_t* d_out,
                                                                  int rank) {
    constexpr int NT = 64 * kLoraWaves;
    constexpr int PITCH = kLoraMaxK + 8;  // bf16 per LDS row (16 bytes of pad spread the banks)
    constexpr int U = RT <= 4 ? 2 : 1;    // projection slices whose operands load together
    static_assert((kLoraWaves - 1) * RT * 64 * 16 <= 16 * PITCH * 2, "partial sums fit in the LDS copy");
    typedef float f32x2 __attribute__((ext_vector_type(2)));
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    __shared__ __align__(16) uint16_t xs[16 * PITCH];
    __shared__ float rtab[128];
    const int t = threadIdx.x, lane = t & 63;
    const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
    const int64_t m0 = (int64_t)blockIdx.x * 16;
    const int cg = __builtin_amdgcn_readfirstlane(t >> 8);  // chunk group: chunks cg, cg + 4, ...
    const int rl = (t >> 4) & 15, bl = t & 15;             // row within the band, block within a chunk
    const int64_t row = m0 + rl;
    const bool row_ok = row < p.m;
    const int64_t rrow = row_ok ? row : p.m - 1;  // loads of rows past m read a valid row
    const int nbk = (int)(p.K / 16);
    const int nchunk = (nbk + 15) / 16;
    const int ks = (int)((p.K + 31) / 32) * 32;  // K rounded up to whole MFMA slices
    const int nsl = ks / 32;
    const int nmine = (nsl - wave + kLoraWaves - 1) / kLoraWaves;  // projection slices of this wave
    const int r16 = lane & 15, kg = lane >> 4;
    const float gs = p.gs[0];
    if (t < 128) {
        const float dec = ue4m3_decode((uint32_t)t);
        rtab[t] = dec == 0.0f ? 0.0f : gs / dec;
    }
    // zero the LDS copy's columns past K up to the last whole slice
    for (int i = t; i < 16 * (ks - (int)p.K); i += NT) {
        const int rr = i / (ks - (int)p.K), cc = (int)p.K + i % (ks - (int)p.K);
        xs[rr * PITCH + cc] = 0;
    }
    __syncthreads();

    // projection operands (l2 rows and pqs) of U slices; past this wave's
    // slices or past K: zeros
    u32x4 bf[U][RT], pf[U];
    auto load_group = [&](int g) {
#pragma unroll
        for (int u = 0; u < U; u++) {
            const int col = (wave + kLoraWaves * (g + u)) * 32 + kg * 8;
            const bool ok = g + u < nmine && col < p.K;
#pragma unroll
            for (int i = 0; i < RT; i++)
                bf[u][i] = ok ? *(const u32x4*)(l2 + (int64_t)(i * 16 + r16) * p.K + col) : u32x4{0u, 0u, 0u, 0u};
            pf[u] = ok ? *(const u32x4*)(p.pqs + col) : u32x4{0u, 0u, 0u, 0u};
        }
    };

    // ---- phase 1: quantize, keep the raw rows in LDS
    {
        u32x4 raw[kLoraPerThread][2], pqb[kLoraPerThread][2];
#pragma unroll
        for (int i = 0; i < kLoraPerThread; i++) {  // every load in flight before any use
            int cb = (cg + 4 * i) * 16 + bl;
            cb = cb < nbk ? cb : nbk - 1;
            const u32x4* src = (const u32x4*)((const uint16_t*)p.x + rrow * p.k_in + (int64_t)cb * 16);
            raw[i][0] = src[0];
            raw[i][1] = src[1];
            load_pqs<V_BF16_SMOOTH>(p, (int64_t)cb * 16, pqb[i]);
        }
        load_group(0);  // the first projection operands, behind the rows
        uint8_t* q = p.out_fp4;
#pragma unroll
        for (int i = 0; i < kLoraPerThread; i++) {
            const int c = cg + 4 * i;
            if (c >= nchunk) break;  // uniform in the wave
            const int cb = c * 16 + bl;  // block column
            const bool blk_ok = row_ok && cb < nbk;
            float f[16];
            const float bamax = process_block<V_BF16_SMOOTH>(raw[i], pqb[i], f);
            const uint32_t sc = blk_ok ? ue4m3_encode((bamax / 6.0f) * gs) : 0u;
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
            if (blk_ok) *(uint2*)(q + row * (p.K / 2) + (int64_t)cb * 8) = uint2{w0, w1};
            // the 4 scale bytes of a swizzle dword sit in 4 neighbouring lanes
            uint32_t v = sc << (8 * (bl & 3));
            v |= __shfl_xor(v, 1);
            v |= __shfl_xor(v, 2);
            if ((bl & 3) == 0 && cb < nbk)
                *(uint32_t*)(p.out_sf + ((row >> 7) * p.nct + (cb >> 2)) * 512 + (row & 31) * 16 +
                             ((row & 127) >> 5) * 4) = v;
            // the projection's A operand: the raw rows (the plain product
            // x * pqs enters the projection, no nan_to_num), 0 past m
            if (cb < nbk) {
                u32x4* dst = (u32x4*)(xs + rl * PITCH + cb * 16);
                dst[0] = row_ok ? raw[i][0] : u32x4{0u, 0u, 0u, 0u};
                dst[1] = row_ok ? raw[i][1] : u32x4{0u, 0u, 0u, 0u};
            }
        }
    }
    __syncthreads();

    // ---- phase 2: d = x @ (l2 * pqs)^T over K
    f32x4 acc[RT];
#pragma unroll
    for (int i = 0; i < RT; i++) acc[i] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    for (int g = 0; g < nmine; g += U) {
        if (g > 0) load_group(g);
#pragma unroll
        for (int u = 0; u < U; u++) {
            if (g + u >= nmine) break;
            const int col = (wave + kLoraWaves * (g + u)) * 32 + kg * 8;  // this lane's 8 columns of the slice
            const bf16x8 afr = __builtin_bit_cast(bf16x8, *(const u32x4*)(xs + r16 * PITCH + col));
#pragma unroll
            for (int i = 0; i < RT; i++) {
                uint32_t hi[4], lo[4];
#pragma unroll
                for (int j = 0; j < 4; j++) {
                    const f32x2 prod = {bf16_lo(bf[u][i][j]) * bf16_lo(pf[u][j]),
                                        bf16_hi(bf[u][i][j]) * bf16_hi(pf[u][j])};
                    const bf16x2 h = __builtin_convertvector(prod, bf16x2);
                    const f32x2 rest = {prod[0] - (float)h[0], prod[1] - (float)h[1]};
                    hi[j] = __builtin_bit_cast(uint32_t, h);
                    lo[j] = __builtin_bit_cast(uint32_t, __builtin_convertvector(rest, bf16x2));
                }
                acc[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                    __builtin_bit_cast(bf16x8, u32x4{hi[0], hi[1], hi[2], hi[3]}), afr, acc[i], 0, 0, 0);
                acc[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                    __builtin_bit_cast(bf16x8, u32x4{lo[0], lo[1], lo[2], lo[3]}), afr, acc[i], 0, 0, 0);
            }
        }
    }
    __syncthreads();  // the LDS copy is free: it now holds the waves' partial sums
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

hipError_t launch_quantize_lora(const QuantizeArgs& a, const uint16_t* l2, uint16_t* d, int rank,
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
        p.amax_blocks = p.nrt * ((p.nct + 1) / 2);
        k_amax<V_BF16_SMOOTH, 2><<<dim3(p.amax_blocks, 1), 256, 0, st>>>(p);
        k_finish_gs<<<1, 256, 0, st>>>(p);
    }
    const dim3 grid((unsigned)(p.nrt * 8));  // 16-row bands over the padded rows (their scales are zeroed)
    constexpr int nt = 64 * kLoraWaves;
    switch (rank / 16) {
    case 2: k_quantize_lora<2><<<grid, nt, 0, st>>>(p, l2, d, rank); break;
    case 4: k_quantize_lora<4><<<grid, nt, 0, st>>>(p, l2, d, rank); break;
    case 6: k_quantize_lora<6><<<grid, nt, 0, st>>>(p, l2, d, rank); break;
    default: k_quantize_lora<8><<<grid, nt, 0, st>>>(p, l2, d, rank); break;
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
static void launch_quantize_pass(const QParams& p, hipStream_t st) {
    k_quantize<V, CT><<<dim3((p.nct + CT - 1) / CT, p.nrt, p.b), 256, 0, st>>>(p);
}

template <int V>
static hipError_t launch_variant(QParams p, bool dynamic, hipStream_t st) {
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
    if (dynamic) {
        // one amax workgroup, and one partial maximum, per amax tile
        p.amax_blocks = p.nrt * ((p.nct + CTA - 1) / CTA);
        k_amax<V, CTA><<<dim3(p.amax_blocks, p.b), 256, 0, st>>>(p);
        k_finish_gs<<<p.b, 256, 0, st>>>(p);
    }
    if constexpr (V == V_SILU) {
        launch_quantize_pass<V, 1>(p, st);
    } else {
        if (quant_ct_for<V>(p) == 4) launch_quantize_pass<V, 4>(p, st);
        else launch_quantize_pass<V, 2>(p, st);
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
    if (a.silu) return launch_variant<V_SILU>(p, dyn, st);
    if (a.x_dtype == 0) {
        if (a.pqs) return launch_variant<V_BF16_SMOOTH>(p, dyn, st);
        return launch_variant<V_BF16>(p, dyn, st);
    }
    if (a.pqs) return launch_variant<V_F32_SMOOTH>(p, dyn, st);
    return launch_variant<V_F32>(p, dyn, st);
}

hipError_t launch_alpha(const float* ga, const float* gb, float* alpha, int64_t n, hipStream_t st) {
    int blocks = (int)((n + 255) / 256);
    k_alpha<<<blocks, 256, 0, st>>>(ga, gb, alpha, n);
    return hipGetLastError();
}

}  // namespace nvfp4
