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
// Work decomposition: one workgroup of 256 threads owns one 128-row x
// 64-column tile of the output, i.e. exactly one 512-byte tile of the
// swizzled scale layout.  Thread t handles rows (t/8) + 32*i, i = 0..3, and
// the 8 consecutive columns 8*(t%8).. of the tile, so a 16-element block is
// shared by a lane pair (block amax via one DPP exchange), and a wave reads
// 8 rows x 128 contiguous bytes per load.  The 512 scale bytes are gathered
// in LDS and written with 32 16-byte stores.
//
// DYNAMIC mode runs three kernels on the caller's stream: the amax pass, in
// which every workgroup writes its partial maximum into the call's own scale
// buffer (free until the quantize pass overwrites it; it holds at least one
// float per amax workgroup), a one-block-per-item finish that reduces the
// partials and writes gs, and the quantize pass.  No atomics and no
// device-wide fences are involved.
#include "device_common.h"
#include "internal.h"

namespace nvfp4 {

enum Variant { V_BF16 = 0, V_F32 = 1, V_BF16_SMOOTH = 2, V_F32_SMOOTH = 3, V_SILU = 4 };

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
    int nct;               // column tiles = ceil(K/64) = Cp/4
    int nrt;               // row tiles = ceil(m/128)
    int amax_blocks;       // amax workgroups per item (partials per item)
};

// silu(g) = g / (1 + e^-g), evaluated in fp64 and rounded once to fp32.
__device__ __forceinline__ float silu_f32(float g) {
    double x = (double)g;
    return (float)(x / (1.0 + exp(-x)));
}

struct Chunk {
    float f[8];
    float amax;
};

// Raw bytes behind eight consecutive elements: x (or the gate half) in `a`,
// the up half (silu) or the second 16 bytes of fp32 input in `b`.
struct Raw {
    uint4 a, b;
};

template <int V>
__device__ __forceinline__ Raw load_raw(const QParams& p, int64_t e, int64_t row, int64_t col) {
    Raw r;
    const int64_t roff = (e * p.m + row) * p.k_in;
    if constexpr (V == V_F32 || V == V_F32_SMOOTH) {
        const float* xf = (const float*)p.x + roff + col;
        r.a = *(const uint4*)xf;
        r.b = *(const uint4*)(xf + 4);
    } else if constexpr (V == V_SILU) {
        const uint16_t* xb = (const uint16_t*)p.x + roff;
        r.a = *(const uint4*)(xb + col);
        r.b = *(const uint4*)(xb + p.K + col);
    } else {
        r.a = *(const uint4*)((const uint16_t*)p.x + roff + col);
        r.b = uint4{0u, 0u, 0u, 0u};
    }
    return r;
}

// Eight elements after the prologue and nan_to_num, plus their largest
// magnitude.  pq holds the eight pre_quant_scale values (smooth variants).
template <int V>
__device__ __forceinline__ Chunk process(const Raw& raw, const uint4& pq) {
    Chunk c;
    if constexpr (V == V_BF16 || V == V_SILU) {
        uint32_t w[4];
        if constexpr (V == V_BF16) {
            w[0] = raw.a.x; w[1] = raw.a.y; w[2] = raw.a.z; w[3] = raw.a.w;
        } else {
            const uint32_t gw[4] = {raw.a.x, raw.a.y, raw.a.z, raw.a.w};
            const uint32_t uw[4] = {raw.b.x, raw.b.y, raw.b.z, raw.b.w};
#pragma unroll
            for (int j = 0; j < 4; j++) {
                float h0 = silu_f32(bf16_lo(gw[j])) * bf16_lo(uw[j]);
                float h1 = silu_f32(bf16_hi(gw[j])) * bf16_hi(uw[j]);
                w[j] = f32_to_bf16_rne(h0) | (f32_to_bf16_rne(h1) << 16);
            }
        }
        uint32_t mb = absmax_bits_bf16x8(w);
#pragma unroll
        for (int j = 0; j < 4; j++) {
            c.f[2 * j] = bf16_lo(w[j]);
            c.f[2 * j + 1] = bf16_hi(w[j]);
        }
        if (mb >= 0x7F80u) {  // inf or NaN present: the slow, exact path
            float a = 0.0f;
#pragma unroll
            for (int j = 0; j < 8; j++) {
                c.f[j] = nan_to_num(c.f[j]);
                a = __builtin_fmaxf(a, __builtin_fabsf(c.f[j]));
            }
            c.amax = a;
        } else {
            c.amax = bits_f(mb << 16);
        }
    } else {
        if constexpr (V == V_F32 || V == V_F32_SMOOTH) {
            const uint32_t w[8] = {raw.a.x, raw.a.y, raw.a.z, raw.a.w, raw.b.x, raw.b.y, raw.b.z, raw.b.w};
#pragma unroll
            for (int j = 0; j < 8; j++) c.f[j] = bits_f(w[j]);
        } else {
            const uint32_t w[4] = {raw.a.x, raw.a.y, raw.a.z, raw.a.w};
#pragma unroll
            for (int j = 0; j < 4; j++) {
                c.f[2 * j] = bf16_lo(w[j]);
                c.f[2 * j + 1] = bf16_hi(w[j]);
            }
        }
        if constexpr (V == V_BF16_SMOOTH || V == V_F32_SMOOTH) {
            const uint32_t pw[4] = {pq.x, pq.y, pq.z, pq.w};
#pragma unroll
            for (int j = 0; j < 4; j++) {
                c.f[2 * j] = c.f[2 * j] * bf16_lo(pw[j]);
                c.f[2 * j + 1] = c.f[2 * j + 1] * bf16_hi(pw[j]);
            }
        }
        uint32_t bad = 0;
        float a = 0.0f;
#pragma unroll
        for (int j = 0; j < 8; j++) {
            bad |= (f_bits(c.f[j]) & 0x7FFFFFFFu) >= 0x7F800000u;
            a = __builtin_fmaxf(a, __builtin_fabsf(c.f[j]));
        }
        if (bad) {
            a = 0.0f;
#pragma unroll
            for (int j = 0; j < 8; j++) {
                c.f[j] = nan_to_num(c.f[j]);
                a = __builtin_fmaxf(a, __builtin_fabsf(c.f[j]));
            }
        }
        c.amax = a;
    }
    return c;
}

template <int V>
__device__ __forceinline__ uint4 load_pqs(const QParams& p, int64_t col) {
    if constexpr (V == V_BF16_SMOOTH || V == V_F32_SMOOTH) return *(const uint4*)(p.pqs + col);
    return uint4{0u, 0u, 0u, 0u};
}

// ---------------------------------------------------------------------------
// DYNAMIC mode: amax partials, finish, then quantize.
// ---------------------------------------------------------------------------

// Thread layout of a workgroup tile of 128 rows x CT*64 columns (CT 64-column
// swizzle tiles): LPR = 8*CT lanes cover a row segment (8 elements each, a
// lane pair per 16-element block), RPP = 256/LPR rows are covered per pass,
// NP = 128/RPP passes.  A wave reads 64/LPR rows x 16*LPR contiguous bytes.
template <int CT>
struct TileMap {
    static constexpr int LPR = 8 * CT;
    static constexpr int RPP = 256 / LPR;
    static constexpr int NP = 128 / RPP;
};

// Partial maxima of item e live at the start of its scale buffer.
__device__ __forceinline__ float* partials(const QParams& p, int e) {
    return (float*)(p.out_sf + (int64_t)e * p.sfsz);
}

template <int V, int CT>
__global__ __launch_bounds__(256) void k_amax(QParams p) {
    using TM = TileMap<CT>;
    const int e = blockIdx.y;
    const int t = threadIdx.x;
    const int rsub = t / TM::LPR, lane = t % TM::LPR;
    const int valid = clamp_rows(p.mask, e, (int)p.m);
    const int nwct = (p.nct + CT - 1) / CT;
    const int ntiles = p.nrt * nwct;
    float amax = 0.0f;
    for (int tile = blockIdx.x; tile < ntiles; tile += gridDim.x) {
        const int rt = tile / nwct, wct = tile - rt * nwct;
        if ((int64_t)rt * 128 >= valid) continue;  // tile entirely past the valid rows
        int64_t col = (int64_t)wct * 64 * CT + lane * 8;
        const bool col_ok = col < p.K;
        col = col_ok ? col : p.K - 8;
        const uint4 pq = load_pqs<V>(p, col);
#pragma unroll
        for (int i0 = 0; i0 < TM::NP; i0 += 4) {
            Raw raw[4];
#pragma unroll
            for (int i = 0; i < 4; i++) {  // four loads in flight before any use
                const int64_t row = (int64_t)rt * 128 + rsub + TM::RPP * (i0 + i);
                raw[i] = load_raw<V>(p, e, row < p.m ? row : p.m - 1, col);
            }
#pragma unroll
            for (int i = 0; i < 4; i++) {
                const int64_t row = (int64_t)rt * 128 + rsub + TM::RPP * (i0 + i);
                if (col_ok && row < valid) amax = __builtin_fmaxf(amax, process<V>(raw[i], pq).amax);
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
        partials(p, e)[blockIdx.x] =
            __builtin_fmaxf(__builtin_fmaxf(wmax[0], wmax[1]), __builtin_fmaxf(wmax[2], wmax[3]));
}

// gs[e] = 2688 / max(amax_e, 1e-12) from item e's partial maxima.
__global__ __launch_bounds__(256) void k_finish_gs(QParams p) {
    const int e = blockIdx.x, t = threadIdx.x;
    const float* part = partials(p, e);
    float a = 0.0f;
    for (int i = t; i < p.amax_blocks; i += 256) a = __builtin_fmaxf(a, part[i]);
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) a = __builtin_fmaxf(a, __shfl_xor(a, off));
    __shared__ float wmax[4];
    if ((t & 63) == 0) wmax[t >> 6] = a;
    __syncthreads();
    if (t == 0) {
        const float am = __builtin_fmaxf(__builtin_fmaxf(wmax[0], wmax[1]), __builtin_fmaxf(wmax[2], wmax[3]));
        const float lo = 1e-12f;
        p.gs[e] = 2688.0f / (am < lo ? lo : am);
    }
}

template <int V, int CT>
__global__ __launch_bounds__(256) void k_quantize(QParams p) {
    using TM = TileMap<CT>;
    const int wct = blockIdx.x, rt = blockIdx.y, e = blockIdx.z;
    const int t = threadIdx.x;
    const int rsub = t / TM::LPR, lane = t % TM::LPR;
    const int c = lane >> 3;                 // swizzle tile within the workgroup
    const int blk = (lane & 7) >> 1;         // 16-element block within that tile
    const int valid = clamp_rows(p.mask, e, (int)p.m);
    const float gs = p.gs[e];
    int64_t col = (int64_t)wct * 64 * CT + lane * 8;
    const bool col_ok = col < p.K;
    col = col_ok ? col : p.K - 8;
    __shared__ __align__(16) uint8_t sbuf[512 * CT];
    uint8_t* q = p.out_fp4 + (int64_t)e * p.m * (p.K / 2);
    // swizzle tiles this workgroup owns that exist in the buffer
    const int ntile_here = (p.nct - wct * CT) < CT ? (p.nct - wct * CT) : CT;
    uint8_t* sf_dst = p.out_sf + (int64_t)e * p.sfsz + ((int64_t)rt * p.nct + (int64_t)wct * CT) * 512;

    if ((int64_t)rt * 128 >= valid) {  // tile entirely past the valid rows: zero scales only
        for (int i = t; i < ntile_here * 32; i += 256) *(uint4*)(sf_dst + i * 16) = uint4{0u, 0u, 0u, 0u};
        return;
    }
    const uint4 pq = load_pqs<V>(p, col);
#pragma unroll
    for (int i0 = 0; i0 < TM::NP; i0 += 4) {
        Raw raw[4];
#pragma unroll
        for (int i = 0; i < 4; i++) {  // four loads in flight before any use
            const int64_t row = (int64_t)rt * 128 + rsub + TM::RPP * (i0 + i);
            raw[i] = load_raw<V>(p, e, row < p.m ? row : p.m - 1, col);
        }
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const int rl = rsub + TM::RPP * (i0 + i);       // row within the 128-row tile
            const int64_t row = (int64_t)rt * 128 + rl;
            const bool active = col_ok && row < valid;
            Chunk ch;
            if (active) {
                ch = process<V>(raw[i], pq);
            } else {
#pragma unroll
                for (int j = 0; j < 8; j++) ch.f[j] = 0.0f;
                ch.amax = 0.0f;
            }
            // block amax over the lane pair sharing this 16-element block
            const float bamax = __builtin_fmaxf(ch.amax, xor1(ch.amax));
            const uint32_t sc = ue4m3_encode((bamax / 6.0f) * gs);
            const float dec = ue4m3_decode(sc);
            const float r = dec == 0.0f ? 0.0f : gs / dec;
            if (active) {
                uint32_t w = 0;
                w = NVFP4_PACK_FP4(w, ch.f[0] * r, ch.f[1] * r, 0);
                w = NVFP4_PACK_FP4(w, ch.f[2] * r, ch.f[3] * r, 1);
                w = NVFP4_PACK_FP4(w, ch.f[4] * r, ch.f[5] * r, 2);
                w = NVFP4_PACK_FP4(w, ch.f[6] * r, ch.f[7] * r, 3);
                *(uint32_t*)(q + row * (p.K / 2) + col / 2) = w;
            }
            if ((lane & 1) == 0)
                sbuf[c * 512 + (rl & 31) * 16 + (rl >> 5) * 4 + blk] = active ? (uint8_t)sc : (uint8_t)0;
        }
    }
    __syncthreads();
    for (int i = t; i < ntile_here * 32; i += 256) *(uint4*)(sf_dst + i * 16) = *(const uint4*)(sbuf + i * 16);
}

__global__ void k_alpha(const float* ga, const float* gb, float* alpha, int64_t n) {
    int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) alpha[i] = 1.0f / (ga[i] * gb[i]);
}

// ---------------------------------------------------------------------------
// host-side launch
// ---------------------------------------------------------------------------

// 64-column swizzle tiles per workgroup: two for the memory-bound variants
// (longer contiguous row segments per wave); one for the silu variant, whose
// fp64 silu makes it compute-heavy, so more workgroups pay off (measured).
template <int V>
constexpr int quant_ct() { return V == V_SILU ? 1 : 2; }

template <int V>
static hipError_t launch_variant(QParams p, bool dynamic, hipStream_t st) {
    constexpr int CT = quant_ct<V>();
    if (dynamic) {
        const int ntiles = p.nrt * ((p.nct + CT - 1) / CT);
        int g = (1024 + p.b - 1) / p.b;
        g = g < ntiles ? g : ntiles;
        p.amax_blocks = g < 1 ? 1 : g;
        k_amax<V, CT><<<dim3(p.amax_blocks, p.b), 256, 0, st>>>(p);
        k_finish_gs<<<p.b, 256, 0, st>>>(p);
    }
    k_quantize<V, CT><<<dim3((p.nct + CT - 1) / CT, p.nrt, p.b), 256, 0, st>>>(p);
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
