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
// DYNAMIC mode runs three kernels on the caller's stream: a one-block clear
// of the accumulators, the amax pass (one atomic max per workgroup on the
// fp32 bit pattern, which orders non-negative floats, then the last workgroup
// to finish turns each amax into gs), and the quantize pass.
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
    uint32_t* counter;     // DYNAMIC: scratch word (first bytes of out_sf)
    int64_t m;             // rows per item
    int64_t K;             // quantized width
    int64_t k_in;          // input row stride in elements
    int64_t sfsz;          // per-item scale bytes
    int b;
    int nct;               // column tiles = ceil(K/64) = Cp/4
    int nrt;               // row tiles = ceil(m/128)
    int total_blocks;      // amax grid size (for the finish counter)
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

// Eight consecutive elements (row, col..col+7) of item e after the prologue
// and nan_to_num, plus their largest magnitude.
template <int V>
__device__ __forceinline__ Chunk load_chunk(const QParams& p, int64_t e, int64_t row, int64_t col) {
    Chunk c;
    const int64_t roff = (e * p.m + row) * p.k_in;
    if constexpr (V == V_BF16 || V == V_SILU) {
        uint32_t w[4];
        if constexpr (V == V_BF16) {
            uint4 v = *(const uint4*)((const uint16_t*)p.x + roff + col);
            w[0] = v.x; w[1] = v.y; w[2] = v.z; w[3] = v.w;
        } else {
            const uint16_t* xb = (const uint16_t*)p.x;
            uint4 gv = *(const uint4*)(xb + roff + col);
            uint4 uv = *(const uint4*)(xb + roff + p.K + col);
            uint32_t gw[4] = {gv.x, gv.y, gv.z, gv.w};
            uint32_t uw[4] = {uv.x, uv.y, uv.z, uv.w};
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
        uint32_t bad = 0;
        if constexpr (V == V_F32 || V == V_F32_SMOOTH) {
            const float* xf = (const float*)p.x + roff + col;
            float4 v0 = *(const float4*)xf;
            float4 v1 = *(const float4*)(xf + 4);
            c.f[0] = v0.x; c.f[1] = v0.y; c.f[2] = v0.z; c.f[3] = v0.w;
            c.f[4] = v1.x; c.f[5] = v1.y; c.f[6] = v1.z; c.f[7] = v1.w;
        } else {
            uint4 v = *(const uint4*)((const uint16_t*)p.x + roff + col);
            uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int j = 0; j < 4; j++) {
                c.f[2 * j] = bf16_lo(w[j]);
                c.f[2 * j + 1] = bf16_hi(w[j]);
            }
        }
        if constexpr (V == V_BF16_SMOOTH || V == V_F32_SMOOTH) {
            uint4 pv = *(const uint4*)(p.pqs + col);
            uint32_t pw[4] = {pv.x, pv.y, pv.z, pv.w};
#pragma unroll
            for (int j = 0; j < 4; j++) {
                c.f[2 * j] = c.f[2 * j] * bf16_lo(pw[j]);
                c.f[2 * j + 1] = c.f[2 * j + 1] * bf16_hi(pw[j]);
            }
        }
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

// ---------------------------------------------------------------------------
// DYNAMIC mode: clear, amax (+ finish), then quantize.
// ---------------------------------------------------------------------------

__global__ void k_clear_dynamic(float* gs, int b, uint32_t* counter) {
    for (int i = threadIdx.x; i < b; i += blockDim.x) gs[i] = 0.0f;
    if (threadIdx.x == 0) *counter = 0u;
}

template <int V>
__global__ __launch_bounds__(256) void k_amax(QParams p) {
    const int e = blockIdx.y;
    const int t = threadIdx.x;
    const int rho = t >> 3, l8 = t & 7;
    const int valid = clamp_rows(p.mask, e, (int)p.m);
    const int ntiles = p.nrt * p.nct;
    float amax = 0.0f;
    for (int tile = blockIdx.x; tile < ntiles; tile += gridDim.x) {
        const int rt = tile / p.nct, ct = tile - rt * p.nct;
        const int64_t col = (int64_t)ct * 64 + l8 * 8;
        if (col >= p.K) continue;
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const int64_t row = (int64_t)rt * 128 + rho + 32 * i;
            if (row < valid) {
                Chunk c = load_chunk<V>(p, e, row, col);
                amax = __builtin_fmaxf(amax, c.amax);
            }
        }
    }
    // workgroup max: wave reduction through shuffles, then LDS across waves
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) amax = __builtin_fmaxf(amax, __shfl_xor(amax, off));
    __shared__ float wmax[4];
    if ((t & 63) == 0) wmax[t >> 6] = amax;
    __syncthreads();
    if (t == 0) {
        float a = __builtin_fmaxf(__builtin_fmaxf(wmax[0], wmax[1]), __builtin_fmaxf(wmax[2], wmax[3]));
        atomicMax((unsigned int*)&p.gs[e], f_bits(a));
        __threadfence();
        unsigned int done = atomicAdd(p.counter, 1u);
        if (done == (unsigned int)p.total_blocks - 1u) {
            // last workgroup: every amax is final; turn each into gs
            __threadfence();
            for (int i = 0; i < p.b; i++) {
                float am = bits_f(atomicOr((unsigned int*)&p.gs[i], 0u));
                const float lo = 1e-12f;
                p.gs[i] = 2688.0f / (am < lo ? lo : am);
            }
        }
    }
}

template <int V>
__global__ __launch_bounds__(256) void k_quantize(QParams p) {
    const int ct = blockIdx.x, rt = blockIdx.y, e = blockIdx.z;
    const int t = threadIdx.x;
    const int rho = t >> 3, l8 = t & 7;
    const int valid = clamp_rows(p.mask, e, (int)p.m);
    const float gs = p.gs[e];
    const int64_t col = (int64_t)ct * 64 + l8 * 8;
    const bool col_ok = col < p.K;
    __shared__ __align__(16) uint8_t sbuf[512];
    uint8_t* q = p.out_fp4 + (int64_t)e * p.m * (p.K / 2);

#pragma unroll
    for (int i = 0; i < 4; i++) {
        const int64_t row = (int64_t)rt * 128 + rho + 32 * i;
        const bool active = col_ok && row < valid;
        Chunk c;
        if (active) {
            c = load_chunk<V>(p, e, row, col);
        } else {
#pragma unroll
            for (int j = 0; j < 8; j++) c.f[j] = 0.0f;
            c.amax = 0.0f;
        }
        // block amax over the lane pair sharing this 16-element block
        const float bamax = __builtin_fmaxf(c.amax, xor1(c.amax));
        const uint32_t s = ue4m3_encode((bamax / 6.0f) * gs);
        const float dec = ue4m3_decode(s);
        const float r = dec == 0.0f ? 0.0f : gs / dec;
        if (active) {
            uint32_t w = 0;
            w = NVFP4_PACK_FP4(w, c.f[0] * r, c.f[1] * r, 0);
            w = NVFP4_PACK_FP4(w, c.f[2] * r, c.f[3] * r, 1);
            w = NVFP4_PACK_FP4(w, c.f[4] * r, c.f[5] * r, 2);
            w = NVFP4_PACK_FP4(w, c.f[6] * r, c.f[7] * r, 3);
            *(uint32_t*)(q + row * (p.K / 2) + col / 2) = w;
        }
        if ((l8 & 1) == 0) sbuf[rho * 16 + i * 4 + (l8 >> 1)] = active ? (uint8_t)s : (uint8_t)0;
    }
    __syncthreads();
    if (t < 32) {
        uint8_t* dst = p.out_sf + (int64_t)e * p.sfsz + ((int64_t)rt * p.nct + ct) * 512 + t * 16;
        *(uint4*)dst = *(const uint4*)(sbuf + t * 16);
    }
}

__global__ void k_alpha(const float* ga, const float* gb, float* alpha, int64_t n) {
    int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) alpha[i] = 1.0f / (ga[i] * gb[i]);
}

// ---------------------------------------------------------------------------
// host-side launch
// ---------------------------------------------------------------------------

template <int V>
static hipError_t launch_variant(QParams p, bool dynamic, hipStream_t st) {
    if (dynamic) {
        k_clear_dynamic<<<1, 256, 0, st>>>(p.gs, p.b, p.counter);
        int ntiles = p.nrt * p.nct;
        int g = ntiles < 1024 ? ntiles : 1024;
        if (p.b > 1) {
            int per = (2048 + p.b - 1) / p.b;
            g = ntiles < per ? ntiles : per;
        }
        if (g < 1) g = 1;
        p.total_blocks = g * p.b;
        k_amax<V><<<dim3(g, p.b), 256, 0, st>>>(p);
    }
    k_quantize<V><<<dim3(p.nct, p.nrt, p.b), 256, 0, st>>>(p);
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
    p.counter = (uint32_t*)a.out_sf;
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
