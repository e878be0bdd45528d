// linear_small.hip -- the dynamic-scale NVFP4 linear for a few activation
// rows (decode) in one launch.
//
// What is computed: exactly nvfp4_quantize of x in DYNAMIC mode (FastVideo
// PR #1350 _global_sf: gs = 448*6 / amax; TensorRT-LLM
// NVFP4LinearMethod.create_weights: e2m1 values with an FP8 scale per 16
// elements), alpha = 1 / (gs * gs_w), then nvfp4_gemm of that activation
// against the NVFP4 weight (NVIDIA/Fuser PR #5737: dequantize, then a plain
// linear), out = bf16(alpha * acc (+ bias)).
//
// Why one launch: at m <= 16 both the quantization and the GEMM are short
// enough that a launch's fixed cost is most of their time.  Every workgroup
// reads the whole activation (at most 16 x 4096 bf16, 128 KB, from L2 after
// the first touch), forms the global amax and gs with the quantize kernels'
// own block functions, and quantizes the activation into LDS; the weight
// chunks its waves need are already in flight by then.  The K loop is the
// skinny GEMM's (a 16 x 16 output tile per workgroup, the K chunks split
// over eight waves, v_mfma_f32_16x16x32_f16 on exactly dequantized fp16
// operands, partial tiles added in wave order), so the output equals that
// of the separate quantize, alpha and GEMM calls bit for bit.
#include "device_common.h"
#include "gemm_common.h"
#include "internal.h"
#include "quant_block.h"

namespace nvfp4 {
namespace {

constexpr int kLsWaves = 8;        // waves of a workgroup (two per SIMD)
constexpr int kLsThreads = 64 * kLsWaves;

struct LParams {
    const uint16_t* x;     // [M, K] bf16
    const uint8_t* b;      // [N, K/2]
    const uint8_t* b_sf;   // swizzled, pad_up(N,128) * pad_up(K/16,4)
    const float* gs_b;     // [1]
    const uint16_t* bias;  // [N] or null
    uint16_t* out;         // [M, N]
    float* gs_out;         // [1] or null
    int64_t M, N, K;
    int cpa4;              // pad_up(K/16,4)/4 of the weight's scale layout
};

// JB: activation blocks per thread (16 rows x K/16 blocks over 512 threads).
template <int JB>
__global__ __launch_bounds__(kLsThreads) void k_linear_small(LParams p) {
#if defined(__HIP_DEVICE_COMPILE__)  // the host pass only needs the launch stub
    // the quantized activation in the K loop's lane order: chunk c (128
    // columns), lane l = row + 16 g holds columns 128c + 32g .. +31 of row
    // `row` as 16 FP4 bytes and their two block scales
    __shared__ __align__(16) uint8_t a_fp4[kLinearSmallMaxK * 8];
    __shared__ __align__(4) uint8_t a_sf[kLinearSmallMaxK];
    __shared__ f32x4 part[kLsWaves - 1][64];
    __shared__ float wmax[kLsWaves];

    const int t = threadIdx.x, lane = t & 63;
    const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
    const int64_t n0 = (int64_t)blockIdx.x * 16;
    const int64_t rowb = p.K / 2;
    const int r = lane & 15, g = lane >> 4;
    const int64_t brow = n0 + r < p.N ? n0 + r : p.N - 1;
    const uint8_t* B = p.b + brow * rowb;
    const int nch = (int)(p.K / 128);
    const int per = (nch + kLsWaves - 1) / kLsWaves;
    const int c0 = wave * per, c1 = c0 + per < nch ? c0 + per : nch;

    // 1. the first chunks of this wave's weight rows, in flight during the
    //    activation's quantization
    constexpr int U = 4;  // chunks whose loads are in flight together
    u32x4 fb[U];
    uint32_t sb[U];
    auto load_b = [&](int cb) {
#pragma unroll
        for (int u = 0; u < U; u++) {
            int c = cb + u < c1 ? cb + u : c1 - 1;  // past the range: reload, never used
            c = c < 0 ? 0 : c;                      // a wave without chunks (nch < 8 waves)
            fb[u] = *(const u32x4*)(B + (int64_t)c * 64 + g * 16);
            sb[u] = *(const uint16_t*)(p.b_sf + scale_byte_off(brow, c * 8 + 2 * g, p.cpa4));
        }
    };
    load_b(c0);

    // 2. the activation: thread t owns the blocks of LDS slots s = t + 512 j
    //    (slot s = 2 (64 c + l) + half: chunk c, lane l = row + 16 g of the
    //    K loop, half of its 32 columns), so consecutive lanes write
    //    consecutive LDS bytes; block (row, 8c + 2g + half) of the 16 x K/16
    //    grid.  Rows past M read row M - 1 again and are not quantized.
    const int nbt = (int)p.K;  // slots = 16 rows x K/16 blocks
    auto slot_block = [&](int s_, int& row, int& kb) {
        const int l = (s_ >> 1) & 63;
        row = l & 15;
        kb = (s_ >> 7) * 8 + (l >> 4) * 2 + (s_ & 1);
    };
    u32x4 raw[JB][2];
    u32x4 pq[2] = {u32x4{0u, 0u, 0u, 0u}, u32x4{0u, 0u, 0u, 0u}};
#pragma unroll
    for (int j = 0; j < JB; j++) {
        int q = t + kLsThreads * j;
        q = q < nbt ? q : nbt - 1;
        int row, kb;
        slot_block(q, row, kb);
        row = row < p.M ? row : (int)p.M - 1;
        const u32x4* src = (const u32x4*)(p.x + (int64_t)row * p.K + (int64_t)kb * 16);
        raw[j][0] = src[0];
        raw[j][1] = src[1];
    }
    float am = 0.0f;
#pragma unroll
    for (int j = 0; j < JB; j++) {
        const int q = t + kLsThreads * j;
        int row, kb;
        slot_block(q, row, kb);
        float f[16];
        const float bm = process_block<V_BF16>(raw[j], pq, f);
        if (q < nbt && row < p.M) am = __builtin_fmaxf(am, bm);
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) am = __builtin_fmaxf(am, __shfl_xor(am, off));
    if (lane == 0) wmax[wave] = am;
    __syncthreads();
    am = wmax[0];
#pragma unroll
    for (int w = 1; w < kLsWaves; w++) am = __builtin_fmaxf(am, wmax[w]);
    const float lo = 1e-12f;
    const float gs = 2688.0f / (am < lo ? lo : am);  // 448 * 6 over the clamped amax
    const float alpha = 1.0f / (gs * p.gs_b[0]);
    if (blockIdx.x == 0 && t == 0 && p.gs_out) p.gs_out[0] = gs;

    // 3. quantize into LDS (rows past M: zero codes and scales); the two
    //    halves of a lane's 32 columns sit in neighbouring lanes, whose scale
    //    bytes leave as one 16-bit store
#pragma unroll
    for (int j = 0; j < JB; j++) {
        const int q = t + kLsThreads * j;  // the same for every lane of a wave: K is a multiple of 128
        int row, kb;
        slot_block(q, row, kb);
        uint32_t w0 = 0, w1 = 0, sc = 0;
        if (row < p.M) {
            float f[16];
            const float bm = process_block<V_BF16>(raw[j], pq, f);  // the block's maximum again
            sc = ue4m3_encode(div6(bm) * gs);
            const float dec = ue4m3_decode(sc);
            pack_block(f, dec == 0.0f ? 0.0f : gs / dec, w0, w1);
        }
        const uint32_t sc_next = (uint32_t)__shfl_xor((int)sc, 1);
        if (q < nbt) {
            *(u32x2*)(a_fp4 + q * 8) = u32x2{w0, w1};
            if ((q & 1) == 0) *(uint16_t*)(a_sf + q) = (uint16_t)(sc | (sc_next << 8));
        }
    }
    __syncthreads();

    // 4. the skinny GEMM's K loop, the activation from LDS
    f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
    for (int cb = c0; cb < c1; cb += U) {
        if (cb != c0) load_b(cb);
#pragma unroll
        for (int u = 0; u < U; u++) {
            if (cb + u >= c1) break;
            const int c = cb + u;
            const u32x4 fa = *(const u32x4*)(a_fp4 + (c * 64 + lane) * 16);
            const uint32_t sa = *(const uint16_t*)(a_sf + (c * 64 + lane) * 2);
            const f16x2 ssa = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(sa, 1.0f, false);
            const f16x2 ssb = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(sb[u], 1.0f, false);
#pragma unroll
            for (int jw = 0; jw < 4; jw++) {
                const f16x8 oa = dequant8(word(fa, jw), ssa[jw >> 1]);
                const f16x8 ob = dequant8(word(fb[u], jw), ssb[jw >> 1]);
                acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(ob, oa, acc, 0, 0, 0);
            }
        }
    }
    // 5. the waves' partial tiles, in wave order; lane: output row r,
    //    columns n0 + 4g .. n0 + 4g + 3
    if (wave > 0) part[wave - 1][lane] = acc;
    __syncthreads();
    if (wave != 0) return;
#pragma unroll
    for (int w = 0; w < kLsWaves - 1; w++) acc += part[w][lane];
    if (r >= p.M) return;
    uint16_t* O = p.out + (int64_t)r * p.N;
    const int64_t n = n0 + 4 * g;
    float y[4];
#pragma unroll
    for (int v = 0; v < 4; v++) {
        y[v] = alpha * acc[v];
        if (p.bias && n + v < p.N) y[v] += bf16_lo((uint32_t)p.bias[n + v]);
    }
    if ((p.N & 3) == 0 && n + 3 < p.N) {
        *(u32x2*)(O + n) = u32x2{pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3])};
    } else {
#pragma unroll
        for (int v = 0; v < 4; v++)
            if (n + v < p.N) O[n + v] = (uint16_t)pack_bf16x2(y[v], 0.0f);
    }
#endif
}

}  // namespace

hipError_t launch_linear_small(const LinearSmallArgs& a, hipStream_t st) {
    LParams p{};
    p.x = (const uint16_t*)a.x;
    p.b = a.b;
    p.b_sf = a.b_sf;
    p.gs_b = a.gs_b;
    p.bias = a.bias;
    p.out = a.out;
    p.gs_out = a.gs_out;
    p.M = a.m;
    p.N = a.n;
    p.K = a.k;
    p.cpa4 = (int)((a.k / 16 + 3) / 4);
    const dim3 grid((unsigned)((a.n + 15) / 16));
    const int64_t jb = (a.k + kLsThreads - 1) / kLsThreads;  // 16 * (K/16) blocks over the threads
    if (jb <= 1) k_linear_small<1><<<grid, kLsThreads, 0, st>>>(p);
    else if (jb <= 2) k_linear_small<2><<<grid, kLsThreads, 0, st>>>(p);
    else if (jb <= 4) k_linear_small<4><<<grid, kLsThreads, 0, st>>>(p);
    else k_linear_small<8><<<grid, kLsThreads, 0, st>>>(p);
    return hipGetLastError();
}

}  // namespace nvfp4
