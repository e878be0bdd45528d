// bench_issue_rate.hip -- standalone measurement (not part of the library):
// how much dequantization VALU work one SIMD can issue beside the fp16
// matrix pipe.  The NVFP4 GEMM feeds v_mfma_f32_32x32x16_f16 with operands
// dequantized in registers (per two elements: one FP4 -> fp16 convert and one
// packed fp16 multiply by the block scale), so its speed depends on how many
// such pairs fit beside each MFMA.
//
// Each kernel keeps 4 independent accumulators per wave and issues, after
// every MFMA, P independent (convert, multiply) pairs; the grid puts W waves
// on every SIMD of the chip.  Printed: ns per MFMA per SIMD for P = 0..6 and
// W = 1..4, and ns per pair with no MFMA.
//
// Build and run (gfx950):
//   hipcc --offload-arch=gfx950 -O3 -std=c++17 \
//     -Xclang -target-feature -Xclang -packed-fp32-ops \
//     nvfp4_block_scaled_04_amd/csrc/bench_issue_rate.hip -o /tmp/bench_issue_rate && /tmp/bench_issue_rate
#include <hip/hip_runtime.h>
#include <cstdint>
#include <cstdio>
#include <cstdlib>

#define CK(x)                                                                         \
    do {                                                                              \
        hipError_t e_ = (x);                                                          \
        if (e_ != hipSuccess) {                                                       \
            printf("HIP error %s at line %d\n", hipGetErrorString(e_), __LINE__);     \
            exit(1);                                                                  \
        }                                                                             \
    } while (0)

typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kIters = 2048;

// MFMA: 0 = pairs only (8 chains per wave), 1 = one MFMA then P pairs, repeated
template <int MFMA, int P>
__global__ __launch_bounds__(256) void k_issue(uint32_t* out, uint32_t seed) {
    const int gid = blockIdx.x * 256 + threadIdx.x;
    uint32_t w[8];
#pragma unroll
    for (int j = 0; j < 8; j++) w[j] = seed * (gid + 1) + j * 0x9E3779B9u;
    const _Float16 hm = (_Float16)(1.0f - (float)(seed & 3) * 0.0001f);  // a run-time scale
    const f16x2 sc = f16x2{hm, hm};
    f32x16 acc[4];
#pragma unroll
    for (int i = 0; i < 4; i++)
#pragma unroll
        for (int v = 0; v < 16; v++) acc[i][v] = 0.0f;
    const f16x8 a = f16x8{(_Float16)0.5f, 0, 0, 0, 0, 0, 0, (_Float16)0.25f};
    for (int it = 0; it < kIters; it++) {
        if constexpr (MFMA == 0) {
#pragma unroll
            for (int j = 0; j < 8; j++)
                w[j] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w[j], 1.0f, 0) * sc);
        } else {
#pragma unroll
            for (int i = 0; i < 4; i++) {
                acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, a, acc[i], 0, 0, 0);
#pragma unroll
                for (int j = 0; j < P; j++) {
                    const int jj = (i * P + j) & 7;
                    w[jj] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w[jj], 1.0f, 0) * sc);
                }
            }
        }
    }
    uint32_t s = 0;
#pragma unroll
    for (int j = 0; j < 8; j++) s ^= w[j];
#pragma unroll
    for (int i = 0; i < 4; i++) s ^= __builtin_bit_cast(uint32_t, acc[i][0]);
    out[gid] = s;  // one word per thread: the buffer holds blocks * 256
}

template <int MFMA, int P>
static float best_ms(uint32_t* out, int blocks) {
    hipEvent_t e0, e1;
    CK(hipEventCreate(&e0));
    CK(hipEventCreate(&e1));
    k_issue<MFMA, P><<<blocks, 256>>>(out, 1);
    CK(hipDeviceSynchronize());
    float best = 1e30f;
    for (int r = 0; r < 5; r++) {
        CK(hipEventRecord(e0));
        k_issue<MFMA, P><<<blocks, 256>>>(out, r + 2);
        CK(hipEventRecord(e1));
        CK(hipEventSynchronize(e1));
        float ms;
        CK(hipEventElapsedTime(&ms, e0, e1));
        best = ms < best ? ms : best;
    }
    CK(hipEventDestroy(e0));
    CK(hipEventDestroy(e1));
    return best;
}

int main() {
    int cus = 0;
    CK(hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, 0));
    printf("%d CUs; ns per MFMA per SIMD (v_mfma_f32_32x32x16_f16) with P (convert, multiply) pairs after each\n", cus);
    printf("waves/SIMD      P=0     P=1     P=2     P=3     P=4     P=5     P=6  | pairs alone, ns/pair\n");
    for (int wps = 1; wps <= 4; wps++) {
        const int blocks = cus * wps;  // 4 waves per block: wps waves on every SIMD
        uint32_t* out;
        CK(hipMalloc(&out, (size_t)blocks * 256 * sizeof(uint32_t)));
        const double mfmas = (double)kIters * 4 * wps;  // per SIMD
        const float t[7] = {best_ms<1, 0>(out, blocks), best_ms<1, 1>(out, blocks), best_ms<1, 2>(out, blocks),
                            best_ms<1, 3>(out, blocks), best_ms<1, 4>(out, blocks), best_ms<1, 5>(out, blocks),
                            best_ms<1, 6>(out, blocks)};
        const float tp = best_ms<0, 0>(out, blocks);
        printf("%d           ", wps);
        for (int p = 0; p < 7; p++) printf(" %7.2f", t[p] * 1e6 / mfmas);
        printf("  | %.2f\n", tp * 1e6 / ((double)kIters * 8 * wps));
        CK(hipFree(out));
    }
    return 0;
}
