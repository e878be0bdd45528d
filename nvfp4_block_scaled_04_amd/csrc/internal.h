// internal.h -- launcher interfaces between the C ABI (abi.cpp) and the
// kernels.  Arguments arrive here already validated.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nvfp4 {

struct QuantizeArgs {
    const void* x;
    int x_dtype;          // 0 bf16, 1 fp32
    const void* pqs;      // [K] bf16 or null
    const int32_t* mask;  // [b] or null
    float* gs;            // [b]
    uint8_t* out_fp4;
    uint8_t* out_sf;
    int64_t b, m, k_in;   // k_in: input row width (2*K for silu)
    bool silu;
    bool dynamic;
    const float* gs_other = nullptr;  // with alpha_out: [b] the other operand's global scales
    float* alpha_out = nullptr;       // [b] alpha = 1 / (gs * gs_other), or null
};

hipError_t launch_quantize(const QuantizeArgs& a, hipStream_t st);
// Smooth quantize of a bf16 [m, k] (a.pqs set, a.b = 1) with the LoRA-down
// projection d = bf16((x * pqs) @ l2^T), l2 bf16 [rank, k]; rank in
// {32, 64, 96, 128}, k <= 4096.
hipError_t launch_quantize_lora(const QuantizeArgs& a, const uint16_t* l2, uint16_t* d, int rank,
                                hipStream_t st);
hipError_t launch_alpha(const float* ga, const float* gb, float* alpha, int64_t n, hipStream_t st);

struct GemmArgs {
    const uint8_t* a;      // [E, m, k/2]
    const uint8_t* b;      // [E, n, k/2]
    const uint8_t* a_sf;   // [E, sfa]
    const uint8_t* b_sf;   // [E, sfb]
    const float* alpha;    // [E]
    const int32_t* mask;   // [E] or null
    const uint16_t* bias;  // [n] or null
    const uint16_t* d;     // [m, r] or null
    const uint16_t* l1;    // [n, r] or null
    uint16_t* out;         // [E, m, n]
    int64_t E, m, n, k, r;
};

hipError_t launch_gemm(const GemmArgs& g, hipStream_t st);
// Weight-only form: g.a is the bf16 activation [m, k] (a_sf unused).
hipError_t launch_gemm_w4a16(const GemmArgs& g, hipStream_t st);

// Grouped masked GEMM (g.n = 2H gate | up rows, g.out unused) whose output
// h is turned into silu(gate) * up and quantized to NVFP4 with the static
// per-expert global scales gs.
struct SiluQuantOut {
    uint8_t* fp4;     // [E, m, H/2]
    uint8_t* sf;      // [E, pad_up(m,128) * pad_up(H/16,4)]
    const float* gs;  // [E]
};
hipError_t launch_gemm_silu_quantize(const GemmArgs& g, const SiluQuantOut& q, hipStream_t st);

// MX setting (32-element blocks, ue8m0 scales, no global scale).
struct MxQuantizeArgs {
    const void* x;        // [m, k] bf16 or fp32
    int x_dtype;          // 0 bf16, 1 fp32
    uint8_t* out_fp4;     // [m, k/2]
    uint8_t* out_sf;      // [pad_up(m,128) * pad_up(k/32,4)]
    int64_t m, k;         // k % 32 == 0
};
hipError_t launch_quantize_mx(const MxQuantizeArgs& a, hipStream_t st);
// g.E = 1; g.alpha may be null (1.0); g.mask, g.d, g.l1 unused.
hipError_t launch_gemm_mx(const GemmArgs& g, hipStream_t st);

}  // namespace nvfp4
