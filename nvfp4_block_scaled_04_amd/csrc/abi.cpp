// abi.cpp -- the extern "C" entry points declared in include/nvfp4.h:
// argument validation (before anything is enqueued) and dispatch to the
// kernel launchers.  The library allocates no memory and keeps no state.
#include <hip/hip_runtime.h>

#include "../../include/nvfp4.h"
#include "internal.h"

namespace {

constexpr int64_t kMaxDim = (int64_t)1 << 30;

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

bool dim_ok(int64_t v) { return v >= 1 && v <= kMaxDim; }

int launch_status(hipError_t e) { return e == hipSuccess ? NVFP4_OK : NVFP4_LAUNCH_FAILED; }

// Sizes must keep every per-item element count and every grid dimension in
// range of the kernels' 32-bit tile indices.
bool quant_sizes_ok(int64_t b, int64_t m, int64_t K) {
    if (!dim_ok(b) || !dim_ok(m) || !dim_ok(K)) return false;
    if (b > 65535) return false;
    int64_t nrt = (m + 127) / 128, nct = (K + 63) / 64;
    if (nrt > 65535 || nct > ((int64_t)1 << 31) - 1) return false;
    if (nrt * nct > ((int64_t)1 << 31) - 1) return false;
    return true;
}

// Bytes of a swizzled scale buffer for `rows` rows of `nblk` blocks:
// pad_up(rows,128) * pad_up(nblk,4).  The GEMM kernels address a scale
// buffer through a 32-bit buffer descriptor with 32-bit signed per-step
// offsets, so each one must stay below 2^31 bytes.
bool gemm_sf_ok(int64_t rows, int64_t nblk) {
    return ((rows + 127) / 128 * 128) * ((nblk + 3) / 4 * 4) < ((int64_t)1 << 31);
}

}  // namespace

extern "C" {

static int quantize_check(const void* x, int x_dtype, int64_t m, int64_t k, const void* pre_quant_scale,
                          float* global_scale, int gs_mode, const float* gs_other, float* alpha,
                          uint8_t* out_fp4, uint8_t* out_sf) {
    if (!x || !global_scale || !out_fp4 || !out_sf) return NVFP4_NULL_POINTER;
    if (x_dtype != NVFP4_BF16 && x_dtype != NVFP4_F32) return NVFP4_BAD_DTYPE;
    if (gs_mode != NVFP4_GS_STATIC && gs_mode != NVFP4_GS_DYNAMIC) return NVFP4_UNSUPPORTED;
    if (k < 16 || k % 16 != 0 || !quant_sizes_ok(1, m, k)) return NVFP4_BAD_SHAPE;
    if (!aligned16(x) || !aligned16(out_fp4) || !aligned16(out_sf) ||
        (pre_quant_scale && !aligned16(pre_quant_scale)) || ((uintptr_t)global_scale & 3u) ||
        ((uintptr_t)gs_other & 3u) || ((uintptr_t)alpha & 3u))
        return NVFP4_MISALIGNED;
    return NVFP4_OK;
}

// Arguments already checked by quantize_check.
static int quantize_launch(const void* x, int x_dtype, int64_t m, int64_t k, const void* pre_quant_scale,
                           float* global_scale, int gs_mode, const float* gs_other, float* alpha,
                           uint8_t* out_fp4, uint8_t* out_sf, float* ws, void* stream) {
    nvfp4::QuantizeArgs a{};
    a.x = x; a.x_dtype = x_dtype; a.pqs = pre_quant_scale; a.mask = nullptr;
    a.gs = global_scale; a.out_fp4 = out_fp4; a.out_sf = out_sf;
    a.b = 1; a.m = m; a.k_in = k; a.silu = false; a.dynamic = gs_mode == NVFP4_GS_DYNAMIC;
    a.gs_other = gs_other; a.alpha_out = alpha;
    a.ws = a.dynamic ? ws : nullptr;
    return launch_status(nvfp4::launch_quantize(a, (hipStream_t)stream));
}

static int quantize_common(const void* x, int x_dtype, int64_t m, int64_t k, const void* pre_quant_scale,
                           float* global_scale, int gs_mode, const float* gs_other, float* alpha,
                           uint8_t* out_fp4, uint8_t* out_sf, float* ws, void* stream) {
    const int st = quantize_check(x, x_dtype, m, k, pre_quant_scale, global_scale, gs_mode, gs_other, alpha,
                                  out_fp4, out_sf);
    if (st != NVFP4_OK) return st;
    return quantize_launch(x, x_dtype, m, k, pre_quant_scale, global_scale, gs_mode, gs_other, alpha, out_fp4,
                           out_sf, ws, stream);
}

int nvfp4_quantize(const void* x, int x_dtype, int64_t m, int64_t k, const void* pre_quant_scale,
                   float* global_scale, int gs_mode, uint8_t* out_fp4, uint8_t* out_sf,
                   void* stream) {
    return quantize_common(x, x_dtype, m, k, pre_quant_scale, global_scale, gs_mode, nullptr, nullptr,
                           out_fp4, out_sf, nullptr, stream);
}

int nvfp4_quantize_alpha(const void* x, int x_dtype, int64_t m, int64_t k, const void* pre_quant_scale,
                         float* global_scale, int gs_mode, const float* gs_other, float* alpha,
                         uint8_t* out_fp4, uint8_t* out_sf, void* stream) {
    if (!gs_other || !alpha) return NVFP4_NULL_POINTER;
    return quantize_common(x, x_dtype, m, k, pre_quant_scale, global_scale, gs_mode, gs_other, alpha,
                           out_fp4, out_sf, nullptr, stream);
}

int nvfp4_quantize_ws(const void* x, int x_dtype, int64_t m, int64_t k, const void* pre_quant_scale,
                      float* global_scale, int gs_mode, const float* gs_other, float* alpha,
                      uint8_t* out_fp4, uint8_t* out_sf, void* workspace, int64_t workspace_bytes,
                      void* stream) {
    if (!gs_other != !alpha) return NVFP4_NULL_POINTER;
    if (gs_mode == NVFP4_GS_DYNAMIC) {
        if (!workspace) return NVFP4_NULL_POINTER;
        if (workspace_bytes < NVFP4_QUANTIZE_WS_BYTES) return NVFP4_BAD_SHAPE;
        if (!aligned16(workspace)) return NVFP4_MISALIGNED;
    }
    static_assert(NVFP4_QUANTIZE_WS_BYTES >= nvfp4::kQuantizeWsFloats * 4, "workspace holds the partials");
    return quantize_common(x, x_dtype, m, k, pre_quant_scale, global_scale, gs_mode, gs_other, alpha,
                           out_fp4, out_sf, (float*)workspace, stream);
}

int nvfp4_quantize_noalloc(const void* x, int x_dtype, int64_t m, int64_t k, const void* pre_quant_scale,
                           float* global_scale, int gs_mode, const float* gs_other, float* alpha,
                           uint8_t* out_fp4, uint8_t* out_sf, void* stream) {
    if (!gs_other != !alpha) return NVFP4_NULL_POINTER;
    // every argument is checked before the device is touched (symbol lookup)
    const int st = quantize_check(x, x_dtype, m, k, pre_quant_scale, global_scale, gs_mode, gs_other, alpha,
                                  out_fp4, out_sf);
    if (st != NVFP4_OK) return st;
    float* ws = nullptr;
    if (gs_mode == NVFP4_GS_DYNAMIC && nvfp4::scratch_for_current_device(&ws) != hipSuccess)
        return NVFP4_LAUNCH_FAILED;
    return quantize_launch(x, x_dtype, m, k, pre_quant_scale, global_scale, gs_mode, gs_other, alpha, out_fp4,
                           out_sf, ws, stream);
}

static int lora_down_common(const void* x, int64_t m, int64_t k, const void* pre_quant_scale, const void* l2,
                            int64_t r, float* global_scale, int gs_mode, uint8_t* out_fp4, uint8_t* out_sf, void* d,
                            bool prepared, void* stream) {
    if (!x || !pre_quant_scale || !l2 || !global_scale || !out_fp4 || !out_sf || !d) return NVFP4_NULL_POINTER;
    if (gs_mode != NVFP4_GS_STATIC && gs_mode != NVFP4_GS_DYNAMIC) return NVFP4_UNSUPPORTED;
    if (r <= 0 || r % 32 != 0 || r > 128) return NVFP4_BAD_RANK;
    if (k < 16 || k % 16 != 0 || !quant_sizes_ok(1, m, k)) return NVFP4_BAD_SHAPE;
    if (!aligned16(x) || !aligned16(pre_quant_scale) || !aligned16(l2) || !aligned16(out_fp4) ||
        !aligned16(out_sf) || !aligned16(d) || ((uintptr_t)global_scale & 3u))
        return NVFP4_MISALIGNED;
    nvfp4::QuantizeArgs a{};
    a.x = x; a.x_dtype = NVFP4_BF16; a.pqs = pre_quant_scale; a.mask = nullptr;
    a.gs = global_scale; a.out_fp4 = out_fp4; a.out_sf = out_sf;
    a.b = 1; a.m = m; a.k_in = k; a.silu = false; a.dynamic = gs_mode == NVFP4_GS_DYNAMIC;
    return launch_status(nvfp4::launch_quantize_lora(a, (const uint16_t*)l2, (uint16_t*)d, (int)r, prepared,
                                                      (hipStream_t)stream));
}

int nvfp4_quantize_lora_down(const void* x, int64_t m, int64_t k, const void* pre_quant_scale,
                             const void* l2, int64_t r, float* global_scale, int gs_mode, uint8_t* out_fp4,
                             uint8_t* out_sf, void* d, void* stream) {
    return lora_down_common(x, m, k, pre_quant_scale, l2, r, global_scale, gs_mode, out_fp4, out_sf, d, false,
                            stream);
}

int nvfp4_lora_down_prepare(const void* pre_quant_scale, const void* l2, int64_t r, int64_t k, void* w_out,
                            void* stream) {
    if (!pre_quant_scale || !l2 || !w_out) return NVFP4_NULL_POINTER;
    if (r <= 0 || r % 32 != 0 || r > 128) return NVFP4_BAD_RANK;
    if (k < 16 || k % 16 != 0 || !dim_ok(k)) return NVFP4_BAD_SHAPE;
    if (!aligned16(pre_quant_scale) || !aligned16(l2) || !aligned16(w_out)) return NVFP4_MISALIGNED;
    return launch_status(nvfp4::launch_lora_split((const uint16_t*)pre_quant_scale, (const uint16_t*)l2,
                                                  (uint16_t*)w_out, (int)r, k, (hipStream_t)stream));
}

int nvfp4_quantize_lora_down_prepared(const void* x, int64_t m, int64_t k, const void* pre_quant_scale,
                                      const void* w_prepared, int64_t r, float* global_scale, int gs_mode,
                                      uint8_t* out_fp4, uint8_t* out_sf, void* d, void* stream) {
    return lora_down_common(x, m, k, pre_quant_scale, w_prepared, r, global_scale, gs_mode, out_fp4, out_sf, d,
                            true, stream);
}

// The batched forms (k_in: the input row width, 2K for silu): every check of
// the call, then the launch; with_ws: the *_ws forms (gs_other / alpha and,
// in DYNAMIC mode, the workspace).
static int batched_common(const void* x, int64_t b, int64_t m, int64_t k_in, bool silu, const int32_t* mask,
                          float* global_scale, int gs_mode, const float* gs_other, float* alpha,
                          uint8_t* out_fp4, uint8_t* out_sf, bool with_ws, void* workspace,
                          int64_t workspace_bytes, void* stream) {
    if (!x || !global_scale || !out_fp4 || !out_sf) return NVFP4_NULL_POINTER;
    if (!gs_other != !alpha) return NVFP4_NULL_POINTER;
    if (gs_mode != NVFP4_GS_STATIC && gs_mode != NVFP4_GS_DYNAMIC) return NVFP4_UNSUPPORTED;
    int64_t k = k_in;
    if (silu) {
        if (k_in < 32 || k_in % 2 != 0 || (k_in / 2) % 16 != 0) return NVFP4_BAD_SHAPE;
        k = k_in / 2;
    }
    if (k < 16 || k % 16 != 0 || !quant_sizes_ok(b, m, k)) return NVFP4_BAD_SHAPE;
    const bool use_ws = with_ws && gs_mode == NVFP4_GS_DYNAMIC;
    if (use_ws) {
        if (!workspace) return NVFP4_NULL_POINTER;
        if (workspace_bytes < NVFP4_BATCHED_WS_BYTES(b, m, k)) return NVFP4_BAD_SHAPE;
    }
    if (!aligned16(x) || !aligned16(out_fp4) || !aligned16(out_sf) || ((uintptr_t)global_scale & 3u) ||
        ((uintptr_t)mask & 3u) || ((uintptr_t)gs_other & 3u) || ((uintptr_t)alpha & 3u) ||
        (use_ws && !aligned16(workspace)))
        return NVFP4_MISALIGNED;
    nvfp4::QuantizeArgs a{};
    a.x = x; a.x_dtype = NVFP4_BF16; a.pqs = nullptr; a.mask = mask;
    a.gs = global_scale; a.out_fp4 = out_fp4; a.out_sf = out_sf;
    a.b = b; a.m = m; a.k_in = k_in; a.silu = silu; a.dynamic = gs_mode == NVFP4_GS_DYNAMIC;
    a.gs_other = gs_other; a.alpha_out = alpha;
    a.ws = use_ws ? (float*)workspace : nullptr;
    // silu with room for h after the partials: silu is evaluated once
    if (silu && use_ws && workspace_bytes >= NVFP4_SILU_WS_BYTES(b, m, k))
        a.hbuf = (uint16_t*)((char*)workspace + (NVFP4_BATCHED_WS_BYTES(b, m, k) + 255) / 256 * 256);
    return launch_status(nvfp4::launch_quantize(a, (hipStream_t)stream));
}

static_assert(NVFP4_BATCHED_WS_BYTES(1, 1, 16) >= nvfp4::kQuantizeWsFloats * 4, "the flat amax pass's partials fit");

int nvfp4_quantize_masked_batched(const void* x, int64_t b, int64_t m, int64_t k,
                                  const int32_t* mask, float* global_scale, int gs_mode,
                                  uint8_t* out_fp4, uint8_t* out_sf, void* stream) {
    return batched_common(x, b, m, k, false, mask, global_scale, gs_mode, nullptr, nullptr, out_fp4, out_sf,
                          false, nullptr, 0, stream);
}

int nvfp4_quantize_masked_batched_ws(const void* x, int64_t b, int64_t m, int64_t k, const int32_t* mask,
                                     float* global_scale, int gs_mode, const float* gs_other, float* alpha,
                                     uint8_t* out_fp4, uint8_t* out_sf, void* workspace,
                                     int64_t workspace_bytes, void* stream) {
    return batched_common(x, b, m, k, false, mask, global_scale, gs_mode, gs_other, alpha, out_fp4, out_sf,
                          true, workspace, workspace_bytes, stream);
}

int silu_mul_nvfp4_quantize(const void* x, int64_t b, int64_t m, int64_t k2, const int32_t* mask,
                            float* global_scale, int gs_mode, uint8_t* out_fp4, uint8_t* out_sf,
                            void* stream) {
    return batched_common(x, b, m, k2, true, mask, global_scale, gs_mode, nullptr, nullptr, out_fp4, out_sf,
                          false, nullptr, 0, stream);
}

int silu_mul_nvfp4_quantize_ws(const void* x, int64_t b, int64_t m, int64_t k2, const int32_t* mask,
                               float* global_scale, int gs_mode, const float* gs_other, float* alpha,
                               uint8_t* out_fp4, uint8_t* out_sf, void* workspace, int64_t workspace_bytes,
                               void* stream) {
    return batched_common(x, b, m, k2, true, mask, global_scale, gs_mode, gs_other, alpha, out_fp4, out_sf,
                          true, workspace, workspace_bytes, stream);
}

static_assert(NVFP4_GEMM_WS_BYTES == nvfp4::kGemmWsBytes, "GEMM workspace size");

static int gemm_common(const uint8_t* a, const uint8_t* b, const uint8_t* a_sf, const uint8_t* b_sf,
                       const float* alpha, const int32_t* mask, const void* bias, const void* d,
                       const void* l1, void* out, int64_t E, int64_t m, int64_t n, int64_t k,
                       int64_t r, void* ws, int64_t ws_bytes, void* stream) {
    if (!a || !b || !a_sf || !b_sf || !alpha || !out) return NVFP4_NULL_POINTER;
    if (!dim_ok(E) || !dim_ok(m) || !dim_ok(n) || k < 16 || k % 16 != 0 || k > kMaxDim)
        return NVFP4_BAD_SHAPE;
    if (E > 65535 || ((m + 63) / 64) * ((n + 63) / 64) > ((int64_t)1 << 31) - 1) return NVFP4_BAD_SHAPE;
    // the GEMM kernels address one FP4 matrix with 32-bit byte offsets
    if (m * (k / 2) > ((int64_t)1 << 32) - 64 || n * (k / 2) > ((int64_t)1 << 32) - 64) return NVFP4_UNSUPPORTED;
    if (!gemm_sf_ok(m, k / 16) || !gemm_sf_ok(n, k / 16)) return NVFP4_UNSUPPORTED;
    if (!aligned16(a) || !aligned16(b) || !aligned16(a_sf) || !aligned16(b_sf) || !aligned16(out) ||
        ((uintptr_t)alpha & 3u) || (bias && !aligned16(bias)) || (d && !aligned16(d)) ||
        (l1 && !aligned16(l1)) || ((uintptr_t)mask & 3u))
        return NVFP4_MISALIGNED;
    if (ws && ws_bytes < NVFP4_GEMM_WS_BYTES) return NVFP4_BAD_SHAPE;
    if (ws && !aligned16(ws)) return NVFP4_MISALIGNED;
    nvfp4::GemmArgs g{};
    g.a = a; g.b = b; g.a_sf = a_sf; g.b_sf = b_sf; g.alpha = alpha; g.mask = mask;
    g.bias = (const uint16_t*)bias; g.d = (const uint16_t*)d; g.l1 = (const uint16_t*)l1;
    g.out = (uint16_t*)out; g.E = E; g.m = m; g.n = n; g.k = k; g.r = r;
    g.ws = (float*)ws;
    return launch_status(nvfp4::launch_gemm(g, (hipStream_t)stream));
}

int nvfp4_gemm(const uint8_t* a, const uint8_t* b, const uint8_t* a_sf, const uint8_t* b_sf,
               const float* alpha, const void* bias, void* out, int64_t m, int64_t n, int64_t k,
               void* stream) {
    return gemm_common(a, b, a_sf, b_sf, alpha, nullptr, bias, nullptr, nullptr, out, 1, m, n, k, 0,
                       nullptr, 0, stream);
}

int nvfp4_gemm_ws(const uint8_t* a, const uint8_t* b, const uint8_t* a_sf, const uint8_t* b_sf,
                  const float* alpha, const void* bias, void* out, int64_t m, int64_t n, int64_t k,
                  void* workspace, int64_t workspace_bytes, void* stream) {
    return gemm_common(a, b, a_sf, b_sf, alpha, nullptr, bias, nullptr, nullptr, out, 1, m, n, k, 0,
                       workspace, workspace_bytes, stream);
}

int nvfp4_gemm_grouped_masked(const uint8_t* a, const uint8_t* b, const uint8_t* a_sf,
                              const uint8_t* b_sf, const float* alpha, const int32_t* mask,
                              void* out, int64_t E, int64_t m, int64_t n, int64_t k, void* stream) {
    if (!mask) return NVFP4_NULL_POINTER;
    return gemm_common(a, b, a_sf, b_sf, alpha, mask, nullptr, nullptr, nullptr, out, E, m, n, k, 0,
                       nullptr, 0, stream);
}

int nvfp4_gemm_grouped_masked_ws(const uint8_t* a, const uint8_t* b, const uint8_t* a_sf,
                                 const uint8_t* b_sf, const float* alpha, const int32_t* mask,
                                 void* out, int64_t E, int64_t m, int64_t n, int64_t k,
                                 void* workspace, int64_t workspace_bytes, void* stream) {
    if (!mask) return NVFP4_NULL_POINTER;
    return gemm_common(a, b, a_sf, b_sf, alpha, mask, nullptr, nullptr, nullptr, out, E, m, n, k, 0,
                       workspace, workspace_bytes, stream);
}

int nvfp4_gemm_grouped_masked_silu_quantize(const uint8_t* a, const uint8_t* b, const uint8_t* a_sf,
                                            const uint8_t* b_sf, const float* alpha, const int32_t* mask,
                                            const float* global_scale, int64_t E, int64_t m, int64_t n2,
                                            int64_t k, uint8_t* out_fp4, uint8_t* out_sf, void* stream) {
    if (!a || !b || !a_sf || !b_sf || !alpha || !mask || !global_scale || !out_fp4 || !out_sf)
        return NVFP4_NULL_POINTER;
    if (!dim_ok(E) || !dim_ok(m) || !dim_ok(n2) || k < 16 || k % 16 != 0 || k > kMaxDim) return NVFP4_BAD_SHAPE;
    if (n2 % 2 != 0 || n2 / 2 < 16 || (n2 / 2) % 16 != 0 || !quant_sizes_ok(E, m, n2 / 2)) return NVFP4_BAD_SHAPE;
    if (E > 65535 || ((m + 127) / 128) * ((n2 / 2 + 63) / 64) > ((int64_t)1 << 31) - 1) return NVFP4_BAD_SHAPE;
    if (m * (k / 2) > ((int64_t)1 << 32) - 64 || n2 * (k / 2) > ((int64_t)1 << 32) - 64) return NVFP4_UNSUPPORTED;
    if (!gemm_sf_ok(m, k / 16) || !gemm_sf_ok(n2, k / 16)) return NVFP4_UNSUPPORTED;
    if (!aligned16(a) || !aligned16(b) || !aligned16(a_sf) || !aligned16(b_sf) || !aligned16(out_fp4) ||
        !aligned16(out_sf) || ((uintptr_t)alpha & 3u) || ((uintptr_t)mask & 3u) || ((uintptr_t)global_scale & 3u))
        return NVFP4_MISALIGNED;
    nvfp4::GemmArgs g{};
    g.a = a; g.b = b; g.a_sf = a_sf; g.b_sf = b_sf; g.alpha = alpha; g.mask = mask;
    g.E = E; g.m = m; g.n = n2; g.k = k;
    nvfp4::SiluQuantOut q{out_fp4, out_sf, global_scale};
    return launch_status(nvfp4::launch_gemm_silu_quantize(g, q, (hipStream_t)stream));
}

int nvfp4_gemm_svdquant(const uint8_t* a, const uint8_t* b, const uint8_t* a_sf, const uint8_t* b_sf,
                        const float* alpha, const void* d, const void* l1, const void* bias,
                        void* out, int64_t m, int64_t n, int64_t k, int64_t r, void* stream) {
    if (!d || !l1) return NVFP4_NULL_POINTER;
    if (r <= 0 || r % 32 != 0 || r > 4096) return NVFP4_BAD_RANK;
    return gemm_common(a, b, a_sf, b_sf, alpha, nullptr, bias, d, l1, out, 1, m, n, k, r, nullptr, 0, stream);
}

int nvfp4_gemm_svdquant_ws(const uint8_t* a, const uint8_t* b, const uint8_t* a_sf, const uint8_t* b_sf,
                           const float* alpha, const void* d, const void* l1, const void* bias,
                           void* out, int64_t m, int64_t n, int64_t k, int64_t r, void* workspace,
                           int64_t workspace_bytes, void* stream) {
    if (!d || !l1) return NVFP4_NULL_POINTER;
    if (r <= 0 || r % 32 != 0 || r > 4096) return NVFP4_BAD_RANK;
    return gemm_common(a, b, a_sf, b_sf, alpha, nullptr, bias, d, l1, out, 1, m, n, k, r, workspace,
                       workspace_bytes, stream);
}

int nvfp4_gemm_w4a16(const void* a, const uint8_t* b, const uint8_t* b_sf, const float* alpha,
                     const void* bias, void* out, int64_t m, int64_t n, int64_t k, void* stream) {
    if (!a || !b || !b_sf || !alpha || !out) return NVFP4_NULL_POINTER;
    if (!dim_ok(m) || !dim_ok(n) || k < 16 || k % 16 != 0 || k > kMaxDim) return NVFP4_BAD_SHAPE;
    if ((m + 15) / 16 > 65535 || (n + 15) / 16 > ((int64_t)1 << 31) - 1) return NVFP4_BAD_SHAPE;
    if (!aligned16(a) || !aligned16(b) || !aligned16(b_sf) || !aligned16(out) || ((uintptr_t)alpha & 3u) ||
        (bias && !aligned16(bias)))
        return NVFP4_MISALIGNED;
    nvfp4::GemmArgs g{};
    g.a = (const uint8_t*)a; g.b = b; g.b_sf = b_sf; g.alpha = alpha;
    g.bias = (const uint16_t*)bias; g.out = (uint16_t*)out;
    g.E = 1; g.m = m; g.n = n; g.k = k;
    return launch_status(nvfp4::launch_gemm_w4a16(g, (hipStream_t)stream));
}

int nvfp4_linear_small(const void* x, int64_t m, int64_t k, const uint8_t* b, const uint8_t* b_sf,
                       const float* gs_b, const void* bias, void* out, int64_t n, float* gs_out, void* stream) {
    if (!x || !b || !b_sf || !gs_b || !out) return NVFP4_NULL_POINTER;
    if (!dim_ok(m) || !dim_ok(n) || k < 16 || k % 16 != 0 || k > kMaxDim) return NVFP4_BAD_SHAPE;
    if (m > nvfp4::kLinearSmallMaxRows || k % 128 != 0 || k > nvfp4::kLinearSmallMaxK) return NVFP4_UNSUPPORTED;
    if ((n + 15) / 16 > ((int64_t)1 << 31) - 1 || !gemm_sf_ok(n, k / 16)) return NVFP4_BAD_SHAPE;
    if (!aligned16(x) || !aligned16(b) || !aligned16(b_sf) || !aligned16(out) || ((uintptr_t)gs_b & 3u) ||
        ((uintptr_t)gs_out & 3u) || (bias && !aligned16(bias)))
        return NVFP4_MISALIGNED;
    nvfp4::LinearSmallArgs a{};
    a.x = x; a.b = b; a.b_sf = b_sf; a.gs_b = gs_b; a.bias = (const uint16_t*)bias;
    a.out = (uint16_t*)out; a.gs_out = gs_out; a.m = m; a.n = n; a.k = k;
    return launch_status(nvfp4::launch_linear_small(a, (hipStream_t)stream));
}

int mxfp4_quantize(const void* x, int x_dtype, int64_t m, int64_t k, uint8_t* out_fp4, uint8_t* out_sf,
                   void* stream) {
    if (!x || !out_fp4 || !out_sf) return NVFP4_NULL_POINTER;
    if (x_dtype != NVFP4_BF16 && x_dtype != NVFP4_F32) return NVFP4_BAD_DTYPE;
    if (k < 32 || k % 32 != 0 || !quant_sizes_ok(1, m, k)) return NVFP4_BAD_SHAPE;
    if (!aligned16(x) || !aligned16(out_fp4) || !aligned16(out_sf)) return NVFP4_MISALIGNED;
    nvfp4::MxQuantizeArgs a{x, x_dtype, out_fp4, out_sf, m, k};
    return launch_status(nvfp4::launch_quantize_mx(a, (hipStream_t)stream));
}

int mxfp4_gemm(const uint8_t* a, const uint8_t* b, const uint8_t* a_sf, const uint8_t* b_sf, const float* alpha,
               const void* bias, void* out, int64_t m, int64_t n, int64_t k, void* stream) {
    if (!a || !b || !a_sf || !b_sf || !out) return NVFP4_NULL_POINTER;
    if (!dim_ok(m) || !dim_ok(n) || k < 32 || k % 32 != 0 || k > kMaxDim) return NVFP4_BAD_SHAPE;
    if (((m + 127) / 128) * ((n + 127) / 128) > ((int64_t)1 << 31) - 1) return NVFP4_BAD_SHAPE;
    if (m * (k / 2) > ((int64_t)1 << 32) - 64 || n * (k / 2) > ((int64_t)1 << 32) - 64) return NVFP4_UNSUPPORTED;
    if (!gemm_sf_ok(m, k / 32) || !gemm_sf_ok(n, k / 32)) return NVFP4_UNSUPPORTED;
    if (!aligned16(a) || !aligned16(b) || !aligned16(a_sf) || !aligned16(b_sf) || !aligned16(out) ||
        ((uintptr_t)alpha & 3u) || (bias && !aligned16(bias)))
        return NVFP4_MISALIGNED;
    nvfp4::GemmArgs g{};
    g.a = a; g.b = b; g.a_sf = a_sf; g.b_sf = b_sf; g.alpha = alpha;
    g.bias = (const uint16_t*)bias; g.out = (uint16_t*)out;
    g.E = 1; g.m = m; g.n = n; g.k = k;
    return launch_status(nvfp4::launch_gemm_mx(g, (hipStream_t)stream));
}

int nvfp4_alpha(const float* gs_a, const float* gs_b, float* alpha, int64_t count, void* stream) {
    if (!gs_a || !gs_b || !alpha) return NVFP4_NULL_POINTER;
    if (!dim_ok(count)) return NVFP4_BAD_SHAPE;
    if (((uintptr_t)gs_a & 3u) || ((uintptr_t)gs_b & 3u) || ((uintptr_t)alpha & 3u))
        return NVFP4_MISALIGNED;
    return launch_status(nvfp4::launch_alpha(gs_a, gs_b, alpha, count, (hipStream_t)stream));
}

}  // extern "C"
