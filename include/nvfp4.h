/*
 * nvfp4.h -- C ABI of the MI355X (gfx950) NVFP4 quantization and block-scaled
 * FP4 GEMM library (libnvfp4_amd.so).
 *
 * Formats (shared by every entry point):
 *   - e2m1 ("FP4"): 4-bit code, bit 3 = sign, magnitudes {0, 0.5, 1, 1.5, 2,
 *     3, 4, 6}.  Packed two per byte, element 2i in the low nibble of byte i.
 *     A matrix of `rows` x `k` elements is `rows` x `k/2` bytes, row-major
 *     (TensorRT-LLM NVFP4LinearMethod.create_weights: weight [out, in/2] of
 *     float4_e2m1x2; flashinfer mm_nvfp4_svdquant: a, b are (rows, k/2)
 *     uint8, row-major).
 *   - ue4m3 block scale: one byte per 16 consecutive elements of a row (the
 *     e4m3 layout with the sign bit 0; max 448), stored in the "128x4
 *     swizzled" padded layout (flashinfer mm_nvfp4_svdquant, parameter
 *     a_sf; TensorRT-LLM create_weights, weight_scale "Padding is
 *     required"): a buffer of pad_up(rows,128) * pad_up(k/16,4) bytes in
 *     which scale (r, c) sits at byte
 *        ((r/128)*(Cp/4) + c/4)*512 + (r%32)*16 + ((r%128)/32)*4 + c%4,
 *     Cp = pad_up(k/16,4).  Every padding byte is written as 0.
 *   - global scale gs: fp32, gs = 448*6 / max(amax, 1e-12) where amax is the
 *     largest |x| after NaN -> 0 and +-inf -> +-FLT_MAX (FastVideo PR #1350
 *     review thread, _global_sf; TensorRT-LLM input_scale comment).
 *   - block scale s = ue4m3((block_amax / 6) * gs), round-to-nearest-even,
 *     saturating at 448; element code = e2m1(x * (gs / dec(s))),
 *     round-to-nearest-even, saturating at 6 (0 when dec(s) = 0); all fp32.
 *   - alpha = 1 / (gs_a * gs_b) (TensorRT-LLM alpha comment: amax_in *
 *     amax_w / (448*6)^2).
 *
 * Conventions:
 *   - Every tensor pointer is a device pointer on the current HIP device and
 *     must be 16-byte aligned.  Outputs are caller-allocated; the library
 *     allocates and frees no memory and keeps no state between calls.
 *   - `stream` is a hipStream_t passed as void*; NULL means the default
 *     stream.  Calls only enqueue work and return (no host synchronisation).
 *   - Every argument is validated before anything is enqueued; on a non-zero
 *     status nothing has been written.  NVFP4_LAUNCH_FAILED reports an error
 *     from the HIP launch itself; device faults surface at the caller's next
 *     synchronisation, as for any HIP call.
 *   - Calls that overlap on the same buffers race like any kernels.
 *   - In DYNAMIC mode the call uses the first bytes of each item's out_sf
 *     region as scratch for partial maxima before it writes the scales
 *     (nvfp4_quantize_ws takes a workspace for them instead); out_sf and
 *     global_scale hold their final values when the call's work completes.
 *   - The *_ws GEMM calls take a caller-owned workspace for the partial sums
 *     of a split-tail schedule.
 */
#ifndef NVFP4_AMD_H
#define NVFP4_AMD_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum nvfp4_status {
    NVFP4_OK = 0,
    NVFP4_NULL_POINTER = 1,   /* a required pointer is NULL */
    NVFP4_BAD_SHAPE = 2,      /* a size is out of range or k % 16 != 0 */
    NVFP4_MISALIGNED = 3,     /* a pointer is not 16-byte aligned */
    NVFP4_BAD_RANK = 4,       /* svdquant rank r is not a positive multiple of 32 */
    NVFP4_BAD_DTYPE = 5,      /* unknown x_dtype */
    NVFP4_UNSUPPORTED = 6,    /* unknown gs_mode, or a size beyond the kernels' limits */
    NVFP4_LAUNCH_FAILED = 7   /* hipLaunchKernel (or hipGetLastError) failed */
};

enum nvfp4_dtype { NVFP4_BF16 = 0, NVFP4_F32 = 1 };
enum nvfp4_gs_mode {
    NVFP4_GS_STATIC = 0,      /* read global_scale[] (a calibrated input scale) */
    NVFP4_GS_DYNAMIC = 1      /* compute global_scale[] from the amax and write it */
};

static inline const char *nvfp4_status_string(int s)
{
    switch (s) {
    case NVFP4_OK: return "ok";
    case NVFP4_NULL_POINTER: return "null pointer";
    case NVFP4_BAD_SHAPE: return "bad shape";
    case NVFP4_MISALIGNED: return "pointer not 16-byte aligned";
    case NVFP4_BAD_RANK: return "rank must be a positive multiple of 32";
    case NVFP4_BAD_DTYPE: return "unknown dtype";
    case NVFP4_UNSUPPORTED: return "unsupported argument";
    case NVFP4_LAUNCH_FAILED: return "kernel launch failed";
    default: return "unknown status";
    }
}

/*
 * Quantize x [m, k] to NVFP4.
 *   x:               [m, k] row-major, bf16 (x_dtype 0) or fp32 (x_dtype 1).
 *   pre_quant_scale: NULL, or [k] bf16; x is multiplied by it element-wise in
 *                    fp32 before quantization (the SVDQuant smoothing folded
 *                    into quantization, flashinfer mm_nvfp4_svdquant,
 *                    parameter a).
 *   global_scale:    [1] fp32; read (STATIC) or written (DYNAMIC).
 *   out_fp4:         [m, k/2] bytes.
 *   out_sf:          pad_up(m,128)*pad_up(k/16,4) bytes, swizzled.
 * Requires m >= 1, k >= 16, k % 16 == 0.
 */
int nvfp4_quantize(const void *x, int x_dtype, int64_t m, int64_t k,
                   const void *pre_quant_scale, float *global_scale, int gs_mode,
                   uint8_t *out_fp4, uint8_t *out_sf, void *stream);

/*
 * nvfp4_quantize, plus the GEMM's alpha written by the same launch: once
 * this call's global scale is final, alpha[0] = 1 / (global_scale[0] *
 * gs_other[0]) in fp32, the value nvfp4_alpha(global_scale, gs_other)
 * writes (TensorRT-LLM create_weights, the alpha parameter: the product of
 * the two operands' dequantization scales).  For a dynamically quantized
 * activation, this saves the separate alpha launch before the GEMM.
 *   gs_other: [1] fp32 device pointer, read (the weight's global scale).
 *   alpha:    [1] fp32 device pointer, written.
 * Everything else, the bytes written and the errors are as nvfp4_quantize;
 * NVFP4_NULL_POINTER also for a NULL gs_other or alpha, NVFP4_MISALIGNED
 * when either is not 4-byte aligned.
 */
int nvfp4_quantize_alpha(const void *x, int x_dtype, int64_t m, int64_t k,
                         const void *pre_quant_scale, float *global_scale, int gs_mode,
                         const float *gs_other, float *alpha,
                         uint8_t *out_fp4, uint8_t *out_sf, void *stream);

/*
 * nvfp4_quantize / nvfp4_quantize_alpha with a caller workspace for the
 * DYNAMIC mode's partial maxima (FastVideo PR #1350 review thread,
 * _global_sf: the per-call global-amax step whose cost this reduces).
 * Without a workspace a dynamic call is three launches: the amax pass, a
 * one-workgroup reduction of its partial maxima (kept in out_sf) to the
 * global scale, and the quantize pass.  With one, the partials go to the
 * workspace and every quantize workgroup reduces them itself: two launches,
 * the same bytes.
 *   gs_other, alpha: both NULL (no alpha), or as nvfp4_quantize_alpha.
 *   workspace:       DYNAMIC mode: a device buffer of workspace_bytes >=
 *                    NVFP4_QUANTIZE_WS_BYTES, 16-byte aligned, owned by the
 *                    caller; its contents on entry are ignored and on exit
 *                    undefined.  Calls sharing a workspace must not overlap
 *                    (same stream, or ordered by events).  STATIC mode does
 *                    not touch it (it may be NULL).
 * Everything else, the bytes written and the errors are as
 * nvfp4_quantize_alpha; in DYNAMIC mode NVFP4_NULL_POINTER also for a NULL
 * workspace, NVFP4_BAD_SHAPE for workspace_bytes below
 * NVFP4_QUANTIZE_WS_BYTES, NVFP4_MISALIGNED for a workspace not 16-byte
 * aligned; NVFP4_NULL_POINTER when exactly one of gs_other and alpha is NULL.
 */
#define NVFP4_QUANTIZE_WS_BYTES 4096
int nvfp4_quantize_ws(const void *x, int x_dtype, int64_t m, int64_t k,
                      const void *pre_quant_scale, float *global_scale, int gs_mode,
                      const float *gs_other, float *alpha,
                      uint8_t *out_fp4, uint8_t *out_sf,
                      void *workspace, int64_t workspace_bytes, void *stream);

/*
 * nvfp4_quantize_ws without the workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc): the DYNAMIC mode's partial maxima go to
 * a static device array inside the library (NVFP4_QUANTIZE_WS_BYTES = 4 KiB
 * per GPU, held until the process ends; it holds the at most 1024 partials
 * of any call, so no size is refused for it).  Its address is looked up on
 * the first DYNAMIC call on each device, with that device current -- the
 * one piece of host state the library keeps.  The call allocates nothing.
 * Calls that overlap on one GPU (other streams, other threads) share the
 * array and race; serialise them.  Arguments, bytes written and errors are
 * those of nvfp4_quantize_ws (without the workspace checks);
 * NVFP4_LAUNCH_FAILED also when the array's address cannot be obtained.
 */
int nvfp4_quantize_noalloc(const void *x, int x_dtype, int64_t m, int64_t k,
                           const void *pre_quant_scale, float *global_scale, int gs_mode,
                           const float *gs_other, float *alpha,
                           uint8_t *out_fp4, uint8_t *out_sf, void *stream);

/*
 * Smooth quantization with the SVDQuant LoRA-down projection fused
 * (flashinfer docs, flashinfer.gemm.mm_nvfp4_svdquant: parameter a is x with
 * pre_quant_scale folded into its quantization, and d = x @ (pqs[:, None] *
 * L2^T) is the rank-r LoRA-down output): one read of x gives
 *   out_fp4, out_sf, global_scale  exactly as nvfp4_quantize(x, bf16,
 *                                  pre_quant_scale = pqs) would, and
 *   d = bf16(sum_k x[i,k] * pqs[k] * l2[p,k]), every product exact,
 *       accumulated in fp32.
 *   x: [m, k] bf16; pre_quant_scale: [k] bf16; l2: [r, k] bf16 (the LoRA-down
 *   weight, row-major); d: [m, r] bf16 (16-byte aligned, ready for
 *   nvfp4_gemm_svdquant).  The product x * pqs enters the projection as is
 *   (non-finite values propagate; only the quantization applies nan_to_num).
 * Requires r in {32, 64, 96, 128} (NVFP4_BAD_RANK otherwise), k >= 16,
 * k % 16 == 0.  Device pointers owned by
 * the caller; nothing is allocated.
 */
int nvfp4_quantize_lora_down(const void *x, int64_t m, int64_t k, const void *pre_quant_scale,
                             const void *l2, int64_t r, float *global_scale, int gs_mode,
                             uint8_t *out_fp4, uint8_t *out_sf, void *d, void *stream);

/*
 * Elements (bf16) of the prepared LoRA-down weight for rank r and width k:
 * two halves x r ranks x k rounded up to 32 columns.
 */
#define NVFP4_LORA_PREPARED_ELEMS(r, k) (2 * (int64_t)(r) * (((int64_t)(k) + 31) / 32 * 32))

/*
 * The LoRA-down weight with the smoothing folded in, prepared once for
 * nvfp4_quantize_lora_down_prepared (flashinfer docs,
 * flashinfer.gemm.mm_nvfp4_svdquant, parameter d: the factor
 * pqs[:, None] * L2^T is fixed once the layer is calibrated).  Each product
 * pqs[k] * l2[p, k] (exact in fp32) is written as two bf16 halves whose sum
 * is that product exactly:
 *   hi[p, k] = bf16(pqs[k] * l2[p, k])   (round to nearest even),
 *   lo[p, k] = bf16(pqs[k] * l2[p, k] - hi[p, k])   (exact).
 * w_out holds NVFP4_LORA_PREPARED_ELEMS(r, k) bf16 in the order the fused
 * kernel reads its MFMA operands: fragment (h, t, s) (h = 0 hi, 1 lo; rank
 * tile t of 16 ranks; column slice s of 32) starts at element
 * ((h * r/16 + t) * ceil(k/32) + s) * 512, and its element l * 8 + e
 * (l = 0..63, e = 0..7) is half h of rank 16 t + l % 16 at column
 * 32 s + 8 (l / 16) + e, or 0 where that column is >= k.
 *   pre_quant_scale: [k] bf16; l2: [r, k] bf16, row-major.
 * Exact while the products are finite and not below fp32's normal range.
 * Requires r in {32, 64, 96, 128} (NVFP4_BAD_RANK otherwise), k >= 16,
 * k % 16 == 0, 16-byte aligned pointers.  Device pointers owned by the
 * caller; nothing is allocated.
 */
int nvfp4_lora_down_prepare(const void *pre_quant_scale, const void *l2, int64_t r, int64_t k,
                            void *w_out, void *stream);

/*
 * nvfp4_quantize_lora_down with the weight from nvfp4_lora_down_prepare
 * (w_prepared: NVFP4_LORA_PREPARED_ELEMS(r, k) bf16) in place of l2: the
 * same out_fp4, out_sf and global_scale bytes, and
 * d = bf16(sum_k x[i,k] * (hi[p,k] + lo[p,k])), every product exact and
 * accumulated in fp32, so d meets the same bound against
 * sum_k x[i,k] * pqs[k] * l2[p,k].  x enters the projection as is
 * (non-finite values propagate).  Arguments, requirements and errors are
 * those of nvfp4_quantize_lora_down.
 */
int nvfp4_quantize_lora_down_prepared(const void *x, int64_t m, int64_t k, const void *pre_quant_scale,
                                      const void *w_prepared, int64_t r, float *global_scale, int gs_mode,
                                      uint8_t *out_fp4, uint8_t *out_sf, void *d, void *stream);

/*
 * Batched, optionally masked quantization (flashinfer PR #1774, the
 * nvfp4_batched_quantize op and its per-item global scale).
 *   x:            [b, m, k] bf16.
 *   mask:         NULL (all m rows valid) or [b] int32 valid-row counts,
 *                 clamped to [0, m]; rows >= mask[e] do not enter item e's
 *                 amax, their FP4 bytes are not written and their scale bytes
 *                 are written as 0.
 *   global_scale: [b] fp32, one per item (read or written).
 *   out_fp4:      [b, m, k/2];  out_sf: [b, pad_up(m,128)*pad_up(k/16,4)].
 * Requires b >= 1, m >= 1, k >= 16, k % 16 == 0.
 */
int nvfp4_quantize_masked_batched(const void *x, int64_t b, int64_t m, int64_t k,
                                  const int32_t *mask, float *global_scale, int gs_mode,
                                  uint8_t *out_fp4, uint8_t *out_sf, void *stream);

/*
 * silu_and_mul fused before batched, optionally masked quantization
 * (flashinfer PR #1774, silu_and_mul_fp4_batched_quantize: a row of width
 * k2 = 2*h maps to h).  Gate is the first half of the row, up the second:
 *   h = bf16(fp32(silu(gate) * up)), silu(g) = g / (1 + e^-g) correctly
 *   rounded to fp32; h is then quantized as in nvfp4_quantize_masked_batched.
 *   x:       [b, m, k2] bf16;  out_fp4: [b, m, k2/4];
 *   out_sf:  [b, pad_up(m,128)*pad_up(k2/32,4)].
 * Requires k2 even and (k2/2) % 16 == 0.
 */
int silu_mul_nvfp4_quantize(const void *x, int64_t b, int64_t m, int64_t k2,
                            const int32_t *mask, float *global_scale, int gs_mode,
                            uint8_t *out_fp4, uint8_t *out_sf, void *stream);

/*
 * nvfp4_quantize_masked_batched and silu_mul_nvfp4_quantize with the two
 * additions of nvfp4_quantize_ws, per item:
 *   gs_other, alpha: both NULL, or [b] fp32 each: the GEMM partner's global
 *                    scales (read) and alpha[e] = 1 / (gs[e] * gs_other[e])
 *                    (written by the same call, from the final gs[e]).
 *   workspace:       DYNAMIC mode: a device buffer of workspace_bytes >=
 *                    NVFP4_BATCHED_WS_BYTES(b, m, k) (k: the quantized
 *                    width, k2/2 for the silu form), 16-byte aligned, owned
 *                    by the caller, contents ignored on entry and undefined
 *                    on exit; it receives the items' partial maxima, so the
 *                    amax pass and the quantize pass are the whole call (no
 *                    finishing launch, no separate alpha launch).  Calls
 *                    sharing a workspace must not overlap.  STATIC mode does
 *                    not touch it (it may be NULL).
 * The bytes written and the errors are those of the plain calls;
 * NVFP4_NULL_POINTER also when exactly one of gs_other and alpha is NULL or
 * when the workspace is NULL in DYNAMIC mode, NVFP4_BAD_SHAPE for a
 * workspace below the size above, NVFP4_MISALIGNED for a workspace not
 * 16-byte aligned or gs_other / alpha not 4-byte aligned.
 */
#define NVFP4_BATCHED_WS_BYTES(b, m, k) \
    (4096 + 4 * (int64_t)(b) * (((int64_t)(m) + 127) / 128) * (((int64_t)(k) + 63) / 64))
/*
 * silu_mul_nvfp4_quantize_ws with workspace_bytes >= NVFP4_SILU_WS_BYTES(b,
 * m, k) (k = k2/2) in DYNAMIC mode: the workspace also holds h = bf16(silu(g)
 * * u) of the valid rows, which the amax pass stores and the quantize pass
 * reads back, so silu is evaluated once instead of twice.  Same bytes out,
 * same errors; smaller workspaces (down to NVFP4_BATCHED_WS_BYTES) take the
 * two-evaluation path.
 */
#define NVFP4_SILU_WS_BYTES(b, m, k) \
    ((NVFP4_BATCHED_WS_BYTES(b, m, k) + 255) / 256 * 256 + 2 * (int64_t)(b) * (int64_t)(m) * (int64_t)(k))
int nvfp4_quantize_masked_batched_ws(const void *x, int64_t b, int64_t m, int64_t k,
                                     const int32_t *mask, float *global_scale, int gs_mode,
                                     const float *gs_other, float *alpha,
                                     uint8_t *out_fp4, uint8_t *out_sf,
                                     void *workspace, int64_t workspace_bytes, void *stream);
int silu_mul_nvfp4_quantize_ws(const void *x, int64_t b, int64_t m, int64_t k2,
                               const int32_t *mask, float *global_scale, int gs_mode,
                               const float *gs_other, float *alpha,
                               uint8_t *out_fp4, uint8_t *out_sf,
                               void *workspace, int64_t workspace_bytes, void *stream);

/*
 * out[m, n] = bf16(alpha * (A @ B^T) (+ bias[n])) with A [m, k] and B [n, k]
 * in NVFP4 (flashinfer mm_nvfp4_svdquant without the LoRA term; the FP4
 * linear of FastVideo PR #1350 and the scaled_mm of NVIDIA/Fuser PR #5737).
 *   a: [m, k/2], b: [n, k/2], a_sf / b_sf: swizzled scales of a / b.
 *   alpha: device fp32 scalar (numel >= 1).  bias: NULL or [n] bf16.
 *   out: [m, n] bf16, row-major.  Accumulation is fp32.
 * Requires m, n >= 1, k >= 16, k % 16 == 0.  Returns NVFP4_UNSUPPORTED when
 * an FP4 operand (per expert, for the grouped form) spans more than
 * 2^32 - 64 bytes (the kernels address a matrix with 32-bit offsets).
 */
int nvfp4_gemm(const uint8_t *a, const uint8_t *b, const uint8_t *a_sf, const uint8_t *b_sf,
               const float *alpha, const void *bias, void *out,
               int64_t m, int64_t n, int64_t k, void *stream);

/*
 * Grouped masked GEMM over E experts (flashinfer PR #1774: the quantized
 * batched outputs feed grouped_gemm_nt_masked): for each e and each row
 * i < mask[e] (clamped to [0, m]):
 *   out[e, i, :] = bf16(alpha[e] * (A[e] @ B[e]^T)[i, :]).
 *   a: [E, m, k/2]; b: [E, n, k/2]; a_sf: [E, pad_up(m,128)*pad_up(k/16,4)];
 *   b_sf: [E, pad_up(n,128)*pad_up(k/16,4)]; alpha, mask: [E] on device;
 *   out: [E, m, n] bf16, rows >= mask[e] are not written.
 */
int nvfp4_gemm_grouped_masked(const uint8_t *a, const uint8_t *b, const uint8_t *a_sf,
                              const uint8_t *b_sf, const float *alpha, const int32_t *mask,
                              void *out, int64_t E, int64_t m, int64_t n, int64_t k,
                              void *stream);

/*
 * Front half of a routed-expert SwiGLU in one launch (flashinfer PR #1774:
 * the gate_up grouped_gemm_nt_masked whose bf16 output feeds
 * silu_and_mul_scaled_nvfp4_experts_quantize with a given per-expert global
 * scale).  For each e and each row i < mask[e] (clamped to [0, m]):
 *   h[i, :]   = bf16(alpha[e] * (A[e] @ B[e]^T)[i, :])      (n2 = 2H columns)
 *   out[e, i] = NVFP4 quantize of bf16(silu(h[i, :H]) * h[i, H:]) with the
 *               static global scale global_scale[e],
 * bit for bit what nvfp4_gemm_grouped_masked followed by
 * silu_mul_nvfp4_quantize (STATIC mode) produce, without the bf16 h ever
 * reaching memory.
 *   a: [E, m, k/2]; b: [E, n2, k/2], gate rows [0, H) then up rows [H, 2H);
 *   a_sf: [E, pad_up(m,128)*pad_up(k/16,4)]; b_sf: [E, pad_up(n2,128)*
 *   pad_up(k/16,4)]; alpha, mask, global_scale: [E] on device (read only);
 *   out_fp4: [E, m, H/2], rows >= mask[e] not written; out_sf: [E,
 *   pad_up(m,128)*pad_up(H/16,4)] swizzled, fully written (masked rows and
 *   padding 0).  All pointers are device pointers owned by the caller.
 * Requires E, m >= 1, n2 even with H = n2/2 >= 16 and H % 16 == 0, k >= 16,
 * k % 16 == 0.  Returns NVFP4_NULL_POINTER, NVFP4_BAD_SHAPE,
 * NVFP4_MISALIGNED or NVFP4_UNSUPPORTED (as nvfp4_gemm) before launching
 * anything when an argument is invalid.
 */
int nvfp4_gemm_grouped_masked_silu_quantize(const uint8_t *a, const uint8_t *b, const uint8_t *a_sf,
                                            const uint8_t *b_sf, const float *alpha,
                                            const int32_t *mask, const float *global_scale,
                                            int64_t E, int64_t m, int64_t n2, int64_t k,
                                            uint8_t *out_fp4, uint8_t *out_sf, void *stream);

/*
 * SVDQuant fused GEMM (flashinfer docs, flashinfer.gemm.mm_nvfp4_svdquant):
 *   out = bf16(alpha * (A @ B^T + d @ l1^T) (+ bias)), the rank-r term
 *   added to the same fp32 accumulator after the NVFP4 K loop; l1 must be
 *   pre-divided by alpha by the caller so the term comes out unscaled.
 *   d: [m, r] bf16 (the LoRA-down output); l1: [n, r] bf16; bias: NULL or
 *   [n] bf16.  Requires r > 0 and r % 32 == 0.
 */
int nvfp4_gemm_svdquant(const uint8_t *a, const uint8_t *b, const uint8_t *a_sf,
                        const uint8_t *b_sf, const float *alpha, const void *d, const void *l1,
                        const void *bias, void *out, int64_t m, int64_t n, int64_t k, int64_t r,
                        void *stream);

/*
 * nvfp4_gemm, nvfp4_gemm_grouped_masked and nvfp4_gemm_svdquant with a
 * workspace for a split-tail schedule: when the output tiles do not divide
 * evenly over the CUs, the last tiles' K loops are split over all CUs and
 * their fp32 partial sums pass through the workspace (a second launch adds
 * them in a fixed order, so results are deterministic).  The results equal
 * the plain calls' up to the order of the fp32 accumulation (the sums of
 * split tiles are formed in a different order); every bar that holds for
 * the plain calls holds for these.  Without a workspace (NULL) the calls
 * behave as the plain ones.
 *   workspace: NULL, or a device buffer of workspace_bytes >=
 *              NVFP4_GEMM_WS_BYTES (32 MiB: one fp32 128x256 partial tile
 *              for each of up to 256 CUs), 16-byte aligned, owned by the
 *              caller; its contents on entry are ignored and on exit
 *              undefined.  Calls sharing a workspace must not overlap (same
 *              stream, or ordered by events).
 * Every other argument, the bytes written and the errors are those of the
 * plain call; NVFP4_BAD_SHAPE also for workspace_bytes below
 * NVFP4_GEMM_WS_BYTES and NVFP4_MISALIGNED for a workspace not 16-byte
 * aligned.
 */
#define NVFP4_GEMM_WS_BYTES 33554432
int nvfp4_gemm_ws(const uint8_t *a, const uint8_t *b, const uint8_t *a_sf, const uint8_t *b_sf,
                  const float *alpha, const void *bias, void *out,
                  int64_t m, int64_t n, int64_t k, void *workspace, int64_t workspace_bytes,
                  void *stream);
int nvfp4_gemm_grouped_masked_ws(const uint8_t *a, const uint8_t *b, const uint8_t *a_sf,
                                 const uint8_t *b_sf, const float *alpha, const int32_t *mask,
                                 void *out, int64_t E, int64_t m, int64_t n, int64_t k,
                                 void *workspace, int64_t workspace_bytes, void *stream);
int nvfp4_gemm_svdquant_ws(const uint8_t *a, const uint8_t *b, const uint8_t *a_sf,
                           const uint8_t *b_sf, const float *alpha, const void *d, const void *l1,
                           const void *bias, void *out, int64_t m, int64_t n, int64_t k, int64_t r,
                           void *workspace, int64_t workspace_bytes, void *stream);

/*
 * Weight-only GEMM (NVIDIA/Fuser PR #5737: f16a_nvfp4weight_scaled_mm, whose
 * eager meaning is the weight dequantized, then a plain linear with the
 * 16-bit activation):
 *   out = bf16(alpha * (A @ Bdq^T) (+ bias)),  Bdq = e2m1(b) * ue4m3(b_sf),
 * accumulated in fp32, alpha = 1 / the weight's global scale (nvfp4_alpha
 * with gs_a = 1 forms it on the device).  For decode, where the weight read
 * bounds the time and the activation is used as is, without quantization.
 *   a: [m, k] bf16 row-major, 16-byte aligned; b: [n, k/2] uint8 packed e2m1;
 *   b_sf: pad_up(n,128)*pad_up(k/16,4) ue4m3 in the 128x4 swizzled layout;
 *   alpha: device fp32 scalar; bias: NULL or [n] bf16; out: [m, n] bf16.
 * Requires m, n >= 1, k >= 16, k % 16 == 0.  All pointers are device
 * pointers owned by the caller; nothing is allocated.  Returns
 * NVFP4_NULL_POINTER, NVFP4_BAD_SHAPE or NVFP4_MISALIGNED before launching
 * anything when an argument is invalid.
 */
int nvfp4_gemm_w4a16(const void *a, const uint8_t *b, const uint8_t *b_sf, const float *alpha,
                     const void *bias, void *out, int64_t m, int64_t n, int64_t k, void *stream);

/*
 * Dynamic-scale NVFP4 linear for a few activation rows (decode), in one
 * launch.  The result is exactly that of three calls: nvfp4_quantize of x in
 * DYNAMIC mode (FastVideo PR #1350, _global_sf: gs = 448*6 / amax(x);
 * TensorRT-LLM NVFP4LinearMethod.create_weights: e2m1 with an FP8 scale per
 * 16 elements), alpha = 1 / (gs * gs_b) as nvfp4_alpha forms it, and
 * nvfp4_gemm of that activation against the NVFP4 weight (NVIDIA/Fuser PR
 * #5737: dequantize, then a plain linear):
 *   out = bf16(alpha * (Aq @ Bq^T) (+ bias)),
 * bit for bit.  The quantized activation itself stays on chip.
 *   x: [m, k] bf16 row-major, 16-byte aligned, 1 <= m <= 16;
 *   k: a multiple of 128, 128 <= k <= 4096;
 *   b: [n, k/2] uint8 packed e2m1; b_sf: pad_up(n,128)*pad_up(k/16,4) ue4m3
 *   in the 128x4 swizzled layout; gs_b: device fp32 [1], the weight's global
 *   scale; bias: NULL or [n] bf16; out: [m, n] bf16;
 *   gs_out: NULL, or device fp32 [1] that receives the activation's gs.
 * All pointers are device pointers owned by the caller; nothing is
 * allocated.  Returns NVFP4_NULL_POINTER, NVFP4_BAD_SHAPE, NVFP4_MISALIGNED,
 * or NVFP4_UNSUPPORTED for m > 16, k % 128 != 0 or k > 4096 (use the three
 * calls there), before launching anything.
 */
int nvfp4_linear_small(const void *x, int64_t m, int64_t k, const uint8_t *b, const uint8_t *b_sf,
                       const float *gs_b, const void *bias, void *out, int64_t n, float *gs_out,
                       void *stream);

/*
 * MX setting of the quantizer (flashinfer PR #1774: fp4_quantize's block
 * width and ue8m0 flags, there 16 / off; the other setting read as the OCP
 * Microscaling Formats v1.0 MXFP4 conversion): per 32 consecutive elements of
 * a row, after nan_to_num, the ue8m0 scale code 127 + floor(log2 amax) - 2
 * (clamped to [0, 254]; 0 for an all-zero block) and e2m1 codes of x / X,
 * X = 2^(code - 127), nearest even, saturating at 6.  No global scale.
 *   x: [m, k] bf16 or fp32 (x_dtype), row-major, 16-byte aligned.
 *   out_fp4: [m, k/2] uint8; out_sf: pad_up(m,128) * pad_up(k/32,4) bytes in
 *   the 128x4 swizzled layout over k/32 columns, fully written (padding 0).
 * Requires m >= 1, k >= 32, k % 32 == 0.  Returns NVFP4_NULL_POINTER,
 * NVFP4_BAD_DTYPE, NVFP4_BAD_SHAPE or NVFP4_MISALIGNED before launching
 * anything when an argument is invalid.
 */
int mxfp4_quantize(const void *x, int x_dtype, int64_t m, int64_t k, uint8_t *out_fp4, uint8_t *out_sf,
                   void *stream);

/*
 * MXFP4 GEMM: out[m, n] = bf16(alpha * (A @ B^T) (+ bias[n])) with A, B in
 * the layout mxfp4_quantize writes (dq = e2m1 * 2^(code - 127)), accumulated
 * in fp32 on gfx950's block-scaled MFMA.
 *   a: [m, k/2]; b: [n, k/2]; a_sf / b_sf: their MX scales; alpha: NULL
 *   (1.0) or a device fp32 scalar; bias: NULL or [n] bf16; out: [m, n] bf16.
 * Requires m, n >= 1, k >= 32, k % 32 == 0; NVFP4_UNSUPPORTED when an
 * operand spans more than 2^32 - 64 bytes.
 */
int mxfp4_gemm(const uint8_t *a, const uint8_t *b, const uint8_t *a_sf, const uint8_t *b_sf,
               const float *alpha, const void *bias, void *out, int64_t m, int64_t n, int64_t k,
               void *stream);

/*
 * alpha[i] = 1 / (gs_a[i] * gs_b[i]) in fp32 for i < count, on the device
 * (TensorRT-LLM create_weights, the alpha parameter).  Lets a caller that
 * quantizes activations in DYNAMIC mode form the GEMM's alpha without a host
 * round trip.  gs_a, gs_b, alpha: [count] fp32 device pointers.
 */
int nvfp4_alpha(const float *gs_a, const float *gs_b, float *alpha, int64_t count, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* NVFP4_AMD_H */
