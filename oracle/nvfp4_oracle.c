/*
 * nvfp4_oracle.c -- plain, slow, obviously-correct CPU oracle for NVFP4
 * quantization and the block-scaled FP4 GEMM.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may include, link,
 * load or call this file: only tests/, __graft_entry__.smoke() and the
 * cpu_baseline leg of bench.py use it.  It shares no code, header, table or
 * constant generator with the HIP library; it is built with gcc and includes
 * no HIP header.
 *
 * Sources (the pages):
 *   [FV]  FastVideo PR #1350 "Add NVFP4QAT linear layer" -- review thread,
 *         the module-level _global_sf helper (amax with nan_to_num, clamp at
 *         1e-12, global scale 448*6/amax).
 *   [NVF] NVIDIA/Fuser PR #5737 "Benchmark for nvfp4 scaled mm" -- the eager
 *         op is "dequantize_to_dtype() then F.linear" (sequence diagram); the
 *         weight-only op f16a_nvfp4weight_scaled_mm takes a 16-bit activation,
 *         the FP4 weight, its block scales and its global scale.
 *   [FI]  flashinfer PR #1774 "Masked batch nvfp4 quantization" -- batched
 *         and masked quantize, silu_and_mul fused before quantize, per-item
 *         global scale (review comments on the test and the fake ops).
 *   [TRT] TensorRT-LLM v1.2.1 NVFP4LinearMethod.create_weights -- 16-element
 *         blocks, packed e2m1 weight [out, in/2], FP8 block scales padded to
 *         pad_up(rows,128) x pad_up(in/16,4), fp32 global scale 448*6/amax,
 *         alpha = amax_in*amax_w/(448*6)^2.
 *   [SVD] flashinfer docs, flashinfer.gemm.mm_nvfp4_svdquant -- out =
 *         alpha*(a@b^T) + d@l1^T [+bias]; a,b (rows, k/2) uint8 packed e2m1;
 *         ue4m3 scales in the 128x4 swizzled layout; l1 pre-divided by alpha.
 *
 * Readings taken where the pages are silent:
 *   - e2m1 and ue4m3 encoders round to nearest, ties to the even code, and
 *     saturate (6 and 448); the sign of zero is kept for e2m1.
 *   - ue4m3 is the OCP e4m3 bit layout with the sign bit 0 (bias 7,
 *     subnormals m*2^-9, max 448 = 0x7E); 0x7F is never produced.
 *   - block scale s = ue4m3((bamax / 6) * gs) and element v = x * (gs /
 *     dec(s)), all in fp32 (gs is fp32 on the pages); r = 0 when dec(s) = 0.
 *   - element 2i of a row goes to the low nibble of byte i.
 *   - the 128x4 swizzle: a 128-row x 4-scale-column tile is 512 contiguous
 *     bytes, 32 lines of 16; scale (r,c) sits at line r%32, dword
 *     (r%128)/32, byte c%4; tiles are row-tile-major.  Padding bytes are 0.
 *   - masked rows (r >= mask[e]) are excluded from amax, their FP4 bytes are
 *     not written and their scale bytes are 0.
 *   - silu(g) is rounded once to fp32 from a long-double evaluation; the
 *     gate is the first half of the row; h = bf16(fp32(silu(g) * u)).
 *   - pre_quant_scale multiplies x in fp32 with no intermediate rounding.
 *   - nan_to_num (NaN -> 0, +-inf -> +-FLT_MAX) is applied to the prologue
 *     output before everything else.
 *   - the MX setting of fp4_quantize's flags (32-element blocks, ue8m0
 *     scales) follows the OCP Microscaling Formats (MX) v1.0 conversion; see
 *     the MX section below.
 *
 * The GEMM accumulates in fp64 (products of two dequantized NVFP4 values are
 * exact in either precision); the pages leave the accumulation order free.
 * The weight-only GEMM multiplies the fp64 sum of activation x (e2m1 x
 * block scale) products by 1/global_scale once, where the pages' eager path
 * divides each dequantized weight and rounds it to bf16 first.
 * The GEMM's bf16 output (where a later step reads it back, as the
 * routed-expert gate_up output h does) is the exact fp64 value rounded to
 * fp32, the accumulator type, and then to bf16.
 */
#include <float.h>
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define NVO_OK 0
#define NVO_BAD 2

/* ------------------------------------------------------------------------ */
/* bf16 <-> fp32                                                             */
/* ------------------------------------------------------------------------ */

float nvo_bf16_to_f32(uint16_t h)
{
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

static uint32_t f32_bits(float f)
{
    uint32_t u;
    memcpy(&u, &f, 4);
    return u;
}

/* Round an fp32 value to the nearer of its two bf16 neighbours (the
 * truncation and the next code away from zero); on a tie take the one whose
 * last mantissa bit is 0.  NaN stays a quiet NaN. */
uint16_t nvo_f32_to_bf16(float f)
{
    uint32_t u = f32_bits(f);
    if (isnan(f))
        return (uint16_t)((u >> 16) | 0x0040);
    uint16_t lo = (uint16_t)(u >> 16);      /* toward zero   */
    if ((u & 0xFFFFu) == 0)
        return lo;                          /* exactly representable */
    uint16_t hi = (uint16_t)(lo + 1);       /* away from zero */
    double dv = fabs((double)f);
    double dlo = fabs((double)nvo_bf16_to_f32(lo));
    /* past the largest finite bf16 the next code is inf; for the distance
     * comparison it stands at 2^128, where the exponent range would put the
     * next value (round-to-nearest overflows to inf from the midpoint up) */
    double dhi = ((hi & 0x7FFF) == 0x7F80) ? ldexp(1.0, 128) : fabs((double)nvo_bf16_to_f32(hi));
    double elo = dv - dlo, ehi = dhi - dv;
    if (elo < ehi)
        return lo;
    if (ehi < elo)
        return hi;
    return (lo & 1) ? hi : lo;
}

/* ------------------------------------------------------------------------ */
/* e2m1 (FP4): sign bit 3, magnitude index in bits 0..2                      */
/* ------------------------------------------------------------------------ */

static const double E2M1_MAG[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};

double nvo_e2m1_value(uint8_t code)
{
    double v = E2M1_MAG[code & 7];
    return (code & 8) ? -v : v;
}

/* Nearest magnitude by exhaustive search, ties to the even index, saturating
 * at 6; the sign is taken from the sign bit of v (so -0 gives 0x8). */
uint8_t nvo_e2m1_encode(float v)
{
    if (isnan(v))
        return 0;
    uint8_t sign = signbit(v) ? 8 : 0;
    double a = fabs((double)v);
    if (a >= 6.0)
        return sign | 7;
    int best = 0;
    double bd = INFINITY;
    for (int i = 0; i < 8; i++) {
        double d = fabs(a - E2M1_MAG[i]);
        if (d < bd || (d == bd && (i & 1) == 0)) {
            bd = d;
            best = i;
        }
    }
    return (uint8_t)(sign | best);
}

/* ------------------------------------------------------------------------ */
/* ue4m3: e4m3 layout (bias 7) with the sign bit 0                           */
/* ------------------------------------------------------------------------ */

double nvo_ue4m3_value(uint8_t code)
{
    code &= 0x7F;
    if (code == 0x7F)
        return NAN;
    int e = code >> 3, m = code & 7;
    if (e == 0)
        return ldexp((double)m, -9);
    return ldexp(1.0 + m / 8.0, e - 7);
}

/* Nearest of the codes 0x00..0x7E by exhaustive search, ties to the even
 * code, saturating at 448 (0x7E).  Zero, negative and NaN inputs give 0. */
uint8_t nvo_ue4m3_encode(float v)
{
    if (!(v > 0.0f))
        return 0;
    double a = (double)v;
    if (a >= 448.0)
        return 0x7E;
    int best = 0;
    double bd = INFINITY;
    for (int c = 0; c <= 0x7E; c++) {
        double d = fabs(a - nvo_ue4m3_value((uint8_t)c));
        if (d < bd || (d == bd && (c & 1) == 0)) {
            bd = d;
            best = c;
        }
    }
    return (uint8_t)best;
}

/* ------------------------------------------------------------------------ */
/* scalar pieces of the method                                               */
/* ------------------------------------------------------------------------ */

static float nan_to_num(float v)
{
    if (isnan(v))
        return 0.0f;
    if (isinf(v))
        return v > 0 ? FLT_MAX : -FLT_MAX;
    return v;
}

/* [FV] _global_sf: gs = (448*6) / clamp(amax, min=1e-12), in fp32. */
float nvo_global_scale(float amax)
{
    float lo = 1e-12f;
    float a = amax < lo ? lo : amax;
    return 2688.0f / a;
}

/* silu(g) = g / (1 + e^-g), evaluated in long double and rounded once. */
float nvo_silu(float g)
{
    long double x = (long double)g;
    return (float)(x / (1.0L + expl(-x)));
}

int64_t nvo_pad_up(int64_t v, int64_t to) { return (v + to - 1) / to * to; }

/* [TRT] weight_scale numel = pad_up(rows,128) * pad_up(k/16,4); [SVD] a_sf
 * numel >= ceil(m/128)*128 * ceil(k/16/4)*4. */
int64_t nvo_sf_size(int64_t rows, int64_t k)
{
    return nvo_pad_up(rows, 128) * nvo_pad_up(k / 16, 4);
}

/* [SVD] "128x4 swizzled" layout; the permutation itself is a reading (see
 * the file header). */
int64_t nvo_sf_offset(int64_t r, int64_t c, int64_t k)
{
    int64_t cp = nvo_pad_up(k / 16, 4);
    return ((r / 128) * (cp / 4) + c / 4) * 512 + (r % 32) * 16 + ((r % 128) / 32) * 4 + (c % 4);
}

/* ------------------------------------------------------------------------ */
/* quantization                                                              */
/* ------------------------------------------------------------------------ */

enum { NVO_PRO_NONE = 0, NVO_PRO_SMOOTH = 1, NVO_PRO_SILU = 2 };

/* x' for element (row, col) of batch item e, before nan_to_num. */
static float prologue_value(const void *x, int x_dtype, int64_t row_off, int64_t col,
                            int64_t h, int prologue, const uint16_t *pqs)
{
    if (x_dtype == 1) {
        const float *xf = (const float *)x;
        float v = xf[row_off + col];
        if (prologue == NVO_PRO_SMOOTH)
            v = v * nvo_bf16_to_f32(pqs[col]);
        return v;
    }
    const uint16_t *xb = (const uint16_t *)x;
    if (prologue == NVO_PRO_SILU) {
        float g = nvo_bf16_to_f32(xb[row_off + col]);
        float u = nvo_bf16_to_f32(xb[row_off + h + col]);
        float p = nvo_silu(g) * u;
        return nvo_bf16_to_f32(nvo_f32_to_bf16(p));
    }
    float v = nvo_bf16_to_f32(xb[row_off + col]);
    if (prologue == NVO_PRO_SMOOTH)
        v = v * nvo_bf16_to_f32(pqs[col]);
    return v;
}

/*
 * Quantize b items of m rows each.  k_in is the input row width; the
 * quantized width is K = k_in (or k_in/2 for the silu prologue, whose row is
 * gate | up [FI]).  x_dtype: 0 bf16, 1 fp32 (fp32 only without silu).
 * mask: NULL (all m rows valid) or [b] int32 valid-row counts, clamped to
 * [0, m].  gs_mode: 0 STATIC reads gs[e]; 1 DYNAMIC writes gs[e] from the
 * amax of the valid rows [FV][FI].  out_fp4: [b, m, K/2], rows >= mask[e]
 * untouched.  out_sf: [b, sf_size(m, K)], fully written.
 */
int nvo_quantize(const void *x, int x_dtype, int64_t b, int64_t m, int64_t k_in, int prologue,
                 const uint16_t *pqs, const int32_t *mask, float *gs, int gs_mode,
                 uint8_t *out_fp4, uint8_t *out_sf)
{
    if (b < 1 || m < 0 || k_in < 1)
        return NVO_BAD;
    int64_t K = (prologue == NVO_PRO_SILU) ? k_in / 2 : k_in;
    if (prologue == NVO_PRO_SILU && (k_in % 2 != 0 || x_dtype != 0))
        return NVO_BAD;
    if (K % 16 != 0)
        return NVO_BAD;
    int64_t nblk = K / 16;
    int64_t sfsz = nvo_sf_size(m, K);

    for (int64_t e = 0; e < b; e++) {
        int64_t valid = m;
        if (mask) {
            valid = mask[e];
            if (valid < 0)
                valid = 0;
            if (valid > m)
                valid = m;
        }
        int64_t x_item = e * m * k_in;

        /* global scale */
        float g;
        if (gs_mode == 1) {
            float amax = 0.0f;
            for (int64_t r = 0; r < valid; r++)
                for (int64_t c = 0; c < K; c++) {
                    float v = nan_to_num(prologue_value(x, x_dtype, x_item + r * k_in, c, K, prologue, pqs));
                    float a = fabsf(v);
                    if (a > amax)
                        amax = a;
                }
            g = nvo_global_scale(amax);
            gs[e] = g;
        } else {
            g = gs[e];
        }

        uint8_t *sf = out_sf + e * sfsz;
        memset(sf, 0, (size_t)sfsz);
        uint8_t *q = out_fp4 + e * m * (K / 2);

#pragma omp parallel for schedule(static)
        for (int64_t r = 0; r < valid; r++) {
            float blk[16];
            uint8_t codes[16];
            for (int64_t kb = 0; kb < nblk; kb++) {
                float bamax = 0.0f;
                for (int j = 0; j < 16; j++) {
                    blk[j] = nan_to_num(prologue_value(x, x_dtype, x_item + r * k_in, kb * 16 + j, K, prologue, pqs));
                    float a = fabsf(blk[j]);
                    if (a > bamax)
                        bamax = a;
                }
                /* block scale: (bamax / 6) * gs, encoded saturating to ue4m3 */
                float t = bamax / 6.0f;
                float sfv = t * g;
                uint8_t s = nvo_ue4m3_encode(sfv);
                sf[nvo_sf_offset(r, kb, K)] = s;
                /* element multiplier r = gs / dec(s), or 0 for a zero scale */
                double ds = nvo_ue4m3_value(s);
                float mul = (ds == 0.0) ? 0.0f : g / (float)ds;
                for (int j = 0; j < 16; j++)
                    codes[j] = nvo_e2m1_encode(blk[j] * mul);
                for (int j = 0; j < 8; j++)
                    q[r * (K / 2) + kb * 8 + j] = (uint8_t)(codes[2 * j] | (codes[2 * j + 1] << 4));
            }
        }
    }
    return NVO_OK;
}

/* ------------------------------------------------------------------------ */
/* GEMM: dequantize, then a plain dot product ([NVF] eager semantics)        */
/* ------------------------------------------------------------------------ */

/* Dequantized element (row, col) of a packed NVFP4 matrix with K columns. */
static double dq(const uint8_t *p, const uint8_t *sf, int64_t row, int64_t col, int64_t K)
{
    uint8_t byte = p[row * (K / 2) + col / 2];
    uint8_t code = (col & 1) ? (byte >> 4) : (byte & 15);
    return nvo_e2m1_value(code) * nvo_ue4m3_value(sf[nvo_sf_offset(row, col / 16, K)]);
}

/*
 * For each requested row i of A (rows[j]), out[j, n] = alpha * (sum_k
 * Adq[i,k] * Bdq[n,k] + sum_p d[i,p] * l1[n,p]) + bias[n], in fp64, not
 * rounded to bf16.  d, l1 (bf16, rank r) and bias (bf16 [n]) may be NULL.
 * [SVD] out = alpha*(a@b^T) + d@l1^T [+bias] with l1 pre-divided by alpha,
 * i.e. alpha multiplies the whole accumulator.
 */
int nvo_gemm_rows(const uint8_t *a, const uint8_t *b, const uint8_t *a_sf, const uint8_t *b_sf,
                  float alpha, const uint16_t *bias, const uint16_t *d, const uint16_t *l1, int64_t r,
                  int64_t m, int64_t n, int64_t k, const int64_t *rows, int64_t nrows, double *out)
{
    if (k % 16 != 0 || m < 0 || n < 0)
        return NVO_BAD;
    for (int64_t j = 0; j < nrows; j++)
        if (rows[j] < 0 || rows[j] >= m)
            return NVO_BAD;
    double *bdq = (double *)malloc(sizeof(double) * (size_t)(n * k > 0 ? n * k : 1));
    if (!bdq)
        return NVO_BAD;
#pragma omp parallel for schedule(static)
    for (int64_t nn = 0; nn < n; nn++)
        for (int64_t kk = 0; kk < k; kk++)
            bdq[nn * k + kk] = dq(b, b_sf, nn, kk, k);

#pragma omp parallel
    {
        double *arow = (double *)malloc(sizeof(double) * (size_t)(k > 0 ? k : 1));
#pragma omp for schedule(dynamic, 1)
        for (int64_t j = 0; j < nrows; j++) {
            int64_t i = rows[j];
            for (int64_t kk = 0; kk < k; kk++)
                arow[kk] = dq(a, a_sf, i, kk, k);
            for (int64_t nn = 0; nn < n; nn++) {
                double acc = 0.0;
                const double *brow = bdq + nn * k;
                for (int64_t kk = 0; kk < k; kk++)
                    acc += arow[kk] * brow[kk];
                if (d && l1)
                    for (int64_t p = 0; p < r; p++)
                        acc += (double)nvo_bf16_to_f32(d[i * r + p]) * (double)nvo_bf16_to_f32(l1[nn * r + p]);
                double y = (double)alpha * acc;
                if (bias)
                    y += (double)nvo_bf16_to_f32(bias[nn]);
                out[j * n + nn] = y;
            }
        }
        free(arow);
    }
    free(bdq);
    return NVO_OK;
}

/*
 * Weight-only form ([NVF] f16a_nvfp4weight_scaled_mm: the bf16 activation
 * against the dequantized weight, then F.linear).  For each requested row i
 * (rows[j]): out[j, n] = alpha * sum_k a[i,k] * Bdq[n,k] + bias[n] in fp64,
 * not rounded to bf16.  a: bf16 [m, k]; alpha = 1 / the weight's global
 * scale; bias: NULL or bf16 [n].
 */
int nvo_gemm_w4a16_rows(const uint16_t *a, const uint8_t *b, const uint8_t *b_sf, float alpha,
                        const uint16_t *bias, int64_t m, int64_t n, int64_t k, const int64_t *rows,
                        int64_t nrows, double *out)
{
    if (k % 16 != 0 || m < 0 || n < 0)
        return NVO_BAD;
    for (int64_t j = 0; j < nrows; j++)
        if (rows[j] < 0 || rows[j] >= m)
            return NVO_BAD;
    double *bdq = (double *)malloc(sizeof(double) * (size_t)(n * k > 0 ? n * k : 1));
    if (!bdq)
        return NVO_BAD;
#pragma omp parallel for schedule(static)
    for (int64_t nn = 0; nn < n; nn++)
        for (int64_t kk = 0; kk < k; kk++)
            bdq[nn * k + kk] = dq(b, b_sf, nn, kk, k);
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t j = 0; j < nrows; j++) {
        const uint16_t *arow = a + rows[j] * k;
        for (int64_t nn = 0; nn < n; nn++) {
            double acc = 0.0;
            const double *brow = bdq + nn * k;
            for (int64_t kk = 0; kk < k; kk++)
                acc += (double)nvo_bf16_to_f32(arow[kk]) * brow[kk];
            double y = (double)alpha * acc;
            if (bias)
                y += (double)nvo_bf16_to_f32(bias[nn]);
            out[j * n + nn] = y;
        }
    }
    free(bdq);
    return NVO_OK;
}

/* ------------------------------------------------------------------------ */
/* MX variant: one ue8m0 (power-of-two) scale per 32 elements                 */
/* ------------------------------------------------------------------------ */

/*
 * [FI] the single-item fp4_quantize takes the block width (16) and a ue8m0
 * flag (off) as positional arguments; the pages fix nothing else about the
 * other setting.  Reading: the OCP Microscaling Formats (MX) v1.0 conversion
 * for MXFP4 -- 32-element blocks, an e8m0 scale X = 2^(floor(log2 amax) - 2)
 * (2 is the largest exponent of e2m1), elements e2m1(v / X) nearest-even and
 * saturating at 6, no global scale.  A block whose amax is 0 gets code 0; the
 * shared exponent is clamped to e8m0's range [-127, 127].  nan_to_num is
 * applied first, as on the NVFP4 path.  Scales use the same 128x4 swizzled,
 * zero-padded layout with k/32 columns.
 */
double nvo_ue8m0_value(uint8_t code)
{
    return code == 0xFF ? NAN : ldexp(1.0, (int)code - 127);
}

int64_t nvo_sf_size_mx(int64_t rows, int64_t k)
{
    return nvo_pad_up(rows, 128) * nvo_pad_up(k / 32, 4);
}

int64_t nvo_sf_offset_mx(int64_t r, int64_t c, int64_t k)
{
    int64_t cp = nvo_pad_up(k / 32, 4);
    return ((r / 128) * (cp / 4) + c / 4) * 512 + (r % 32) * 16 + ((r % 128) / 32) * 4 + (c % 4);
}

/* x: bf16 (x_dtype 0) or fp32 (1) [m, k]; out_fp4 [m, k/2]; out_sf
 * [sf_size_mx(m, k)], fully written. */
int nvo_quantize_mx(const void *x, int x_dtype, int64_t m, int64_t k, uint8_t *out_fp4, uint8_t *out_sf)
{
    if (m < 0 || k < 32 || k % 32 != 0 || (x_dtype != 0 && x_dtype != 1))
        return NVO_BAD;
    memset(out_sf, 0, (size_t)nvo_sf_size_mx(m, k));
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < m; r++) {
        for (int64_t kb = 0; kb < k / 32; kb++) {
            float blk[32];
            float amax = 0.0f;
            for (int j = 0; j < 32; j++) {
                int64_t i = r * k + kb * 32 + j;
                float v = x_dtype == 1 ? ((const float *)x)[i] : nvo_bf16_to_f32(((const uint16_t *)x)[i]);
                blk[j] = nan_to_num(v);
                if (fabsf(blk[j]) > amax)
                    amax = fabsf(blk[j]);
            }
            int shared = -127;
            if (amax > 0.0f) {
                int ex;
                frexp((double)amax, &ex);      /* amax = f * 2^ex, 0.5 <= f < 1 */
                shared = (ex - 1) - 2;         /* floor(log2 amax) - emax(e2m1) */
                if (shared < -127)
                    shared = -127;
                if (shared > 127)
                    shared = 127;
            }
            out_sf[nvo_sf_offset_mx(r, kb, k)] = (uint8_t)(amax > 0.0f ? shared + 127 : 0);
            uint8_t codes[32];
            for (int j = 0; j < 32; j++)
                codes[j] = nvo_e2m1_encode((float)ldexp((double)blk[j], -shared));
            for (int j = 0; j < 16; j++)
                out_fp4[r * (k / 2) + kb * 16 + j] = (uint8_t)(codes[2 * j] | (codes[2 * j + 1] << 4));
        }
    }
    return NVO_OK;
}

static double dq_mx(const uint8_t *p, const uint8_t *sf, int64_t row, int64_t col, int64_t K)
{
    uint8_t byte = p[row * (K / 2) + col / 2];
    uint8_t code = (col & 1) ? (byte >> 4) : (byte & 15);
    return nvo_e2m1_value(code) * nvo_ue8m0_value(sf[nvo_sf_offset_mx(row, col / 32, K)]);
}

/* MX GEMM rows: out[j, n] = alpha * sum_k Adq[rows[j],k] * Bdq[n,k] + bias[n]
 * in fp64 (each product of two dequantized MX values is exact). */
int nvo_gemm_mx_rows(const uint8_t *a, const uint8_t *b, const uint8_t *a_sf, const uint8_t *b_sf,
                     float alpha, const uint16_t *bias, int64_t m, int64_t n, int64_t k,
                     const int64_t *rows, int64_t nrows, double *out)
{
    if (k % 32 != 0 || m < 0 || n < 0)
        return NVO_BAD;
    for (int64_t j = 0; j < nrows; j++)
        if (rows[j] < 0 || rows[j] >= m)
            return NVO_BAD;
    double *bdq = (double *)malloc(sizeof(double) * (size_t)(n * k > 0 ? n * k : 1));
    if (!bdq)
        return NVO_BAD;
#pragma omp parallel for schedule(static)
    for (int64_t nn = 0; nn < n; nn++)
        for (int64_t kk = 0; kk < k; kk++)
            bdq[nn * k + kk] = dq_mx(b, b_sf, nn, kk, k);
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t j = 0; j < nrows; j++) {
        double *arow = (double *)malloc(sizeof(double) * (size_t)k);
        if (arow) {
            for (int64_t kk = 0; kk < k; kk++)
                arow[kk] = dq_mx(a, a_sf, rows[j], kk, k);
            for (int64_t nn = 0; nn < n; nn++) {
                double acc = 0.0;
                const double *brow = bdq + nn * k;
                for (int64_t kk = 0; kk < k; kk++)
                    acc += arow[kk] * brow[kk];
                double y = (double)alpha * acc;
                if (bias)
                    y += (double)nvo_bf16_to_f32(bias[nn]);
                out[j * n + nn] = y;
            }
            free(arow);
        }
    }
    free(bdq);
    return NVO_OK;
}

/*
 * bf16 output of an fp32-accumulated GEMM, from the exact fp64 value: round
 * to fp32 (nearest even, the C conversion), then to bf16 (nearest even).
 * [FI] the routed-expert gate_up GEMM writes this bf16 h, which the
 * silu_and_mul quantize then reads.
 */
void nvo_f64_to_bf16_via_f32(const double *v, uint16_t *out, int64_t n)
{
    for (int64_t i = 0; i < n; i++)
        out[i] = nvo_f32_to_bf16((float)v[i]);
}

int nvo_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
