/*
 * CPU oracle for NVFP4 block quantization and fused SwiGLU + NVFP4 quantize.
 *
 * TEST INFRASTRUCTURE ONLY: plain, slow, obviously-correct reference code.
 * Only the test suite, the smoke check and the benchmark's CPU-baseline leg
 * may load it. It shares no code with the HIP library.
 *
 * Build: gcc -std=c11 -O2 -fopenmp -ffp-contract=off -fPIC -shared (no
 * fast-math). Every float expression below is evaluated in binary32 with
 * round-to-nearest-even unless it is explicitly written in double.
 *
 * Page references (see nvfp4_oracle.h for the page list):
 *   [APPROACH-2]  "NVFP4-1.1_APPROACH_PART_2.md"
 *   [STATUS]      "2026-05-28_STATUS.md", commit "NVFP4-1.1: FP4 quantization
 *                 primitives for CuTeDSL kernels"
 *   [APPROACH]    "NVFP4-1.1_APPROACH.md", section "Revised approach:
 *                 Compact SwiGLU output"
 */
#include "nvfp4_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ------------------------------------------------------------------------
 * BF16 -> FP32. A bfloat16 is the top half of a binary32, so the widening
 * is an exact 16-bit shift. [APPROACH] "Revised approach": the L1 output is
 * BF16.
 * ---------------------------------------------------------------------- */
float oracle_bf16_to_f32(uint16_t bits)
{
    uint32_t w = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &w, sizeof f);
    return f;
}

/* ------------------------------------------------------------------------
 * FP32 -> BF16, round to nearest, ties to even. [APPROACH] "Revised
 * approach: Compact SwiGLU output": the target flow writes the SwiGLU
 * result as compact BF16 and quantizes that. BF16 has the binary32
 * exponent range and 8 significant bits for normal values (|x| >= 2^-126);
 * below 2^-126 its values are the multiples of 2^-133. The nearest one is
 * found by rounding the scaled magnitude to an integer with rint (ties to
 * even in the default rounding mode); results of 2^128 or more are
 * infinite. NaN becomes the quiet NaN with the input's sign.
 * ---------------------------------------------------------------------- */
uint16_t oracle_f32_to_bf16(float x)
{
    uint32_t w;
    memcpy(&w, &x, sizeof w);
    const uint16_t sign = (uint16_t)((w >> 16) & 0x8000u);
    if (isnan(x))
        return (uint16_t)(sign | 0x7fc0u);
    if (isinf(x) || x == 0.0f)
        return (uint16_t)(w >> 16);             /* exact */
    double a = fabs((double)x), q;
    if (a >= ldexp(1.0, -126)) {
        int e;
        double m = frexp(a, &e);                /* a = m * 2^e, m in [0.5, 1) */
        q = ldexp(rint(ldexp(m, 8)), e - 8);    /* 8 significant bits */
    } else {
        q = ldexp(rint(ldexp(a, 133)), -133);   /* multiples of 2^-133 */
    }
    float r = (float)q;                         /* exact, or inf for q >= 2^128 */
    uint32_t rw;
    memcpy(&rw, &r, sizeof rw);
    return (uint16_t)(sign | (rw >> 16));
}

/* ------------------------------------------------------------------------
 * SwiGLU: silu(gate) * up = gate * up / (1 + e^-gate).
 * [APPROACH-2] fused-epilogue design: gate subtiles give SiLU(gate), up
 * subtiles give SiLU(gate) * up, kept in FP32 registers (no BF16 rounding).
 * Evaluated in binary64 with libm exp and rounded once to binary32.
 * No clamp: the pages mention clamping in the existing kernel without limits.
 * ---------------------------------------------------------------------- */
float oracle_swiglu(float gate, float up)
{
    double g = (double)gate;
    double u = (double)up;
    double y = g * u / (1.0 + exp(-g));
    return (float)y;
}

/* ------------------------------------------------------------------------
 * FP8 E4M3 (OCP "fn" variant) encode of a non-negative scale, following the
 * [STATUS] commit's list for fp8_e4m3_from_float32 and the [APPROACH-2] log:
 *   - exponent bias 7, exponent field 0..15 all used for numbers;
 *   - exponent 15 with mantissa 7 is NaN, so the largest value is
 *     exp 15 / mant 6 = 448 and larger inputs clamp to 448;
 *   - exponent field 0 is subnormal with value m / 512;
 *   - round to nearest, ties to even, for the mantissa;
 *   - a mantissa that rounds up to 8 carries into the exponent
 *     (250 -> 256 = 0x78, not 240 = 0x77).
 * Scales are magnitudes: inputs <= 0 (and NaN, which is out of contract)
 * encode as 0x00.
 * ---------------------------------------------------------------------- */
uint8_t oracle_fp8_e4m3_encode(float v)
{
    if (!(v > 0.0f))
        return 0x00;
    if (v > 448.0f)
        v = 448.0f;                       /* clamp to the largest finite */

    if (v < 0x1p-6f) {
        /* subnormal range: value = m / 512, m = 0..7; m rounding to 8 is
         * the smallest normal 2^-6, whose code is also 8 (0x08). */
        double m = rint((double)v * 512.0);      /* exact product, RNE */
        return (uint8_t)m;
    }

    int E;
    (void)frexp((double)v, &E);           /* v = f * 2^E, f in [0.5, 1) */
    int e = E - 1;                        /* v = (1 + frac) * 2^e       */
    double mant = rint((ldexp((double)v, -e) - 1.0) * 8.0);   /* RNE */
    if (mant == 8.0) {                    /* mantissa overflow: carry */
        e += 1;
        mant = 0.0;
    }
    int biased = e + 7;                   /* bias 7 */
    if (biased == 15 && mant == 7.0)      /* NaN guard (unreachable after */
        mant = 6.0;                       /* the clamp, kept as the pages do) */
    return (uint8_t)((biased << 3) | (int)mant);
}

/* ------------------------------------------------------------------------
 * FP8 E4M3 decode ([STATUS] fp8_e4m3_to_float32; [APPROACH-2] subnormal fix):
 *   e == 0 : m / 512 (= 2^(1-7) * m/8)
 *   else   : 2^(e-7) * (1 + m/8)
 *   e == 15 && m == 7 : NaN
 * ---------------------------------------------------------------------- */
float oracle_fp8_e4m3_decode(uint8_t code)
{
    int s = code >> 7;
    int e = (code >> 3) & 15;
    int m = code & 7;
    if (e == 15 && m == 7)
        return NAN;
    double mag = (e == 0) ? (double)m / 512.0
                          : ldexp(1.0 + (double)m / 8.0, e - 7);
    return (float)(s ? -mag : mag);
}

/* ------------------------------------------------------------------------
 * Half-step -> E2M1 magnitude index ([STATUS] half_step_to_e2m1_idx,
 * [APPROACH-2] step_to_idx). The half-step is hs = round(2 * min(|s|, 6)),
 * an integer 0..12 counting units of 0.5; the E2M1 magnitudes are
 * {0, 0.5, 1, 1.5, 2, 3, 4, 6} (indices 0..7).
 *   hs 0..4   -> 0..4      exact grid points 0, 0.5, 1, 1.5, 2
 *   hs 5      -> 4         2.5 sits midway between 2 and 3; tie goes down
 *   hs 6      -> 5         exact 3
 *   hs 7      -> 6         3.5 midway between 3 and 4; tie to the even
 *                          mantissa (4), following the pages' RNE rule
 *   hs 8      -> 6         exact 4
 *   hs 9      -> 6         4.5 is nearer 4
 *   hs 10     -> 6         5 midway between 4 and 6: the pages give 6 here
 *   hs 11     -> 7         5.5 is nearer 6: the pages give 7 here
 *   hs 12     -> 7         exact 6 (the E2M1 maximum)
 * ---------------------------------------------------------------------- */
int oracle_e2m1_index(int half_step)
{
    static const int step_to_idx[13] = {0, 1, 2, 3, 4, 4, 5, 6, 6, 6, 6, 7, 7};
    if (half_step < 0 || half_step > 12)
        return -1;
    return step_to_idx[half_step];
}

/* E2M1 nibble -> value: sign in bit 3, magnitude index in bits 0..2. */
float oracle_e2m1_decode(uint8_t nibble)
{
    static const float mag[8] = {0.0f, 0.5f, 1.0f, 1.5f, 2.0f, 3.0f, 4.0f, 6.0f};
    float v = mag[nibble & 7];
    return (nibble & 8) ? -v : v;
}

/* ------------------------------------------------------------------------
 * One NVFP4 block of 16 values ([APPROACH-2] fused-epilogue design: every
 * two 8-wide up subtiles form one block; amax, FP8 scale, E2M1 pack; 16
 * values become 8 packed bytes plus one scale byte).
 *   amax  = max |x_j|                              (exact)
 *   bsf   = RN32(amax / RN32(6 * gs))              block scale before FP8
 *   sf    = fp8_e4m3_encode(bsf)                   stored scale byte
 *   denom = RN32(decode(sf) * gs)
 *   s_j   = RN32(x_j / denom)  (magnitude forced to 0 when denom == 0)
 *   hs_j  = rint(2 * min(|s_j|, 6))                ties to even
 *   code  = signbit(x_j) << 3 | step_to_idx[hs_j]
 *   byte i = code[2i] | code[2i+1] << 4            even element low nibble
 * gs is the per-tensor (or per-expert) FP32 global scale in the decode
 * direction: x ~ e2m1 * decode(sf) * gs.
 * bsf_diag receives bsf, v_diag the pre-rounding 2*min(|s|,6) per element.
 * ---------------------------------------------------------------------- */
void oracle_quantize_block(const float x[16], float gs, uint8_t packed[8],
                           uint8_t *sf_out, float *bsf_diag, float v_diag[16])
{
    float amax = 0.0f;
    for (int j = 0; j < 16; ++j) {
        float a = fabsf(x[j]);
        if (a > amax)
            amax = a;
    }

    float k = 6.0f * gs;
    float bsf = amax / k;
    uint8_t sf = oracle_fp8_e4m3_encode(bsf);
    float denom = oracle_fp8_e4m3_decode(sf) * gs;

    uint8_t code[16];
    for (int j = 0; j < 16; ++j) {
        float v = 0.0f;
        if (denom != 0.0f) {
            float s = x[j] / denom;
            v = 2.0f * fminf(fabsf(s), 6.0f);
        }
        int hs = (int)rint((double)v);
        code[j] = (uint8_t)((signbit(x[j]) ? 8 : 0) | oracle_e2m1_index(hs));
        if (v_diag)
            v_diag[j] = v;
    }
    for (int i = 0; i < 8; ++i)
        packed[i] = (uint8_t)(code[2 * i] | (code[2 * i + 1] << 4));
    *sf_out = sf;
    if (bsf_diag)
        *bsf_diag = bsf;
}

/* ------------------------------------------------------------------------
 * Array drivers.
 * ---------------------------------------------------------------------- */
int oracle_fp8_encode_array(const float *v, int64_t n, uint8_t *out)
{
    if (n < 0 || (n > 0 && (!v || !out)))
        return 1;
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i)
        out[i] = oracle_fp8_e4m3_encode(v[i]);
    return 0;
}

/* De-interleave + SwiGLU. [APPROACH] and [APPROACH-2]: the L1 GEMM writes
 * 2*I BF16 columns per row as repeating 8-wide subtiles [gate x8, up x8].
 * Output column j reads gate at 16*(j/8) + j%8 and up at 16*(j/8) + 8 + j%8. */
int oracle_swiglu_rows(const uint16_t *in, int64_t rows, int64_t inter,
                       int64_t ld_in, float *y)
{
    if (rows < 0 || inter < 0 || inter % 8 != 0 || ld_in < 2 * inter)
        return 1;
    if (rows == 0 || inter == 0)
        return 0;
    if (!in || !y)
        return 1;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        const uint16_t *row = in + r * ld_in;
        for (int64_t j = 0; j < inter; ++j) {
            int64_t base = 16 * (j / 8);
            float g = oracle_bf16_to_f32(row[base + j % 8]);
            float u = oracle_bf16_to_f32(row[base + 8 + j % 8]);
            y[r * inter + j] = oracle_swiglu(g, u);
        }
    }
    return 0;
}

/* De-interleave + SwiGLU of FP32 inputs: the L1 GEMM's FP32 accumulators in
 * the fused-epilogue design ([APPROACH-2]: SiLU(gate) and SwiGLU computed
 * from the accumulators, before any BF16 rounding). Same column mapping as
 * oracle_swiglu_rows. */
int oracle_swiglu_f32_rows(const float *acc, int64_t rows, int64_t inter,
                           int64_t ld_acc, float *y)
{
    if (rows < 0 || inter < 0 || inter % 8 != 0 || ld_acc < 2 * inter)
        return 1;
    if (rows == 0 || inter == 0)
        return 0;
    if (!acc || !y)
        return 1;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        const float *a = acc + r * ld_acc;
        for (int64_t j = 0; j < inter; ++j) {
            int64_t col = 16 * (j / 8) + j % 8;          /* gate column; up is col + 8 */
            y[r * inter + j] = oracle_swiglu(a[col], a[col + 8]);
        }
    }
    return 0;
}

/* The first pass of the two-pass variant ([APPROACH] "Revised approach:
 * Compact SwiGLU output", target flow): the SwiGLU of the interleaved input
 * rounded to BF16, written as a compact [rows][inter] BF16 tensor. */
int oracle_swiglu_bf16_rows(const uint16_t *in, int64_t rows, int64_t inter,
                            int64_t ld_in, uint16_t *out)
{
    if (rows < 0 || inter < 0 || inter % 8 != 0 || ld_in < 2 * inter)
        return 1;
    if (rows == 0 || inter == 0)
        return 0;
    if (!in || !out)
        return 1;
    int bad = 0;
#pragma omp parallel reduction(|: bad)
    {
        float *y = (float *)malloc((size_t)inter * sizeof(float));
        if (!y)
            bad = 1;
#pragma omp for schedule(static)
        for (int64_t r = 0; r < rows; ++r) {
            if (!y)
                continue;
            oracle_swiglu_rows(in + r * ld_in, 1, inter, ld_in, y);   /* FP32 SwiGLU of row r */
            for (int64_t j = 0; j < inter; ++j)
                out[r * inter + j] = oracle_f32_to_bf16(y[j]);
        }
        free(y);
    }
    return bad;
}

int oracle_f32_to_bf16_array(const float *x, int64_t n, uint16_t *out)
{
    if (n < 0 || (n > 0 && (!x || !out)))
        return 1;
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i)
        out[i] = oracle_f32_to_bf16(x[i]);
    return 0;
}

int oracle_quantize_f32_rows(const float *x, int64_t rows, int64_t cols,
                             int64_t ld_x, const float *gs_rows,
                             uint8_t *packed, uint8_t *scales,
                             float *bsf_diag, float *v_diag)
{
    if (rows < 0 || cols < 0 || cols % 16 != 0 || ld_x < cols)
        return 1;
    if (rows == 0 || cols == 0)
        return 0;
    if (!x || !packed || !scales)
        return 1;
    int64_t nb = cols / 16;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        float gs = gs_rows ? gs_rows[r] : 1.0f;
        for (int64_t b = 0; b < nb; ++b) {
            float bsf;
            oracle_quantize_block(x + r * ld_x + 16 * b, gs,
                                  packed + r * (cols / 2) + 8 * b,
                                  scales + r * nb + b, &bsf,
                                  v_diag ? v_diag + r * cols + 16 * b : NULL);
            if (bsf_diag)
                bsf_diag[r * nb + b] = bsf;
        }
    }
    return 0;
}

int oracle_quantize_bf16_rows(const uint16_t *x, int64_t rows, int64_t cols,
                              int64_t ld_x, const float *gs_rows,
                              uint8_t *packed, uint8_t *scales)
{
    if (rows < 0 || cols < 0 || cols % 16 != 0 || ld_x < cols)
        return 1;
    if (rows == 0 || cols == 0)
        return 0;
    if (!x || !packed || !scales)
        return 1;
    int64_t nb = cols / 16;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        float gs = gs_rows ? gs_rows[r] : 1.0f;
        for (int64_t b = 0; b < nb; ++b) {
            float blk[16];
            for (int j = 0; j < 16; ++j)
                blk[j] = oracle_bf16_to_f32(x[r * ld_x + 16 * b + j]);
            oracle_quantize_block(blk, gs, packed + r * (cols / 2) + 8 * b,
                                  scales + r * nb + b, NULL, NULL);
        }
    }
    return 0;
}

int oracle_swiglu_quantize_rows(const uint16_t *in, int64_t rows,
                                int64_t inter, int64_t ld_in,
                                const float *gs_rows, uint8_t *packed,
                                uint8_t *scales, float *swiglu_out,
                                float *bsf_diag, float *v_diag)
{
    if (rows < 0 || inter < 0 || inter % 16 != 0 || ld_in < 2 * inter)
        return 1;
    if (rows == 0 || inter == 0)
        return 0;
    if (!in || !packed || !scales)
        return 1;
    int64_t nb = inter / 16;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        const uint16_t *row = in + r * ld_in;
        float gs = gs_rows ? gs_rows[r] : 1.0f;
        for (int64_t b = 0; b < nb; ++b) {
            float blk[16];
            for (int j = 0; j < 16; ++j) {
                int64_t col = 16 * b + j;
                int64_t base = 16 * (col / 8);
                float g = oracle_bf16_to_f32(row[base + col % 8]);
                float u = oracle_bf16_to_f32(row[base + 8 + col % 8]);
                blk[j] = oracle_swiglu(g, u);
                if (swiglu_out)
                    swiglu_out[r * inter + col] = blk[j];
            }
            float bsf;
            oracle_quantize_block(blk, gs, packed + r * (inter / 2) + 8 * b,
                                  scales + r * nb + b, &bsf,
                                  v_diag ? v_diag + r * inter + 16 * b : NULL);
            if (bsf_diag)
                bsf_diag[r * nb + b] = bsf;
        }
    }
    return 0;
}

/* Dequantize: x = RN32(RN32(e2m1(code) * decode(sf)) * gs). The inner
 * product is exact (at most 2 x 4 significant bits). */
int oracle_dequantize_rows(const uint8_t *packed, const uint8_t *scales,
                           int64_t rows, int64_t cols, const float *gs_rows,
                           float *out)
{
    if (rows < 0 || cols < 0 || cols % 16 != 0)
        return 1;
    if (rows == 0 || cols == 0)
        return 0;
    if (!packed || !scales || !out)
        return 1;
    int64_t nb = cols / 16;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        float gs = gs_rows ? gs_rows[r] : 1.0f;
        for (int64_t c = 0; c < cols; ++c) {
            uint8_t byte = packed[r * (cols / 2) + c / 2];
            uint8_t nib = (c % 2 == 0) ? (byte & 15) : (byte >> 4);
            float dsf = oracle_fp8_e4m3_decode(scales[r * nb + c / 16]);
            float t = oracle_e2m1_decode(nib) * dsf;
            out[r * cols + c] = t * gs;
        }
    }
    return 0;
}

/* Per-group amax of |y| over row ranges [offsets[e], offsets[e+1]). Empty
 * groups give 0. Used for the two-level (per-expert) global scale. */
int oracle_group_amax(const float *y, int64_t rows, int64_t cols,
                      const int32_t *offsets, int32_t groups, float *amax)
{
    if (rows < 0 || cols < 0 || groups < 1 || !offsets || !amax)
        return 1;
    if (offsets[0] != 0 || offsets[groups] != rows)
        return 1;
    for (int32_t e = 0; e < groups; ++e)
        if (offsets[e + 1] < offsets[e])
            return 1;
    if (rows > 0 && cols > 0 && !y)
        return 1;
#pragma omp parallel for schedule(dynamic, 1)
    for (int32_t e = 0; e < groups; ++e) {
        float m = 0.0f;
        for (int64_t r = offsets[e]; r < offsets[e + 1]; ++r)
            for (int64_t c = 0; c < cols; ++c) {
                float a = fabsf(y[r * cols + c]);
                if (a > m)
                    m = a;
            }
        amax[e] = m;
    }
    return 0;
}

int oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

void oracle_set_num_threads(int n)
{
#ifdef _OPENMP
    if (n > 0)
        omp_set_num_threads(n);
#else
    (void)n;
#endif
}
