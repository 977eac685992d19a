/*
 * CPU oracle for NVFP4 block quantization and the fused SwiGLU + NVFP4
 * quantize step of an MoE L1 epilogue.
 *
 * TEST INFRASTRUCTURE ONLY. This library is the slow, plain definition the
 * GPU kernels are checked against. Only the test suite, the smoke check and
 * the CPU-baseline leg of the benchmark may load it; the product path never
 * does, and it shares no code, header or table with the HIP sources.
 *
 * Sources (web pages of the "nvfp4-megamoe-kernel" project log, 2026-05-28):
 *   [APPROACH-2]  "NVFP4-1.1_APPROACH_PART_2.md" - the FP8/E2M1 debugging log
 *                 and the fused-epilogue write-path design.
 *   [STATUS]      "2026-05-28_STATUS.md" - commit message listing the
 *                 quantization primitives and the five fixes found.
 *   [APPROACH]    "NVFP4-1.1_APPROACH.md" - "Revised approach: Compact SwiGLU
 *                 output" (interleaved [gate*8, swiglu*8, ...] L1 layout).
 *
 * Every function is single-threaded per call except the array drivers,
 * which split rows over OpenMP threads (rows are independent).
 */
#ifndef NVFP4_ORACLE_H
#define NVFP4_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- scalar primitives ------------------------------------------------ */
float   oracle_bf16_to_f32(uint16_t bits);
float   oracle_swiglu(float gate, float up);
uint16_t oracle_f32_to_bf16(float x);
uint8_t oracle_fp8_e4m3_encode(float v);
float   oracle_fp8_e4m3_decode(uint8_t code);
int     oracle_e2m1_index(int half_step);
float   oracle_e2m1_decode(uint8_t nibble);
void    oracle_quantize_block(const float x[16], float gs, uint8_t packed[8],
                              uint8_t *sf, float *bsf_diag, float v_diag[16]);

/* ---- array drivers ------------------------------------------------------
 * Row-major; ld_* are row pitches in elements. gs_rows holds one FP32 global
 * scale per row (NULL means 1.0 for every row). Diagnostic outputs may be
 * NULL. All return 0 on success, nonzero on a bad argument. */
int oracle_fp8_encode_array(const float *v, int64_t n, uint8_t *out);

int oracle_swiglu_rows(const uint16_t *in, int64_t rows, int64_t inter,
                       int64_t ld_in, float *y /* rows x inter */);

int oracle_swiglu_f32_rows(const float *acc, int64_t rows, int64_t inter,
                           int64_t ld_acc, float *y /* rows x inter */);
int oracle_swiglu_bf16_rows(const uint16_t *in, int64_t rows, int64_t inter,
                            int64_t ld_in, uint16_t *out /* rows x inter BF16 */);
int oracle_f32_to_bf16_array(const float *x, int64_t n, uint16_t *out);

int oracle_quantize_f32_rows(const float *x, int64_t rows, int64_t cols,
                             int64_t ld_x, const float *gs_rows,
                             uint8_t *packed, uint8_t *scales,
                             float *bsf_diag, float *v_diag);

int oracle_quantize_bf16_rows(const uint16_t *x, int64_t rows, int64_t cols,
                              int64_t ld_x, const float *gs_rows,
                              uint8_t *packed, uint8_t *scales);

int oracle_swiglu_quantize_rows(const uint16_t *in, int64_t rows,
                                int64_t inter, int64_t ld_in,
                                const float *gs_rows, uint8_t *packed,
                                uint8_t *scales, float *swiglu_out,
                                float *bsf_diag, float *v_diag);

int oracle_dequantize_rows(const uint8_t *packed, const uint8_t *scales,
                           int64_t rows, int64_t cols, const float *gs_rows,
                           float *out);

int oracle_group_amax(const float *y, int64_t rows, int64_t cols,
                      const int32_t *offsets, int32_t groups, float *amax);

int oracle_num_threads(void);
void oracle_set_num_threads(int n);

#ifdef __cplusplus
}
#endif
#endif
