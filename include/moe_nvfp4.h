/*
 * moe_nvfp4.h - C ABI of libmoe_nvfp4.so: NVFP4 block quantization and the
 * fused SwiGLU + NVFP4 quantize step of an MoE L1 epilogue, on MI355X
 * (gfx950) with hand-written HIP kernels.
 *
 * The method comes from the "nvfp4-megamoe-kernel" project log pages
 * (2026-05-28): "NVFP4-1.1_APPROACH_PART_2.md" (FP8 E4M3 scale rules, the
 * half-step E2M1 rounding, the fused-epilogue write path) and
 * "NVFP4-1.1_APPROACH.md" ("Revised approach: Compact SwiGLU output": the
 * interleaved [gate x8, up x8, ...] BF16 L1 output; "Implementation plan").
 *
 * Formats
 *   NVFP4 block   16 consecutive values along a row -> 8 bytes of E2M1 codes
 *                 (element 2i in the low nibble of byte i, 2i+1 in the high
 *                 nibble; code = sign << 3 | magnitude index, magnitudes
 *                 {0, .5, 1, 1.5, 2, 3, 4, 6}) plus one FP8 E4M3 scale byte.
 *   scale byte    OCP E4M3 ("fn"): bias 7, exponent field 0..15, exp 15 with
 *                 mantissa 7 is NaN and never written, largest value 448,
 *                 subnormals m/512, round to nearest even with mantissa carry
 *                 into the exponent, saturating at 448 (0x7e).
 *   global scale  gs, FP32, decode direction: value ~ e2m1 * scale * gs.
 *   per block     bsf = RN(amax / RN(6 gs)); sf = E4M3(bsf);
 *                 d = RN(E4M3value(sf) * gs); s = RN(x / d) (0 when d == 0);
 *                 code magnitude = step_to_idx[rint(2 min(|s|, 6))] with
 *                 ties to even; sign = IEEE sign bit of x.
 *
 * Layouts (all row-major; ld_* are row pitches in ELEMENTS of that tensor)
 *   plain input   x[rows][ld_x] BF16 (raw uint16 bit patterns), cols used.
 *   fused input   gate_up[rows][ld_in] BF16, 2*inter columns used, laid out
 *                 as repeating 8-wide subtiles [gate x8, up x8]: output
 *                 column j reads gate at 16*(j/8) + j%8 and up at
 *                 16*(j/8) + 8 + j%8.
 *   packed        [rows][cols/2] bytes, contiguous (pitch cols/2).
 *   scales        [rows][cols/16] bytes, contiguous (pitch cols/16).
 *   swiglu_out    [rows][inter] FP32, contiguous (optional debug output).
 *   out           [rows][cols] FP32, contiguous (dequantize); for
 *                 swiglu_bf16, [rows][ld_out] BF16.
 *
 * Global scales and experts
 *   gs == NULL                      every row uses 1.0.
 *   gs != NULL, expert_offsets NULL gs[0] is used for every row.
 *   expert_offsets != NULL          num_experts >= 1 groups of rows: row r
 *                                   belongs to expert e when
 *                                   expert_offsets[e] <= r < expert_offsets[e+1];
 *                                   it uses gs[e] (or 1.0 when gs == NULL).
 *                                   expert_offsets has num_experts + 1
 *                                   int32 entries, starts at 0, is
 *                                   non-decreasing and ends at rows. Empty
 *                                   experts are allowed.
 *
 * Memory and ownership
 *   Every pointer is a DEVICE pointer (HIP/PyTorch allocations), except that
 *   none is dereferenced on the host. The caller owns every buffer. The
 *   library allocates nothing, keeps no state between calls, never
 *   synchronizes, and enqueues its kernels on `stream` (NULL = the default
 *   stream): one kernel per call, three for the global-scale calls. Inputs
 *   and outputs must not overlap. Every byte of the output regions
 *   described above is written (the paged cache write excepted: it writes
 *   only the cache rows its slots name).
 *
 * Preconditions checked on the host, before any HIP call (so they work on a
 * machine without a GPU) - a failing check returns without launching:
 *   rows, cols/inter >= 0; cols (inter) % 16 == 0; ld >= used columns;
 *   the byte extent rows * ld * 2 of every strided buffer fits in int64;
 *   required pointers non-NULL; BF16 input base and row pitch 16-byte
 *   aligned; packed 8-byte aligned; FP32 outputs 16-byte aligned;
 *   num_experts >= 1 exactly when expert_offsets != NULL; rows < 2^31 and
 *   rows * ceil(cols / 1024) <= 2^30 (tiles of 64 blocks).
 *   rows == 0 or cols == 0 is a successful no-op.
 * Not checked (device data, asynchronous): finite inputs; gs within
 *   [2^-64, 2^64] (there every quotient of the quantizer is correctly
 *   rounded: its remainders stay in the normal binary32 range); the offset
 *   rules above. Violations give unspecified output bytes, never
 *   out-of-bounds accesses on the output region for rows that the offsets
 *   place inside [0, rows). Within them no quotient overflows or turns into
 *   NaN: in a block whose scale saturates, every value beyond 6 scale units
 *   gets the largest magnitude with its own sign, an infinite SwiGLU value
 *   (finite gate and up whose product exceeds the FP32 range) included.
 * Errors: a launch failure reported by hipGetLastError() returns
 *   NVFP4_ERROR_LAUNCH; faults during execution surface at the caller's next
 *   synchronization, as usual for HIP.
 */
#ifndef MOE_NVFP4_H
#define MOE_NVFP4_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    NVFP4_SUCCESS = 0,
    NVFP4_ERROR_INVALID_VALUE = 1,     /* negative size, NULL pointer, bad ld, experts */
    NVFP4_ERROR_UNSUPPORTED_SHAPE = 2, /* cols/inter not a multiple of 16, too large */
    NVFP4_ERROR_MISALIGNED = 3,        /* base or pitch alignment rule broken */
    NVFP4_ERROR_LAUNCH = 4             /* hipGetLastError() after the launch */
} nvfp4_status_t;

/*
 * Standalone NVFP4 quantize of a BF16 tensor.
 * Page: "2026-05-28_STATUS.md", "GPU-only NVFP4 quantize" (byte-exact with
 * the Python reference) and "NVFP4-1.1_APPROACH_PART_2.md" (quantize_nvfp4.cu
 * half-step rounding). Reads x[rows][cols] (pitch ld_x), writes
 * packed[rows][cols/2] and scales[rows][cols/16].
 */
nvfp4_status_t nvfp4_quantize(const uint16_t *x, int64_t rows, int64_t cols,
                              int64_t ld_x, const float *gs,
                              const int32_t *expert_offsets, int32_t num_experts,
                              uint8_t *packed, uint8_t *scales,
                              hipStream_t stream);

/*
 * Fused SwiGLU + NVFP4 quantize (the MoE L1 epilogue as a standalone pass).
 * Page: "NVFP4-1.1_APPROACH_PART_2.md", fused-epilogue design (SiLU of the
 * gate subtile, SwiGLU of the up subtile kept in FP32, two up subtiles per
 * FP4 block, amax + FP8 scale + E2M1 pack) and "NVFP4-1.1_APPROACH.md"
 * (interleaved [gate x8, up x8] L1 layout). Reads gate_up[rows][2*inter]
 * (pitch ld_in), computes y = silu(gate) * up in FP32 and writes
 * packed[rows][inter/2], scales[rows][inter/16] and, when swiglu_out is not
 * NULL, the FP32 y values [rows][inter] (a debug output: the quantized bytes
 * are the same with or without it). Each y is the binary32 rounding of the
 * exact gate * up * sigmoid(gate), for every finite BF16 gate and up, except
 * where that value lies within about 2^-52 (relative) of a rounding
 * midpoint, and where |gate * up| < 2^-126: there y may be the neighbouring
 * value, one subnormal step (2^-149) away. sigmoid comes from a binary64
 * table of every BF16 gate's value; for |gate| < 2^-24 its entry for
 * +-2^-24 stands in (less than 2^-26 away), which gives the same y. y is
 * never NaN for finite inputs; it is +-inf only where the exact value
 * rounds to it.
 */
nvfp4_status_t swiglu_nvfp4_quantize(const uint16_t *gate_up, int64_t rows,
                                     int64_t inter, int64_t ld_in,
                                     const float *gs,
                                     const int32_t *expert_offsets,
                                     int32_t num_experts, uint8_t *packed,
                                     uint8_t *scales, float *swiglu_out,
                                     hipStream_t stream);

/*
 * NVFP4 dequantize: out[r][c] = RN(RN(e2m1(code) * E4M3value(sf)) * gs_row).
 * Page: "2026-05-28_STATUS.md" commit list (fp8_e4m3_to_float32) and the
 * E2M1 code definition. Reads packed[rows][cols/2] and scales[rows][cols/16],
 * writes out[rows][cols] FP32.
 */
nvfp4_status_t nvfp4_dequantize(const uint8_t *packed, const uint8_t *scales,
                                int64_t rows, int64_t cols, const float *gs,
                                const int32_t *expert_offsets,
                                int32_t num_experts, float *out,
                                hipStream_t stream);

/*
 * Global-scale pre-pass of two-level NVFP4 scaling: per expert (or for the
 * whole tensor when expert_offsets is NULL) the largest |value| the
 * quantizer will see, amax_e, and the FP32 global scale
 *     gs[e] = RN(amax_e / (6 * 448))        (1.0 when amax_e == 0 or the
 *                                            expert has no rows),
 * which puts the expert's largest block scale on the FP8 maximum 448,
 * clamped to [2^-64, 2^64], the global scales the quantize calls accept
 * (an expert with amax below 2688 * 2^-64 keeps block scales under 448; one
 * above 2688 * 2^64 saturates them).
 * Page: "NVFP4-1.1_APPROACH_PART_2.md" (the fused kernel's l2_global_scale
 * parameter, the decode-direction global scale in the FP8 scale rule), with
 * the per-expert amax / (6 * 448) recipe of the ragged grouped MoE workload.
 * The values are those of the matching quantize call: BF16 x for
 * nvfp4_global_scale, y = silu(gate) * up in FP32 (bit-identical to what
 * swiglu_nvfp4_quantize computes) for swiglu_nvfp4_global_scale. Inputs and
 * their checks are those of the matching quantize call; rows == 0 still
 * writes the outputs (amax 0, gs 1.0).
 *   amax   [G] FP32 output, or NULL (then gs is used as the accumulator)
 *   gs     [G] FP32 output, required; G = num_experts, or 1 without experts
 * Outputs must be 4-byte aligned; num_experts <= 1024 (else
 * NVFP4_ERROR_UNSUPPORTED_SHAPE). Enqueues three kernels on `stream`: zero
 * the accumulator, reduce the input, write gs. The result does not depend
 * on the order of the reduction.
 */
nvfp4_status_t nvfp4_global_scale(const uint16_t *x, int64_t rows, int64_t cols,
                                  int64_t ld_x, const int32_t *expert_offsets,
                                  int32_t num_experts, float *amax, float *gs,
                                  hipStream_t stream);

nvfp4_status_t swiglu_nvfp4_global_scale(const uint16_t *gate_up, int64_t rows,
                                         int64_t inter, int64_t ld_in,
                                         const int32_t *expert_offsets,
                                         int32_t num_experts, float *amax,
                                         float *gs, hipStream_t stream);

/*
 * Compact SwiGLU output: the first pass of the two-pass variant, in which
 * the SwiGLU result is written as BF16 and then quantized by nvfp4_quantize.
 * Page: "NVFP4-1.1_APPROACH.md", "Revised approach: Compact SwiGLU output"
 * (the target flow: L1 output as compact BF16 SwiGLU values, then the
 * standalone GPU quantize). Reads gate_up[rows][2*inter] (pitch ld_in,
 * interleaved as for swiglu_nvfp4_quantize), computes y = silu(gate) * up in
 * FP32 exactly as swiglu_nvfp4_quantize does, rounds it to BF16 (round to
 * nearest, ties to even) and writes out[rows][inter] (pitch ld_out
 * elements). out must be 16-byte aligned with a pitch of a multiple of
 * 8 elements; inter % 16 == 0. One kernel; rows == 0 is a no-op.
 */
nvfp4_status_t swiglu_bf16(const uint16_t *gate_up, int64_t rows, int64_t inter,
                           int64_t ld_in, uint16_t *out, int64_t ld_out,
                           hipStream_t stream);

/*
 * MoE L1 grouped GEMM with the SwiGLU + NVFP4 quantize fused into its
 * epilogue: the L1 output never reaches memory.
 * Page: "NVFP4-1.1_APPROACH_PART_2.md", fused-epilogue design (SiLU(gate) and
 * SwiGLU of the FP32 accumulators in registers, two 8-wide up subtiles per
 * FP4 block, a 128-row CTA tile holding 512 blocks) and "2026-05-28_STATUS.md"
 * (BLOCKED row "Priority 3: NVFP4-1.1 FP4 quant in MoE epilogue").
 *   x       [tokens][ld_x] BF16 activations, rows grouped by expert
 *   w1      [E][2*inter][ld_w] BF16 weights: row n of expert e is GEMM
 *           output column n (weights stored [out][in]); output columns are
 *           interleaved [gate x8, up x8, ...] as for swiglu_nvfp4_quantize
 *   acc[t][n] = sum_k x[t][k] * w1[e(t)][n][k] in FP32 (matrix cores); then
 *   y = silu(acc_gate) * acc_up in FP32 and NVFP4 blocks of 16 y values as
 *   in swiglu_nvfp4_quantize (gs per expert, or NULL for 1.0); writes
 *   packed[tokens][inter/2], scales[tokens][inter/16] and, if swiglu_out is
 *   not NULL, y [tokens][inter] FP32.
 * expert_offsets: as above (NULL: one expert, w1[0], owns every row);
 * num_experts <= 512. Offsets that break the rules give unspecified bytes
 * but no access outside x, w1 and the outputs: the kernel clamps them to
 * [0, tokens] and raises each to the largest one before it. Shapes: hidden % 64 == 0, inter % 128 == 0, ld_x and
 * ld_w >= hidden, multiples of 8 and below 2^22 (NVFP4_ERROR_UNSUPPORTED_SHAPE
 * otherwise: a 256-row operand window is addressed with 32-bit offsets); x
 * and w1 16-byte aligned. One kernel.
 * hidden == 0 is NVFP4_ERROR_UNSUPPORTED_SHAPE; tokens == 0 or inter == 0
 * is a no-op.
 */
nvfp4_status_t moe_l1_gemm_swiglu_nvfp4(const uint16_t *x, const uint16_t *w1,
                                        int64_t tokens, int64_t hidden,
                                        int64_t inter, int64_t ld_x, int64_t ld_w,
                                        const int32_t *expert_offsets,
                                        int32_t num_experts, const float *gs,
                                        uint8_t *packed, uint8_t *scales,
                                        float *swiglu_out, hipStream_t stream);

/*
 * The same grouped GEMM with a plain epilogue: the L1 output rounded to BF16
 * (round to nearest even), out[tokens][ld_out] with n columns (n = 2*inter in
 * the interleaved layout; n % 256 == 0, ld_out >= n, multiple of 8, out
 * 16-byte aligned). This is the producer of the unfused flow
 * (moe_l1_gemm_bf16, then swiglu_nvfp4_quantize), kept to measure what the
 * fusion saves. Page: "NVFP4-1.1_APPROACH.md", "Revised approach" (current
 * flow: L1 GEMM -> BF16 interleaved -> quantize).
 */
nvfp4_status_t moe_l1_gemm_bf16(const uint16_t *x, const uint16_t *w1,
                                int64_t tokens, int64_t hidden, int64_t n,
                                int64_t ld_x, int64_t ld_w,
                                const int32_t *expert_offsets,
                                int32_t num_experts, uint16_t *out,
                                int64_t ld_out, hipStream_t stream);

/*
 * Paged KV-cache write: the same block quantization as nvfp4_quantize, for a
 * second producer, the keys or values of new tokens going into an NVFP4
 * paged cache. Pages: "2026-05-28_STATUS.md" (table "What's working": KV
 * cache infra with a paged cache; the compressor's flush_write kernels with
 * FP8/FP4 quantize; table "What's BLOCKED": "Priority 7: NVFP4-2 FP4 KV
 * pipeline"). The pages give no cache layout; the one here is the plain
 * reading: one cache row per token slot.
 *   x             [rows][ld_x] BF16: row r is one token's keys (or values),
 *                 all heads, cols = heads * head_dim, cols % 16 == 0 (a block
 *                 never crosses a head when head_dim % 16 == 0).
 *   gs            NULL (1.0) or gs[0], one global scale for the call.
 *   slot_mapping  [rows] int64, device: row r goes to cache row
 *                 slot_mapping[r]. A slot outside [0, num_slots) (such as -1
 *                 for a padding token) is skipped: nothing is written for
 *                 that row. Slots must be distinct (two rows with one slot
 *                 leave that slot's bytes unspecified, still in bounds).
 *   packed_cache  [num_slots][cols/2], scales_cache [num_slots][cols/16],
 *                 contiguous; only the rows named by valid slots are
 *                 written, every other cache byte keeps its value.
 * num_slots < 2^31. rows == 0, cols == 0 or num_slots == 0 is a no-op. x as
 * for nvfp4_quantize (16-byte base and pitch); packed_cache 8-byte and
 * slot_mapping 8-byte aligned. One kernel.
 */
nvfp4_status_t nvfp4_quantize_paged(const uint16_t *x, int64_t rows, int64_t cols,
                                    int64_t ld_x, const float *gs,
                                    const int64_t *slot_mapping, int64_t num_slots,
                                    uint8_t *packed_cache, uint8_t *scales_cache,
                                    hipStream_t stream);

/*
 * Paged KV-cache read: out[r][c] = the nvfp4_dequantize value of cache row
 * slots[r] (the FP4 KV consumer side; same pages as nvfp4_quantize_paged).
 * A slot outside [0, num_slots) gives a row of zeros. gs: NULL (1.0) or
 * gs[0]. out [rows][cols] FP32 contiguous, 16-byte aligned; slots [rows]
 * int64, 8-byte aligned; the caches may be NULL when num_slots == 0.
 * rows == 0 or cols == 0 is a no-op. One kernel.
 */
nvfp4_status_t nvfp4_dequantize_paged(const uint8_t *packed_cache,
                                      const uint8_t *scales_cache, int64_t num_slots,
                                      const int64_t *slots, int64_t rows, int64_t cols,
                                      const float *gs, float *out, hipStream_t stream);

/* Static English text for a status code (never NULL). */
const char *nvfp4_status_string(nvfp4_status_t status);

#ifdef __cplusplus
}
#endif
#endif /* MOE_NVFP4_H */
