// Device-side arithmetic of NVFP4 block quantization for gfx950.
//
// Method: "nvfp4-megamoe-kernel" project log (2026-05-28),
// "NVFP4-1.1_APPROACH_PART_2.md" (FP8 E4M3 scale rules, half-step E2M1
// rounding, fused-epilogue design) and "2026-05-28_STATUS.md" (the commit
// listing the quantization primitives and their five fixes).
//
// Every function here reproduces the binary32 definition of the method
// exactly (bit for bit), except the SwiGLU product through the sigmoid table
// (swiglu_product, swiglu), which is the binary32 rounding of
// g * u * sigmoid(g) except within about 2^-52 (relative) of a rounding
// midpoint, and within one subnormal step when |g u| < 2^-126.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nvfp4 {

// ---- BF16 -> FP32 (exact: a BF16 is the top half of a binary32) ------------
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// ---- SwiGLU through a table of sigmoid values ------------------------------
// A BF16 gate has 65536 values; sigma(g) = 1 / (1 + e^-g) only varies in FP32
// for 2^-24 <= |g| < 256. The table holds sigma for every BF16 magnitude in
// that range (exponent field 103..134, all 128 mantissas: kSigSpan values)
// and both signs, one binary64 RN64(sigma) per entry (gen_sigma_table.py).
// Positive gates use entries [0, kSigSpan), negative ones [kSigSpan,
// 2 kSigSpan): kSigSpan * 8 = 32768 is bit 15 of a BF16 half-word, so the
// sign bit serves as the sign's byte offset where it stands. Magnitudes
// below the range read the first entry (sigma = 1/2 +- 2^-26 there, and
// y = (g u) / 2 exactly after rounding for every smaller gate), magnitudes
// above it the last. binary64 holds sigma as a normal number down to gate
// -255 (about 2^-368), far below the binary32 range that sigma leaves from
// -87.3 down; the last negative entry, read for every gate at or below -255,
// holds 2^-1000, which makes the product a zero with the sign of g u there,
// as the exact value rounds. The entries are copied into LDS once per
// workgroup; a lookup then replaces exp and rcp per element.
constexpr uint32_t kSigLo = 103u << 7;
constexpr uint32_t kSigHi = (134u << 7) | 127u;
constexpr int kSigSpan = (int)(kSigHi - kSigLo + 1);   // 4096
constexpr int kSigFloats = 4 * kSigSpan;               // 16384 32-bit words (64 KB)
static_assert(kSigSpan * 8 == 0x8000, "sign bit is the offset of the negative half");

// Byte offsets of the table entries for the two BF16 gates of w, in the
// matching halves of the result. Both halves are done at once in packed
// 16-bit arithmetic: magnitude bits less kSigLo saturating at 0
// (v_pk_sub_u16 with clamp), capped at kSigSpan - 1 (v_pk_min_u16), times 8
// (at most 15 bits, so one 32-bit shift cannot carry across halves), and the
// sign bits kept in place.
__device__ __forceinline__ uint32_t sigma_offsets(uint32_t w)
{
    typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
    const u16x2 lo = {(unsigned short)kSigLo, (unsigned short)kSigLo};
    const u16x2 top = {(unsigned short)(kSigSpan - 1), (unsigned short)(kSigSpan - 1)};
    u16x2 m = __builtin_bit_cast(u16x2, w & 0x7fff7fffu);
    m = __builtin_elementwise_min(__builtin_elementwise_sub_sat(m, lo), top);
    return (__builtin_bit_cast(uint32_t, m) << 3) | (w & 0x80008000u);
}

// The SwiGLU value from gu = RN32(g u) and the binary64 sigma:
// RN32(RN64(gu sigma)). g u of two BF16 numbers (8 significant bits each) is
// exact in binary32 for 2^-126 <= |g u| < 2^128; then the only errors before
// the final rounding are that of sigma (2^-53 relative) and of the binary64
// product, and the result is RN32(g u sigma) unless that lies within about
// 2^-52 (relative) of a binary32 rounding midpoint. Below 2^-126, gu is off
// by at most 2^-150 and so is the product (sigma < 1): the result is then
// within one subnormal step (2^-149) of RN32(g u sigma). A g u beyond the
// binary32 range is +-inf here (the callers redo those with swiglu). g u =
// -0 gives -0; the table never holds a zero sigma.
__device__ __forceinline__ float swiglu_product(float gu, double sigma)
{
    return (float)((double)gu * sigma);
}

// RN32(RN64(RN64(g u) sigma)) with g u formed in binary64, where it is exact
// for any BF16 g and u (|g u| < 2^256): the rounding of swiglu_product at
// every magnitude, infinite and NaN inputs following IEEE.
__device__ __forceinline__ float swiglu(float g, float u, double sigma)
{
    return (float)(((double)g * (double)u) * sigma);
}

// ---- FP8 E4M3 ("fn") encode of a non-negative block scale -------------------
// Saturates at 448 (exp 15 / mant 6; exp 15 / mant 7 is NaN and never made).
// v < 2^-6 is subnormal, value m / 512: m = rint(v * 512) (exact product,
// ties to even; m == 8 is the smallest normal, code 0x08 as well).
// Otherwise round the binary32 mantissa to 3 bits, ties to even, by adding
// 0x7ffff plus the kept LSB; a carry out of the mantissa moves into the
// exponent by itself (250 -> 256 = 0x78); rebias 127 -> 7.
__device__ __forceinline__ uint32_t fp8_e4m3_encode(float v)
{
    v = fminf(v, 448.0f);
    const uint32_t sub = (uint32_t)__builtin_rintf(v * 512.0f);
    const uint32_t b = __float_as_uint(v);
    const uint32_t nrm = ((b + 0x7ffffu + ((b >> 20) & 1u)) >> 20) - (120u << 3);
    return v < 0x1p-6f ? sub : nrm;
}

// ---- FP8 E4M3 decode (finite codes 0x00..0x7e) -----------------------------
// e == 0: m / 512; else 2^(e-7) (1 + m/8), built directly as binary32 bits.
__device__ __forceinline__ float fp8_e4m3_decode(uint32_t code)
{
    const uint32_t e = code >> 3;
    const uint32_t m = code & 7u;
    const float nrm = __uint_as_float(((e + 120u) << 23) | (m << 20));
    const float sub = (float)m * 0x1p-9f;
    return e ? nrm : sub;
}

// Per-block constants of the element quantizer.
struct BlockScale {
    uint32_t sf;    // E4M3 scale byte
    float half_d;   // d / 2, d = RN(decode(sf) * gs)
    float rcp;      // within one ulp of 2 / d; 0 when d == 0
    bool div_ok;    // rcp serves div_rn: RN(2 / d), or d/2 has an E4M3 significand
};

// Per-row constants: k = RN(6 gs), rk = RN(1 / k) (IEEE division), and
// whether gs is a power of two (then every block divisor d = decode(sf) * gs
// carries an E4M3 mantissa).
struct RowScale {
    float gs, k, rk;
    bool pow2;
};

__device__ __forceinline__ RowScale row_scale(float gs)
{
    RowScale r;
    r.gs = gs;
    r.k = 6.0f * gs;
    r.rk = 1.0f / r.k;
    r.pow2 = (__float_as_uint(gs) & 0x007fffffu) == 0;
    return r;
}

// Correctly rounded quotient a / b from a reciprocal rb of b: q0 = RN(a rb),
// then one Newton/Markstein correction with the exact remainder. The
// remainder is formed as q0 b - a and applied with -rb, which keeps the IEEE
// sign of a in the result also when a is -0 or the quotient underflows.
// Checked exhaustively, for quotients whose intermediates stay in the
// normal binary32 range (the result then depends only on the two
// significands):
//   * rb = RN(1 / b) for every pair of binary32 significands (2^46 pairs, on
//     the GPU against the remainder criterion of correct rounding);
//   * rb = RN(1 / b) and both of its neighbours (a faithful reciprocal such
//     as v_rcp_f32) for every numerator significand against the 8 E4M3
//     significands as divisors (on the CPU against IEEE division).
__device__ __forceinline__ float div_rn(float a, float b, float rb)
{
    const float q0 = a * rb;
    const float rem = __builtin_fmaf(q0, b, -a);
    return __builtin_fmaf(rem, -rb, q0);
}

// amax -> scale byte and element-quantizer constants.
//   bsf = RN(amax / k), sf = E4M3(bsf), d = RN(decode(sf) * gs).
// amax is first capped at 1024 k (an exact power-of-two multiple): every
// amax above it has bsf >= 1024 and saturates to 448 anyway, and the cap
// keeps the quotient finite for an infinite amax. rk = RN(1 / k) is an IEEE
// division. The element quotients need a reciprocal of d/2. When gs is a
// power of two, d/2 has an E4M3 significand, for which div_rn is exact even
// with the faithful v_rcp_f32 as the reciprocal. Otherwise div_rn needs the
// correctly rounded IEEE division, which the exact path of half_steps16
// computes itself when it runs; the guarded fast path (kFast) only needs a
// reciprocal within one ulp, so with kLazyDiv the block takes v_rcp_f32 for
// every gs and leaves the division to the blocks that fall back (the GEMM
// epilogue, short of registers, divides up front instead). The branch is
// uniform (gs is per row). Both hold for gs in [2^-64, 2^64], where every
// remainder stays in the normal range.
template <bool kLazyDiv>
__device__ __forceinline__ BlockScale block_scale(float amax, const RowScale& rs)
{
    BlockScale s;
    const float a = __builtin_fminf(amax, 1024.0f * rs.k);
    const float bsf = div_rn(a, rs.k, rs.rk);
    s.sf = fp8_e4m3_encode(bsf);
    const float d = fp8_e4m3_decode(s.sf) * rs.gs;
    s.half_d = 0.5f * d;
    float r;
    if (kLazyDiv || rs.pow2)
        r = __builtin_amdgcn_rcpf(s.half_d);
    else
        r = 1.0f / s.half_d;                  // IEEE division, correctly rounded
    s.rcp = d != 0.0f ? r : 0.0f;
    s.div_ok = !kLazyDiv || rs.pow2;
    return s;
}

// One element -> signed half-step count +-rint(2|s|), s = RN(x / d), ties to
// even. 2s = RN(2x / d) = RN(x / (d/2)) exactly (power-of-two scaling); rint
// keeps the IEEE sign of x, including -0 and values that round to 0. When
// d == 0, rcp == 0 gives +-0. The clamp 2 min(|s|, 6) of the method is left
// to the E2M1 convert, which saturates: any count >= 12 (|s| >= 6) gives the
// largest magnitude, exactly as the clamped count 12 does.
__device__ __forceinline__ float half_steps(float x, const BlockScale& s)
{
    return __builtin_rintf(div_rn(x, s.half_d, s.rcp));
}

// Largest distance of a fast quotient from its nearest integer that
// half_steps16 accepts: 2^-17 short of a half (a possible tie).
constexpr float kTieGuard = 0.5f - 0x1p-17f;

// The 16 counts of a block. Fast path: q0 = RN(y rcp), one product in place
// of the correctly rounded q = 2y/d. rcp is within one ulp of 2/d and q0 adds
// one rounding, so |q0 - RN(q)| <= |q| 2^-22 (both in the normal range; a q0
// below it is a zero count on both sides, with the sign of y):
//   * for |q| < 16 that is below 2^-18, so when q0 lies more than 2^-17 from
//     every half-integer, RN(q) lies strictly on the same side of each of
//     them, and rint(q0) == rint(RN(q)), sign included;
//   * for |q| >= 16 both counts are at least 15 in magnitude, with the sign
//     of y, and the E2M1 convert saturates them to the same code.
// So the fast counts are taken when every |q0 - rint(q0)| of the block is
// below kTieGuard. Otherwise (a value near a possible tie, or a non-finite
// q0: an infinite value, or an overflowed product) the block takes the exact
// path. The fast path pays for FP32 values with full significands (SwiGLU
// products, GEMM accumulators), whose quotients come near a half-integer
// about 2^-16 of the time; BF16 values (8 significant bits) over E4M3
// divisors land exactly on one for a few percent of elements, so their
// callers ask for the exact path alone (kFast = false). The exact path:
// div_rn per value, and when amax / (d/2) may exceed 16 (a saturated
// scale, or an infinite value) the values are first clamped to
// [-16 d/2, 16 d/2] (v_med3_f32 returns x itself inside the range): every
// such value has |s| > 6 and keeps its largest-magnitude code and its sign,
// and no quotient overflows (an overflowed q0 would turn the correction into
// inf - inf). amax * rcp is within 2 ulp of amax / (d/2), and 0 when d == 0
// (rcp == 0 makes every count +-0 on both paths).
template <bool kFast>
__device__ __forceinline__ void half_steps16(const float (&y)[16], float amax,
                                             const BlockScale& s, float (&h)[16])
{
    float far = __builtin_inff();
    if constexpr (kFast) {
        far = 0.0f;
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            const float q0 = y[j] * s.rcp;
            h[j] = __builtin_rintf(q0);
            far = __builtin_elementwise_maximum(far, __builtin_fabsf(q0 - h[j]));
        }
    }
    if (!(far < kTieGuard)) {
        BlockScale e = s;
        if (!e.div_ok)
            e.rcp = e.half_d != 0.0f ? 1.0f / e.half_d : 0.0f;   // IEEE division
#pragma unroll
        for (int j = 0; j < 16; ++j)
            h[j] = half_steps(y[j], e);
        if (amax * e.rcp > 16.0f) {
            const float lim = 16.0f * e.half_d;
#pragma unroll
            for (int j = 0; j < 16; ++j)
                h[j] = half_steps(__builtin_amdgcn_fmed3f(y[j], -lim, lim), e);
        }
    }
}

// Two signed half-step counts -> one byte of E2M1 codes (first value in the
// low nibble) placed at byte `sel` of `word`. The convert divides by its
// power-of-two scale (2 here, exact) and rounds to nearest even onto E2M1,
// saturating at 6: on the half-step grid {0, .5, ..., 6} that is exactly the
// step_to_idx table (2.5 -> 2, 3.5 -> 4, 4.5 -> 4, 5 -> 4, 5.5 -> 6), and
// every value above 6 gives 6; the sign (also of -0) becomes bit 3.
template <int sel>
__device__ __forceinline__ uint32_t pack_e2m1(uint32_t word, float h0, float h1)
{
    return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(word, h0, h1, 2.0f, sel);
}

// max |y_j| of a block (exact), NaN if some y_j is NaN (v_maximum3_f32
// propagates NaN, unlike v_max3_f32).
__device__ __forceinline__ float block_amax(const float (&y)[16])
{
    float amax = 0.0f;
#pragma unroll
    for (int j = 0; j < 16; ++j)
        amax = __builtin_elementwise_maximum(amax, __builtin_fabsf(y[j]));
    return amax;
}

// 16 FP32 values and their amax -> 8 bytes of packed E2M1 codes (returned
// as uint2) and the scale byte; kFast as in half_steps16, kLazyDiv as in
// block_scale (only with kFast).
template <bool kFast, bool kLazyDiv = kFast>
__device__ __forceinline__ uint2 quantize16(const float (&y)[16], float amax, const RowScale& rs,
                                            uint32_t& sf_out)
{
    static_assert(kFast || !kLazyDiv, "the exact path needs the divided reciprocal");
    const BlockScale s = block_scale<kLazyDiv>(amax, rs);
    float h[16];
    half_steps16<kFast>(y, amax, s, h);
    uint32_t w0 = 0, w1 = 0;
    w0 = pack_e2m1<0>(w0, h[0], h[1]);
    w0 = pack_e2m1<1>(w0, h[2], h[3]);
    w0 = pack_e2m1<2>(w0, h[4], h[5]);
    w0 = pack_e2m1<3>(w0, h[6], h[7]);
    w1 = pack_e2m1<0>(w1, h[8], h[9]);
    w1 = pack_e2m1<1>(w1, h[10], h[11]);
    w1 = pack_e2m1<2>(w1, h[12], h[13]);
    w1 = pack_e2m1<3>(w1, h[14], h[15]);
    sf_out = s.sf;
    return make_uint2(w0, w1);
}

// Byte `sel` of `word` (two E2M1 codes, low nibble first) -> two FP32
// values RN(RN(e2m1 * dec) * gs). The convert with scale 1 is exact.
template <int sel>
__device__ __forceinline__ void dequant_byte(uint32_t word, float dec, float gs, float* out)
{
    const auto v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(word, 1.0f, sel);
    out[0] = (v[0] * dec) * gs;
    out[1] = (v[1] * dec) * gs;
}

// 8 packed bytes + scale -> 16 dequantized FP32 values:
// RN(RN(e2m1 * decode(sf)) * gs); the inner product is exact.
__device__ __forceinline__ void dequantize16(uint2 packed, uint32_t sf, float gs,
                                             float* out)
{
    const float dec = fp8_e4m3_decode(sf);
    dequant_byte<0>(packed.x, dec, gs, out + 0);
    dequant_byte<1>(packed.x, dec, gs, out + 2);
    dequant_byte<2>(packed.x, dec, gs, out + 4);
    dequant_byte<3>(packed.x, dec, gs, out + 6);
    dequant_byte<0>(packed.y, dec, gs, out + 8);
    dequant_byte<1>(packed.y, dec, gs, out + 10);
    dequant_byte<2>(packed.y, dec, gs, out + 12);
    dequant_byte<3>(packed.y, dec, gs, out + 14);
}

// Global scale of a row: gs[0], or gs[e] of the expert holding the row
// (largest e with offsets[e] <= row), or 1.0 without gs. `row` is
// wave-uniform, so the search runs on scalar registers and loads.
__device__ __forceinline__ float row_global_scale(const float* gs, const int32_t* offsets,
                                                  int num_experts, int row)
{
    int e = 0;
    if (offsets != nullptr) {
        int lo = 0, hi = num_experts;
        while (hi - lo > 1) {
            const int mid = (lo + hi) >> 1;
            if (offsets[mid] <= row)
                lo = mid;
            else
                hi = mid;
        }
        e = lo;
    }
    return gs != nullptr ? gs[e] : 1.0f;
}

}  // namespace nvfp4
