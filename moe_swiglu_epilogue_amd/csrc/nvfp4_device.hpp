// Device-side arithmetic of NVFP4 block quantization for gfx950.
//
// Method: "nvfp4-megamoe-kernel" project log (2026-05-28),
// "NVFP4-1.1_APPROACH_PART_2.md" (FP8 E4M3 scale rules, half-step E2M1
// rounding, fused-epilogue design) and "2026-05-28_STATUS.md" (the commit
// listing the quantization primitives and their five fixes).
//
// Every function here reproduces the binary32 definition of the method
// exactly (bit for bit), except times_sigma(), the SwiGLU product through the
// sigmoid table, which is the binary32 rounding of g * u * sigmoid(g) except
// within about 2^-46 of a rounding midpoint.
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
// and both signs, each entry a pair of floats hi = sigma rounded toward zero,
// lo = RN(sigma - hi) >= 0 (8 bytes; hi + lo carries sigma to about 2^-47). Positive
// gates use entries [0, kSigSpan), negative ones [kSigSpan, 2 kSigSpan):
// kSigSpan * 8 = 32768 is bit 15 of a BF16 half-word, so the sign bit serves
// as the sign's byte offset where it stands. Magnitudes below the range read
// the first entry (sigma = 1/2 +- 2^-26 +- ... there), magnitudes above it the
// last (sigma is 1 to within 2^-367, or below 2^-367 for negative g). The
// entries are computed at build time (gen_sigma_table.py) and copied into
// LDS once per workgroup; a lookup then replaces exp and rcp per element.
constexpr uint32_t kSigLo = 103u << 7;
constexpr uint32_t kSigHi = (134u << 7) | 127u;
constexpr int kSigSpan = (int)(kSigHi - kSigLo + 1);   // 4096
constexpr int kSigFloats = 4 * kSigSpan;                // 16384 (64 KB)
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

// (g u) sigma for a table entry {hi, lo}: g u is exact in FP32 for BF16 g and
// u (8 significant bits each); fma adds (g u) hi and RN((g u) lo) exactly and
// rounds once, so the result is RN((g u) sigma) unless (g u) sigma lies
// within about 2^-46 (relative) of a rounding midpoint. hi and lo are both
// >= 0, so both terms carry the sign of g u: g u = -0 gives -0, and a g u
// that overflowed to +-inf gives +-inf (a negative lo would add -0 to -0
// as +0, or make inf - inf).
__device__ __forceinline__ float times_sigma(float gu, float2 s)
{
    return __builtin_fmaf(gu, s.x, gu * s.y);
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
    uint32_t sf;   // E4M3 scale byte
    float half_d;  // d / 2, d = RN(decode(sf) * gs)
    float rcp;     // RN(1 / half_d) = RN(2 / d); 0 when d == 0
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

// Correctly rounded quotient a / b from rb = RN(1 / b): q0 = RN(a rb), then
// one Newton/Markstein correction with the exact remainder. The remainder is
// formed as q0 b - a and applied with -rb, which keeps the IEEE sign of a in
// the result also when a is -0 or the quotient underflows. Checked
// exhaustively on the CPU for every binary32 numerator mantissa against the
// 8 E4M3 mantissas as divisors (the power-of-two global-scale case); in
// general it is Markstein's theorem (rb within half an ulp of 1/b, q0
// faithful, exact remainder).
__device__ __forceinline__ float div_rn(float a, float b, float rb)
{
    const float q0 = a * rb;
    const float rem = __builtin_fmaf(q0, b, -a);
    return __builtin_fmaf(rem, -rb, q0);
}

// amax -> scale byte and element-quantizer constants.
//   bsf = RN(amax / k), sf = E4M3(bsf), d = RN(decode(sf) * gs).
// The element quotients need a reciprocal of d/2 for div_rn. When gs is a
// power of two, d/2 has one of the 8 E4M3 mantissas, and for those divisors
// the div_rn correction is exact for every numerator even when the
// reciprocal is off by one ulp (checked exhaustively on the CPU), so the
// faithful v_rcp_f32 is enough. Otherwise the reciprocal is the correctly
// rounded IEEE division. The branch is uniform (gs is per row).
__device__ __forceinline__ BlockScale block_scale(float amax, const RowScale& rs)
{
    BlockScale s;
    const float bsf = div_rn(amax, rs.k, rs.rk);
    s.sf = fp8_e4m3_encode(bsf);
    const float d = fp8_e4m3_decode(s.sf) * rs.gs;
    s.half_d = 0.5f * d;
    float r;
    if (rs.pow2)
        r = __builtin_amdgcn_rcpf(s.half_d);
    else
        r = 1.0f / s.half_d;                  // IEEE division, correctly rounded
    s.rcp = d != 0.0f ? r : 0.0f;
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

// 16 FP32 values -> 8 bytes of packed E2M1 codes (returned as uint2) and the
// scale byte.
__device__ __forceinline__ uint2 quantize16(const float (&y)[16], const RowScale& rs,
                                            uint32_t& sf_out)
{
    float amax = 0.0f;
#pragma unroll
    for (int j = 0; j < 16; ++j)
        amax = fmaxf(amax, __builtin_fabsf(y[j]));
    const BlockScale s = block_scale(amax, rs);
    float h[16];
#pragma unroll
    for (int j = 0; j < 16; ++j)
        h[j] = half_steps(y[j], s);
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
