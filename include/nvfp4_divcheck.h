/*
 * nvfp4_divcheck.h - C ABI of libnvfp4_divcheck.so, an exhaustive check of
 * the quotient sequence the NVFP4 kernels use (nvfp4_device.hpp div_rn):
 * q0 = RN(a rb), rem = RN(q0 b - a), q = RN(q0 - rem rb) with rb = RN(1 / b)
 * (an IEEE division). Test and verification code, not part of the NVFP4 path.
 *
 * The quantizer's quotients (block scale amax / (6 gs) and element value
 * / (scale / 2)) are correctly rounded only if this sequence is. While every
 * intermediate stays in the normal binary32 range, scaling a or b by a power
 * of two scales every step exactly, so the result depends only on the two
 * significands: checking every pair a, b in [1, 2) covers every such
 * quotient. A quotient q is accepted when it is the correctly rounded a / b by
 * the remainder criterion: r = a - q b (exact in an fma for q within a few
 * ulp), |r| < b ulp(q) / 2, or |r| equal to it with an even significand of q
 * (with the half gap below q when q is a power of two and the quotient lies
 * below it).
 *
 *   nvfp4_divcheck(b_first, b_count, naive, fails, witness, stream)
 *     checks every numerator significand (2^23 of them) against the divisor
 *     significands b_first .. b_first + b_count - 1 (b = 1 + m 2^-23, m < 2^23)
 *     and adds the number of failing pairs to *fails (device uint64). On a
 *     failure *witness (device uint64) receives the smallest failing
 *     (m_b << 23) | m_a; initialise it to UINT64_MAX. naive != 0 checks the
 *     uncorrected q0 instead (it fails for many pairs: a check that the check
 *     can fail). One kernel on `stream`, one 256-thread workgroup per divisor.
 *     Returns 0, 1 for invalid arguments (b_count < 1, the range beyond 2^23,
 *     NULL pointers; checked before any HIP call), 4 for a launch failure.
 */
#ifndef NVFP4_DIVCHECK_H
#define NVFP4_DIVCHECK_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

int nvfp4_divcheck(uint32_t b_first, uint32_t b_count, int naive, uint64_t *fails,
                   uint64_t *witness, hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* NVFP4_DIVCHECK_H */
