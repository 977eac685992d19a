// libnvfp4_divcheck.so: exhaustive check of the quantizer's quotient
// sequence (nvfp4::div_rn with a correctly rounded reciprocal) over every
// pair of binary32 significands, declared in include/nvfp4_divcheck.h.
// Verification code: the NVFP4 path does not use it.
#include "../../include/nvfp4_divcheck.h"
#include "nvfp4_device.hpp"

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr int kThreads = 256;
constexpr uint32_t kOne = 0x3f800000u;
constexpr uint32_t kSig = 1u << 23;

// true when q is RN(a / b), by the remainder criterion (see the header)
__device__ __forceinline__ bool correctly_rounded(float a, float b, float q)
{
    const float r = __builtin_fmaf(-q, b, a);              // a - q b, exact
    const uint32_t qb = __float_as_uint(q);
    const int e = (int)(qb >> 23) - 127;                    // q is normal and positive
    float half_gap = __builtin_ldexpf(b, e - 24);           // b ulp(q) / 2, exact
    if ((qb & 0x7fffffu) == 0u && r < 0.0f)                 // below a power of two
        half_gap *= 0.5f;
    const float ar = __builtin_fabsf(r);
    return ar < half_gap || (ar == half_gap && (qb & 1u) == 0u);
}

__global__ __launch_bounds__(kThreads) void divcheck_kernel(uint32_t b_first, int naive,
                                                            unsigned long long* fails,
                                                            unsigned long long* witness)
{
    const uint32_t mb = b_first + blockIdx.x;
    const float b = __uint_as_float(kOne | mb);
    const float rb = 1.0f / b;                               // IEEE division
    uint32_t bad = 0;
    uint32_t first = kSig;
    for (uint32_t ma = threadIdx.x; ma < kSig; ma += kThreads) {
        const float a = __uint_as_float(kOne | ma);
        const float q = naive ? a * rb : nvfp4::div_rn(a, b, rb);
        if (!correctly_rounded(a, b, q)) {
            ++bad;
            first = first < ma ? first : ma;
        }
    }
    if (bad != 0u) {
        atomicAdd(fails, (unsigned long long)bad);
        atomicMin(witness, ((unsigned long long)mb << 23) | first);
    }
}

}  // namespace

extern "C" int nvfp4_divcheck(uint32_t b_first, uint32_t b_count, int naive, uint64_t* fails,
                              uint64_t* witness, hipStream_t stream)
{
    if (b_count < 1 || b_first >= kSig || b_count > kSig - b_first || !fails || !witness)
        return 1;
    hipLaunchKernelGGL(divcheck_kernel, dim3(b_count), dim3(kThreads), 0, stream, b_first, naive,
                       reinterpret_cast<unsigned long long*>(fails),
                       reinterpret_cast<unsigned long long*>(witness));
    return hipGetLastError() == hipSuccess ? 0 : 4;
}
