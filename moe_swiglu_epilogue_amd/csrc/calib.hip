// libnvfp4_calib.so: bandwidth calibration kernels for gfx950 (declared in
// include/nvfp4_calib.h). They move a known number of bytes with the same
// access style as the NVFP4 kernels (16-byte non-temporal lane accesses,
// wave64, 256-thread workgroups), so that their timings give the achievable
// HBM ceiling and their rocprofv3 FETCH_SIZE / WRITE_SIZE readings give the
// counter-to-bytes scale used to turn counters into HBM traffic.
#include "../../include/nvfp4_calib.h"

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
constexpr int kThreads = 256;
constexpr int kWavesPerBlock = kThreads / 64;
constexpr int kTileWords = 256;     // 4 KB per wave tile, 4 coalesced 1 KB loads

// dst[i] = src[i] for n16 16-byte words; wave tiles of 256 words, word
// j*64 + lane of the tile in instruction j.
__global__ __launch_bounds__(kThreads) void calib_copy_kernel(const u32x4* __restrict__ src,
                                                              u32x4* __restrict__ dst, int64_t n16)
{
    const int lane = threadIdx.x & 63;
    const int64_t wave = blockIdx.x * (int64_t)kWavesPerBlock + (threadIdx.x >> 6);
    const int64_t stride = (int64_t)gridDim.x * kWavesPerBlock;
    for (int64_t base = wave * kTileWords; base < n16; base += stride * kTileWords) {
        u32x4 v[4];
#pragma unroll
        for (int j = 0; j < 4; ++j)
            if (base + j * 64 + lane < n16)
                v[j] = __builtin_nontemporal_load(src + base + j * 64 + lane);
#pragma unroll
        for (int j = 0; j < 4; ++j)
            if (base + j * 64 + lane < n16)
                __builtin_nontemporal_store(v[j], dst + base + j * 64 + lane);
    }
}

// out[block] = xor of every 16-byte word the workgroup read (keeps the loads
// alive); reads n16 words with the same tile pattern, writes one word per
// workgroup.
__global__ __launch_bounds__(kThreads) void calib_read_kernel(const u32x4* __restrict__ src,
                                                              u32x4* __restrict__ out, int64_t n16)
{
    __shared__ u32x4 part[kThreads];
    u32x4 acc = {0u, 0u, 0u, 0u};
    const int lane = threadIdx.x & 63;
    const int64_t wave = blockIdx.x * (int64_t)kWavesPerBlock + (threadIdx.x >> 6);
    const int64_t stride = (int64_t)gridDim.x * kWavesPerBlock;
    for (int64_t base = wave * kTileWords; base < n16; base += stride * kTileWords) {
        u32x4 v[4] = {};
#pragma unroll
        for (int j = 0; j < 4; ++j)
            if (base + j * 64 + lane < n16)
                v[j] = __builtin_nontemporal_load(src + base + j * 64 + lane);
        acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
    }
    part[threadIdx.x] = acc;
    __syncthreads();
    for (int s = kThreads / 2; s > 0; s >>= 1) {
        if (threadIdx.x < s)
            part[threadIdx.x] ^= part[threadIdx.x + s];
        __syncthreads();
    }
    if (threadIdx.x == 0)
        out[blockIdx.x] = part[0];
}

// The fused quantize kernel's traffic mix without its compute: per 4 KB
// tile of src (one wave: four coalesced 1 KB non-temporal loads) a 576-byte
// piece of dst (lanes 0..35, 16 bytes each, through a buffer resource that
// drops the other lanes' stores, with the fused kernel's sc0 sc1 policy).
// One tile per wave and no loop: the hardware dispatches the workgroups in
// order, which measured fastest for this mix. Dynamic LDS, never touched,
// caps the workgroups per CU.
constexpr int kMixTileBytes = 4096;
constexpr int kMixOutBytes = 576;

__global__ __launch_bounds__(kThreads) void calib_mix_kernel(const u32x4* __restrict__ src,
                                                             uint8_t* __restrict__ dst, int64_t tiles)
{
    const int lane = threadIdx.x & 63;
    const int64_t t = blockIdx.x * (int64_t)kWavesPerBlock + (threadIdx.x >> 6);
    if (t >= tiles)
        return;
    const u32x4* in = src + t * (kMixTileBytes / 16);
    u32x4 v[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
        v[j] = __builtin_nontemporal_load(in + j * 64 + lane);
    const u32x4 x = v[0] ^ v[1] ^ v[2] ^ v[3];
    const __amdgpu_buffer_rsrc_t out =
        __builtin_amdgcn_make_buffer_rsrc(dst + t * kMixOutBytes, (short)0, kMixOutBytes, 0x00020000);
    __builtin_amdgcn_raw_buffer_store_b128(x, out, lane * 16, 0, 17);
}

}  // namespace

extern "C" {

int nvfp4_calib_copy(const void* src, void* dst, int64_t bytes, int32_t blocks, hipStream_t stream)
{
    if (bytes < 0 || bytes % 16 != 0 || blocks < 1 || ((uintptr_t)src | (uintptr_t)dst) % 16)
        return 1;
    if (bytes == 0)
        return 0;
    hipLaunchKernelGGL(calib_copy_kernel, dim3(blocks), dim3(kThreads), 0, stream,
                       (const u32x4*)src, (u32x4*)dst, bytes / 16);
    return hipGetLastError() == hipSuccess ? 0 : 4;
}

int nvfp4_calib_read(const void* src, void* out, int64_t bytes, int32_t blocks, hipStream_t stream)
{
    if (bytes < 0 || bytes % 16 != 0 || blocks < 1 || ((uintptr_t)src | (uintptr_t)out) % 16)
        return 1;
    if (bytes == 0)
        return 0;
    hipLaunchKernelGGL(calib_read_kernel, dim3(blocks), dim3(kThreads), 0, stream,
                       (const u32x4*)src, (u32x4*)out, bytes / 16);
    return hipGetLastError() == hipSuccess ? 0 : 4;
}

int nvfp4_calib_mix(const void* src, void* dst, int64_t bytes, int32_t lds_bytes, hipStream_t stream)
{
    if (bytes < 0 || bytes % kMixTileBytes != 0 || lds_bytes < 0 || lds_bytes > 65536 ||
        ((uintptr_t)src | (uintptr_t)dst) % 16)
        return 1;
    const int64_t tiles = bytes / kMixTileBytes;
    const int64_t blocks = (tiles + kWavesPerBlock - 1) / kWavesPerBlock;
    if (blocks > INT32_MAX)
        return 1;
    if (tiles == 0)
        return 0;
    hipLaunchKernelGGL(calib_mix_kernel, dim3((unsigned)blocks), dim3(kThreads), lds_bytes, stream,
                       (const u32x4*)src, (uint8_t*)dst, tiles);
    return hipGetLastError() == hipSuccess ? 0 : 4;
}

}  // extern "C"
