// libmoe_nvfp4.so: HIP kernels for gfx950 and the C ABI declared in
// include/moe_nvfp4.h.
//
// Work decomposition (all three kernels): one lane owns one NVFP4 block of
// 16 output values; one wave64 owns a "tile" of 64 consecutive blocks of one
// row, so the row index, its global scale and its base addresses are
// wave-uniform (scalar registers). Tiles are numbered row-major and handed
// to waves with a grid-stride loop.
//
// Method: "nvfp4-megamoe-kernel" log, "NVFP4-1.1_APPROACH_PART_2.md"
// (fused-epilogue design: SiLU(gate) and SwiGLU in FP32 registers, every two
// 8-wide up subtiles form one 16-value FP4 block: amax, FP8 scale, E2M1
// pack, 8 + 1 bytes per block) and "NVFP4-1.1_APPROACH.md" (interleaved
// [gate x8, up x8] L1 output).
#include "../../include/moe_nvfp4.h"
#include "nvfp4_device.hpp"

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr int kWave = 64;
constexpr int kWavesPerBlock = 4;
constexpr int kThreads = kWave * kWavesPerBlock;
constexpr int kTileBlocks = kWave;   // NVFP4 blocks per wave tile

struct Geometry {
    int rows;
    int bpr;          // NVFP4 blocks per row
    int cpr;          // tiles (chunks of 64 blocks) per row
    int tiles;        // rows * cpr
};

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

// Streaming (read-once / write-once) accesses: non-temporal hint.
__device__ __forceinline__ u32x4 ld_stream(const u32x4* p) { return __builtin_nontemporal_load(p); }
__device__ __forceinline__ u32x2 ld_stream(const u32x2* p) { return __builtin_nontemporal_load(p); }
__device__ __forceinline__ void st_stream(f32x4 v, f32x4* p) { __builtin_nontemporal_store(v, p); }

// ---------------------------------------------------------------------------
// Fused SwiGLU + NVFP4 quantize.
// Lane input: 64 contiguous bytes = [g0..7][u0..7][g8..15][u8..15] (BF16).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kThreads) void swiglu_nvfp4_kernel(
    const uint16_t* __restrict__ in, int64_t ld_in, Geometry geo,
    const float* __restrict__ gs, const int32_t* __restrict__ offsets, int num_experts,
    uint8_t* __restrict__ packed, uint8_t* __restrict__ scales,
    float* __restrict__ swiglu_out)
{
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = uniform(threadIdx.x / kWave);
    const int inter = geo.bpr * 16;
    for (int tile = blockIdx.x * kWavesPerBlock + wave; tile < geo.tiles;
         tile += gridDim.x * kWavesPerBlock) {
        const int row = uniform(tile / geo.cpr);
        const int chunk = tile - row * geo.cpr;
        const int blk = chunk * kTileBlocks + lane;
        if (blk >= geo.bpr)
            continue;
        const u32x4* src = reinterpret_cast<const u32x4*>(in + (int64_t)row * ld_in + (int64_t)blk * 32);
        const u32x4 c0 = ld_stream(src + 0);
        const u32x4 c1 = ld_stream(src + 1);
        const u32x4 c2 = ld_stream(src + 2);
        const u32x4 c3 = ld_stream(src + 3);
        const float g_s = nvfp4::row_global_scale(gs, offsets, num_experts, row);
        const float k = 6.0f * g_s;

        const uint32_t gw[8] = {c0.x, c0.y, c0.z, c0.w, c2.x, c2.y, c2.z, c2.w};
        const uint32_t uw[8] = {c1.x, c1.y, c1.z, c1.w, c3.x, c3.y, c3.z, c3.w};
        float y[16];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            y[2 * i] = nvfp4::swiglu(nvfp4::bf16_lo(gw[i]), nvfp4::bf16_lo(uw[i]));
            y[2 * i + 1] = nvfp4::swiglu(nvfp4::bf16_hi(gw[i]), nvfp4::bf16_hi(uw[i]));
        }
        uint32_t sf;
        const uint2 q = nvfp4::quantize16(y, g_s, k, sf);
        const int64_t ob = (int64_t)row * geo.bpr + blk;
        *reinterpret_cast<uint2*>(packed + ob * 8) = q;
        scales[ob] = (uint8_t)sf;
        if (swiglu_out != nullptr) {
            float4* dst = reinterpret_cast<float4*>(swiglu_out + (int64_t)row * inter + (int64_t)blk * 16);
#pragma unroll
            for (int i = 0; i < 4; ++i)
                dst[i] = make_float4(y[4 * i], y[4 * i + 1], y[4 * i + 2], y[4 * i + 3]);
        }
    }
}

// ---------------------------------------------------------------------------
// Standalone NVFP4 quantize of BF16. Lane input: 32 contiguous bytes.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kThreads) void nvfp4_quantize_kernel(
    const uint16_t* __restrict__ x, int64_t ld_x, Geometry geo,
    const float* __restrict__ gs, const int32_t* __restrict__ offsets, int num_experts,
    uint8_t* __restrict__ packed, uint8_t* __restrict__ scales)
{
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = uniform(threadIdx.x / kWave);
    for (int tile = blockIdx.x * kWavesPerBlock + wave; tile < geo.tiles;
         tile += gridDim.x * kWavesPerBlock) {
        const int row = uniform(tile / geo.cpr);
        const int chunk = tile - row * geo.cpr;
        const int blk = chunk * kTileBlocks + lane;
        if (blk >= geo.bpr)
            continue;
        const u32x4* src = reinterpret_cast<const u32x4*>(x + (int64_t)row * ld_x + (int64_t)blk * 16);
        const u32x4 a = ld_stream(src + 0);
        const u32x4 b = ld_stream(src + 1);
        const float g_s = nvfp4::row_global_scale(gs, offsets, num_experts, row);
        const float k = 6.0f * g_s;
        const uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
        float v[16];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            v[2 * i] = nvfp4::bf16_lo(w[i]);
            v[2 * i + 1] = nvfp4::bf16_hi(w[i]);
        }
        uint32_t sf;
        const uint2 q = nvfp4::quantize16(v, g_s, k, sf);
        const int64_t ob = (int64_t)row * geo.bpr + blk;
        *reinterpret_cast<uint2*>(packed + ob * 8) = q;
        scales[ob] = (uint8_t)sf;
    }
}

// ---------------------------------------------------------------------------
// NVFP4 dequantize to FP32. Lane output: 64 contiguous bytes.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kThreads) void nvfp4_dequantize_kernel(
    const uint8_t* __restrict__ packed, const uint8_t* __restrict__ scales, Geometry geo,
    const float* __restrict__ gs, const int32_t* __restrict__ offsets, int num_experts,
    float* __restrict__ out)
{
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = uniform(threadIdx.x / kWave);
    const int cols = geo.bpr * 16;
    for (int tile = blockIdx.x * kWavesPerBlock + wave; tile < geo.tiles;
         tile += gridDim.x * kWavesPerBlock) {
        const int row = uniform(tile / geo.cpr);
        const int chunk = tile - row * geo.cpr;
        const int blk = chunk * kTileBlocks + lane;
        if (blk >= geo.bpr)
            continue;
        const int64_t ib = (int64_t)row * geo.bpr + blk;
        const u32x2 pv = ld_stream(reinterpret_cast<const u32x2*>(packed) + ib);
        const uint2 p = make_uint2(pv.x, pv.y);
        const uint32_t sf = __builtin_nontemporal_load(scales + ib);
        const float g_s = nvfp4::row_global_scale(gs, offsets, num_experts, row);
        float v[16];
        nvfp4::dequantize16(p, sf, g_s, v);
        f32x4* dst = reinterpret_cast<f32x4*>(out + (int64_t)row * cols + (int64_t)blk * 16);
#pragma unroll
        for (int i = 0; i < 4; ++i)
            st_stream(f32x4{v[4 * i], v[4 * i + 1], v[4 * i + 2], v[4 * i + 3]}, dst + i);
    }
}

// ---------------------------------------------------------------------------
// Host side: validation (no HIP call before it passes) and launch.
// ---------------------------------------------------------------------------
bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

nvfp4_status_t check_experts(const int32_t* offsets, int32_t num_experts)
{
    if (num_experts < 0)
        return NVFP4_ERROR_INVALID_VALUE;
    if ((offsets != nullptr) != (num_experts > 0))
        return NVFP4_ERROR_INVALID_VALUE;
    return NVFP4_SUCCESS;
}

// rows, cols already validated non-negative with cols % 16 == 0.
nvfp4_status_t make_geometry(int64_t rows, int64_t cols, Geometry& g)
{
    const int64_t bpr = cols / 16;
    const int64_t cpr = (bpr + kTileBlocks - 1) / kTileBlocks;
    // tiles <= 2^30 keeps tile + grid stride inside int32 in the kernels
    if (rows > INT32_MAX || bpr > INT32_MAX / 16 || rows * cpr > (int64_t(1) << 30))
        return NVFP4_ERROR_UNSUPPORTED_SHAPE;
    g.rows = (int)rows;
    g.bpr = (int)bpr;
    g.cpr = (int)cpr;
    g.tiles = (int)(rows * cpr);
    return NVFP4_SUCCESS;
}

// One wave per tile: the grid covers every tile exactly once (the
// grid-stride loop then runs a single iteration); capped only so that the
// grid size stays a valid launch dimension.
dim3 grid_for(const Geometry& g)
{
    const int64_t want = ((int64_t)g.tiles + kWavesPerBlock - 1) / kWavesPerBlock;
    const int64_t cap = INT32_MAX / kWavesPerBlock;
    return dim3((unsigned)(want < cap ? want : cap));
}

nvfp4_status_t launched()
{
    return hipGetLastError() == hipSuccess ? NVFP4_SUCCESS : NVFP4_ERROR_LAUNCH;
}

}  // namespace

extern "C" {

nvfp4_status_t nvfp4_quantize(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld_x,
                              const float* gs, const int32_t* expert_offsets,
                              int32_t num_experts, uint8_t* packed, uint8_t* scales,
                              hipStream_t stream)
{
    if (rows < 0 || cols < 0 || ld_x < cols)
        return NVFP4_ERROR_INVALID_VALUE;
    if (cols % 16 != 0)
        return NVFP4_ERROR_UNSUPPORTED_SHAPE;
    nvfp4_status_t st = check_experts(expert_offsets, num_experts);
    if (st != NVFP4_SUCCESS)
        return st;
    if (rows == 0 || cols == 0)
        return NVFP4_SUCCESS;
    if (!x || !packed || !scales)
        return NVFP4_ERROR_INVALID_VALUE;
    if (!aligned(x, 16) || (ld_x * 2) % 16 != 0 || !aligned(packed, 8))
        return NVFP4_ERROR_MISALIGNED;
    Geometry g;
    if ((st = make_geometry(rows, cols, g)) != NVFP4_SUCCESS)
        return st;
    hipLaunchKernelGGL(nvfp4_quantize_kernel, grid_for(g), dim3(kThreads), 0, stream,
                       x, ld_x, g, gs, expert_offsets, (int)num_experts, packed, scales);
    return launched();
}

nvfp4_status_t swiglu_nvfp4_quantize(const uint16_t* gate_up, int64_t rows, int64_t inter,
                                     int64_t ld_in, const float* gs,
                                     const int32_t* expert_offsets, int32_t num_experts,
                                     uint8_t* packed, uint8_t* scales, float* swiglu_out,
                                     hipStream_t stream)
{
    if (rows < 0 || inter < 0 || inter > INT64_MAX / 2 || ld_in < 2 * inter)
        return NVFP4_ERROR_INVALID_VALUE;
    if (inter % 16 != 0)
        return NVFP4_ERROR_UNSUPPORTED_SHAPE;
    nvfp4_status_t st = check_experts(expert_offsets, num_experts);
    if (st != NVFP4_SUCCESS)
        return st;
    if (rows == 0 || inter == 0)
        return NVFP4_SUCCESS;
    if (!gate_up || !packed || !scales)
        return NVFP4_ERROR_INVALID_VALUE;
    if (!aligned(gate_up, 16) || (ld_in * 2) % 16 != 0 || !aligned(packed, 8) ||
        (swiglu_out && !aligned(swiglu_out, 16)))
        return NVFP4_ERROR_MISALIGNED;
    Geometry g;
    if ((st = make_geometry(rows, inter, g)) != NVFP4_SUCCESS)
        return st;
    hipLaunchKernelGGL(swiglu_nvfp4_kernel, grid_for(g), dim3(kThreads), 0, stream,
                       gate_up, ld_in, g, gs, expert_offsets, (int)num_experts, packed, scales,
                       swiglu_out);
    return launched();
}

nvfp4_status_t nvfp4_dequantize(const uint8_t* packed, const uint8_t* scales, int64_t rows,
                                int64_t cols, const float* gs, const int32_t* expert_offsets,
                                int32_t num_experts, float* out, hipStream_t stream)
{
    if (rows < 0 || cols < 0)
        return NVFP4_ERROR_INVALID_VALUE;
    if (cols % 16 != 0)
        return NVFP4_ERROR_UNSUPPORTED_SHAPE;
    nvfp4_status_t st = check_experts(expert_offsets, num_experts);
    if (st != NVFP4_SUCCESS)
        return st;
    if (rows == 0 || cols == 0)
        return NVFP4_SUCCESS;
    if (!packed || !scales || !out)
        return NVFP4_ERROR_INVALID_VALUE;
    if (!aligned(packed, 8) || !aligned(out, 16))
        return NVFP4_ERROR_MISALIGNED;
    Geometry g;
    if ((st = make_geometry(rows, cols, g)) != NVFP4_SUCCESS)
        return st;
    hipLaunchKernelGGL(nvfp4_dequantize_kernel, grid_for(g), dim3(kThreads), 0, stream,
                       packed, scales, g, gs, expert_offsets, (int)num_experts, out);
    return launched();
}

const char* nvfp4_status_string(nvfp4_status_t status)
{
    switch (status) {
    case NVFP4_SUCCESS: return "success";
    case NVFP4_ERROR_INVALID_VALUE: return "invalid value (size, pointer, pitch or expert arguments)";
    case NVFP4_ERROR_UNSUPPORTED_SHAPE: return "unsupported shape (columns must be a multiple of 16; sizes must fit int32 tiles)";
    case NVFP4_ERROR_MISALIGNED: return "misaligned pointer or row pitch";
    case NVFP4_ERROR_LAUNCH: return "kernel launch failed";
    }
    return "unknown status";
}

}  // extern "C"
