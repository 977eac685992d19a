// libmoe_nvfp4.so, second translation unit: the MoE L1 grouped GEMM on the
// gfx950 matrix cores (v_mfma_f32_32x32x16_bf16), with two epilogues:
//
//   * the fused one: SwiGLU of the FP32 accumulators and NVFP4 quantize,
//     writing only the packed E2M1 codes and FP8 scales (the L1 output never
//     exists in memory);
//   * a plain one: the interleaved L1 output as BF16, the producer side of
//     the unfused flow (then swiglu_nvfp4_quantize).
//
// Method: "NVFP4-1.1_APPROACH_PART_2.md", fused-epilogue design (the L1
// epilogue keeps SiLU(gate) in registers, forms SwiGLU with the up subtile,
// and every two 8-wide up subtiles make one 16-value FP4 block: amax, FP8
// scale, E2M1 pack; a 128-row x 64-output CTA tile holds 512 blocks, 4.5 KB
// of output) and "2026-05-28_STATUS.md" (BLOCKED row "Priority 3: NVFP4-1.1
// FP4 quant in MoE epilogue": fuse amax + FP4 pack into the L1 -> L2 path).
//
// Operands: x[tokens][ld_x] BF16, tokens grouped by expert (expert e owns
// rows [offsets[e], offsets[e+1])); w[e][n][ld_w] BF16 with row n the GEMM
// output column n (the weight stored [out][in], K contiguous). Output column
// n of the L1 GEMM follows the interleaved layout [gate x8, up x8, ...].
//
// Decomposition: one workgroup of 8 waves per CU computes 256 x 256 output
// tiles; wave (wm, wn) owns rows 64 wm .. +64 and columns 128 wn .. +128 as
// 2 x 4 MFMA tiles of 32 x 32. The K loop stages 256 x 64 slices of x and w
// in LDS (double-buffered, rows padded against bank conflicts) and
// prefetches the next slice into registers while the matrix cores work on
// the current one. 256 x 256 tiles halve the operand traffic per FLOP of
// 128 x 128 ones (measured: 128 x 128 tiles pulled 13 TB/s through L2 and
// held the matrix cores at 35%). Tiles are enumerated per expert
// (ceil(rows_e / 256) row tiles each, from a prefix sum the workgroup builds
// once in LDS) and handed to a persistent, XCD-aware grid. The epilogue runs
// in four 64-row passes through an LDS buffer that overlays the stages.
#include "../../include/moe_nvfp4.h"
#include "nvfp4_device.hpp"

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr int kWave = 64;
constexpr int kBM = 256, kBN = 256, kBK = 64;
constexpr int kThreads = 512;                             // 8 waves: 4 x 2 wave tiles of 64 x 128
constexpr int kMaxExperts = 512;
constexpr int kRowBytes = kBK * 2;                        // 128 data bytes per staged row
constexpr int kRowPitch = kRowBytes + 16;                 // one 16-byte pad per row
constexpr int kStageBytes = (kBM + kBN) * kRowPitch;      // 73,728 B: x slice then w slice
constexpr int kPassRows = 64;                             // epilogue rows per pass
constexpr int kCPitch = kBN + 4;                          // floats per LDS row of the C buffer
constexpr int kCBytes = kPassRows * kCPitch * 4;          // 66,560 B
constexpr int kLdsBytes = 2 * kStageBytes;
static_assert(kCBytes <= kLdsBytes, "the C buffer overlays the operand stages");
constexpr int kMi355xCUs = 256;
constexpr int kXcds = 8;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

// Byte offset of 16-byte chunk c (0..7) of staged row r. Rows are padded to
// 144 bytes, so the 16 rows whose chunks one LDS cycle serves (a wave reads
// 32 rows at one chunk position) start in 16 different 4-bank groups (no
// bank conflicts), and a lane's chunk for each K step is its row base plus
// an immediate offset.
__device__ __forceinline__ int chunk_at(int r, int c) { return r * kRowPitch + (c << 4); }

struct Gemm {
    const uint16_t* x;
    const uint16_t* w;
    int64_t ld_x, ld_w, w_expert;      // w_expert: elements between experts' weights
    int tokens, k, n;                  // n = GEMM output columns (2 * inter)
    const int32_t* offsets;            // nullptr: one expert owning every row
    int experts;
};

// Where a workgroup's current tile is.
struct TileRef {
    int e;          // expert
    int row0;       // first token row
    int rows;       // valid rows (1..256)
    int n0;         // first output column
};

// Tile prefix in LDS: off[e] (clamped to [0, tokens]) and pre[e] = row tiles
// of experts 0..e-1 (thread t counts expert t; Hillis-Steele scan). Returns
// the total number of row tiles.
__device__ int build_tile_prefix(const Gemm& g, int* off, int* pre, int* part)
{
    const int t = threadIdx.x;
    const int E = g.experts;
    for (int i = t; i <= E; i += kThreads) {
        const int o = g.offsets != nullptr ? g.offsets[i] : (i == 0 ? 0 : g.tokens);
        off[i] = min(max(o, 0), g.tokens);
    }
    __syncthreads();
    const int cnt = t < E ? (max(off[t + 1] - off[t], 0) + kBM - 1) / kBM : 0;
    part[t] = cnt;
    __syncthreads();
    for (int d = 1; d < kThreads; d <<= 1) {
        const int v = t >= d ? part[t - d] : 0;
        __syncthreads();
        part[t] += v;
        __syncthreads();
    }
    if (t < E)
        pre[t + 1] = part[t];
    if (t == 0)
        pre[0] = 0;
    __syncthreads();
    return pre[E];
}

__device__ __forceinline__ TileRef tile_ref(const Gemm& g, const int* off, const int* pre,
                                            int tile)
{
    const int nt = g.n / kBN;
    const int mt = tile / nt;
    int lo = 0, hi = g.experts;                 // largest e with pre[e] <= mt
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (pre[mid] <= mt)
            lo = mid;
        else
            hi = mid;
    }
    TileRef r;
    r.e = uniform(lo);
    r.row0 = uniform(off[lo] + (mt - pre[lo]) * kBM);
    r.rows = uniform(min(kBM, off[lo + 1] - r.row0));
    r.n0 = uniform((tile - mt * nt) * kBN);
    return r;
}

// 256 x 64 slices of x (rows row0.., clamped to the tile's valid rows) and
// w (rows n0..) at K offset k0: thread t loads 16-byte chunk t % 8 of rows
// t / 8 + 64 j, j = 0..3, of each.
struct Slice {
    u32x4 a[4], b[4];
};

__device__ __forceinline__ void load_slice(Slice& s, const Gemm& g, const TileRef& tr, int k0)
{
    const int c = threadIdx.x & 7;
    const int r0 = threadIdx.x >> 3;
    const uint16_t* wb = g.w + (int64_t)tr.e * g.w_expert + (int64_t)tr.n0 * g.ld_w + k0 + 8 * c;
    const uint16_t* xb = g.x + k0 + 8 * c;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int r = r0 + 64 * j;
        const int xr = tr.row0 + min(r, tr.rows - 1);
        s.a[j] = *reinterpret_cast<const u32x4*>(xb + (int64_t)xr * g.ld_x);
        s.b[j] = *reinterpret_cast<const u32x4*>(wb + (int64_t)r * g.ld_w);
    }
}

__device__ __forceinline__ void store_slice(uint8_t* stage, const Slice& s)
{
    const int c = threadIdx.x & 7;
    const int r0 = threadIdx.x >> 3;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int r = r0 + 64 * j;
        *reinterpret_cast<u32x4*>(stage + chunk_at(r, c)) = s.a[j];
        *reinterpret_cast<u32x4*>(stage + kBM * kRowPitch + chunk_at(r, c)) = s.b[j];
    }
}

// acc[tm][tn] += the wave's 64 x 128 part of the staged slice (4 K steps of
// 16): per step 2 A and 4 B fragments feed 8 MFMAs.
__device__ __forceinline__ void mma_slice(f32x16 (&acc)[2][4], const uint8_t* stage, int wm,
                                          int wn, int lane)
{
#pragma unroll
    for (int kk = 0; kk < kBK / 16; ++kk) {
        const int c = 2 * kk + (lane >> 5);
        bf16x8 a[2], b[4];
#pragma unroll
        for (int t = 0; t < 2; ++t)
            a[t] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(
                                                   stage + chunk_at(64 * wm + 32 * t + (lane & 31), c)));
#pragma unroll
        for (int t = 0; t < 4; ++t)
            b[t] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(
                                                   stage + kBM * kRowPitch +
                                                   chunk_at(128 * wn + 32 * t + (lane & 31), c)));
#pragma unroll
        for (int tm = 0; tm < 2; ++tm)
#pragma unroll
            for (int tn = 0; tn < 4; ++tn)
                acc[tm][tn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[tm], b[tn], acc[tm][tn], 0, 0, 0);
    }
}

// The K loop of one tile. Ends with a barrier after the last slice's reads.
__device__ __forceinline__ void gemm_tile(const Gemm& g, const TileRef& tr, uint8_t* smem,
                                          f32x16 (&acc)[2][4], int wm, int wn, int lane)
{
#pragma unroll
    for (int tm = 0; tm < 2; ++tm)
#pragma unroll
        for (int tn = 0; tn < 4; ++tn)
            acc[tm][tn] = f32x16{};
    const int kb_count = g.k / kBK;
    Slice s;
    load_slice(s, g, tr, 0);
    store_slice(smem, s);
    __syncthreads();
    for (int kb = 0; kb < kb_count; ++kb) {
        const bool more = kb + 1 < kb_count;
        if (more)
            load_slice(s, g, tr, (kb + 1) * kBK);
        mma_slice(acc, smem + (kb & 1) * kStageBytes, wm, wn, lane);
        if (more)
            store_slice(smem + ((kb + 1) & 1) * kStageBytes, s);
        __syncthreads();
    }
}

// The waves of row band p (wm == p) write their 64 x 128 accumulator parts
// into the C buffer: row 32 tm + 8 (i / 4) + 4 (lane / 32) + i % 4, column
// 128 wn + 32 tn + lane % 32 (the v_mfma_f32_32x32x16 result layout).
__device__ __forceinline__ void stage_accumulators(float* c, const f32x16 (&acc)[2][4], int wn,
                                                   int lane)
{
#pragma unroll
    for (int tm = 0; tm < 2; ++tm)
#pragma unroll
        for (int tn = 0; tn < 4; ++tn)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int row = 32 * tm + (i >> 2) * 8 + (lane >> 5) * 4 + (i & 3);
                const int col = 128 * wn + 32 * tn + (lane & 31);
                c[row * kCPitch + col] = acc[tm][tn][i];
            }
}

// ---- SwiGLU of FP32 values -------------------------------------------------
// silu(g) u = g u / (1 + e^-g), e^-g = 2^(-g log2 e). log2 e = kL2eHi + kL2eLo
// (kL2eHi = RN(log2 e)); the product -g kL2eHi is split into its rounded
// value p and exact error (fma), so 2^(-g log2 e) = 2^p 2^t with
// t = perr - g kL2eLo, |t| < 2e-5 for |g| < 100, and 2^t = 1 + t ln 2 to
// better than 1e-10. v_exp_f32 and v_rcp_f32 are about 1 ulp each: about
// 4 ulp in all. g < -88.7 overflows 2^p and gives y = +-0 (the exact |y|
// is below 1e-30 while |u| < 1e6).
__device__ __forceinline__ float swiglu_f32(float g, float u)
{
    const float kL2eHi = 0x1.715476p+0f;
    const float kL2eLo = 0x1.4ae0bep-26f;
    const float kLn2 = 0x1.62e430p-1f;
    const float p = -g * kL2eHi;
    const float perr = __builtin_fmaf(-g, kL2eHi, -p);
    const float t = __builtin_fmaf(-g, kL2eLo, perr);
    const float e0 = __builtin_amdgcn_exp2f(p);
    // e0 (1 + t ln 2), not e0 + e0 t ln 2: when 2^p overflows the factor is
    // positive and inf stays inf (inf - inf would be NaN)
    const float e = e0 * __builtin_fmaf(t, kLn2, 1.0f);
    return (g * u) * __builtin_amdgcn_rcpf(1.0f + e);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi)
{
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, bf16x2));
}

struct FusedOut {
    const float* gs;        // per expert, or nullptr (1.0)
    uint8_t* packed;        // [tokens][n/4]
    uint8_t* scales;        // [tokens][n/32]
    float* swiglu_out;      // [tokens][n/2] or nullptr
};

struct Bf16Out {
    uint16_t* out;          // [tokens][ld_out]
    int64_t ld_out;
};

// Fused epilogue of one 64-row pass: 64 rows x 8 NVFP4 blocks (each block =
// 32 interleaved accumulator columns [g x8, u x8, g x8, u x8] -> 16
// outputs); thread t takes block t % 8 of row t / 8.
__device__ __forceinline__ void epilogue(const Gemm& g, const TileRef& tr, int pass,
                                         const float* c, const FusedOut& o,
                                         const nvfp4::RowScale& rs)
{
    const int bl = threadIdx.x & 7;
    const int row = threadIdx.x >> 3;
    const int inter = g.n / 2;
    const float* src = c + row * kCPitch + 32 * bl;
    float v[32];
#pragma unroll
    for (int q = 0; q < 8; ++q) {
        const float4 f = *reinterpret_cast<const float4*>(src + 4 * q);
        v[4 * q] = f.x;
        v[4 * q + 1] = f.y;
        v[4 * q + 2] = f.z;
        v[4 * q + 3] = f.w;
    }
    float y[16];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        y[j] = swiglu_f32(v[j], v[8 + j]);
        y[8 + j] = swiglu_f32(v[16 + j], v[24 + j]);
    }
    uint32_t sf;
    const uint2 q = nvfp4::quantize16(y, rs, sf);
    const int trow = kPassRows * pass + row;
    if (trow < tr.rows) {
        const int64_t grow = tr.row0 + trow;
        const int64_t blk = grow * (inter / 16) + tr.n0 / 32 + bl;
        *reinterpret_cast<uint2*>(o.packed + blk * 8) = q;
        o.scales[blk] = (uint8_t)sf;
        if (o.swiglu_out != nullptr) {
            float* d = o.swiglu_out + grow * inter + tr.n0 / 2 + 16 * bl;
#pragma unroll
            for (int j = 0; j < 16; j += 4)
                *reinterpret_cast<float4*>(d + j) = make_float4(y[j], y[j + 1], y[j + 2], y[j + 3]);
        }
    }
}

// BF16 epilogue of one pass: thread t writes 16-byte chunks t + 512 j
// (j = 0..3) of the 64 x 256 pass, chunk q = row q / 32, columns 8 (q % 32).
__device__ __forceinline__ void epilogue(const Gemm&, const TileRef& tr, int pass, const float* c,
                                         const Bf16Out& o, const nvfp4::RowScale&)
{
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int q = threadIdx.x + kThreads * j;
        const int row = q >> 5;
        const int col = 8 * (q & 31);
        const float4 f0 = *reinterpret_cast<const float4*>(c + row * kCPitch + col);
        const float4 f1 = *reinterpret_cast<const float4*>(c + row * kCPitch + col + 4);
        const u32x4 w = {pack_bf16x2(f0.x, f0.y), pack_bf16x2(f0.z, f0.w), pack_bf16x2(f1.x, f1.y),
                         pack_bf16x2(f1.z, f1.w)};
        const int trow = kPassRows * pass + row;
        if (trow < tr.rows)
            *reinterpret_cast<u32x4*>(o.out + (int64_t)(tr.row0 + trow) * o.ld_out + tr.n0 + col) = w;
    }
}

__device__ __forceinline__ float expert_scale(const FusedOut& o, int e)
{
    return o.gs != nullptr ? o.gs[e] : 1.0f;
}
__device__ __forceinline__ float expert_scale(const Bf16Out&, int) { return 1.0f; }

// Persistent walk over the tiles. With a grid of a multiple of 8 workgroups
// (one per CU, dealt round-robin to the 8 XCDs), XCD x takes the x-th eighth
// of the tile list and its workgroups stride through it: concurrently
// running workgroups of one XCD work on neighbouring tiles (the same row
// tile, successive column tiles), which share their x rows in that XCD's L2.
template <class Out>
__global__ __launch_bounds__(kThreads) void moe_gemm_kernel(Gemm g, Out o)
{
    __shared__ __attribute__((aligned(16))) uint8_t smem[kLdsBytes];
    __shared__ int off[kMaxExperts + 1];
    __shared__ int pre[kMaxExperts + 1];
    __shared__ int part[kThreads];
    const int row_tiles = build_tile_prefix(g, off, pre, part);
    const int tiles = row_tiles * (g.n / kBN);
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = uniform(threadIdx.x / kWave);
    const int wm = wave >> 1, wn = wave & 1;
    float* c = reinterpret_cast<float*>(smem);
    int first = blockIdx.x, step = gridDim.x, end = tiles;
    if (gridDim.x % kXcds == 0) {
        const int per = (tiles + kXcds - 1) / kXcds;
        const int xcd = blockIdx.x % kXcds;
        first = xcd * per + blockIdx.x / kXcds;
        step = gridDim.x / kXcds;
        end = min(tiles, (xcd + 1) * per);
    }
    f32x16 acc[2][4];
    for (int tile = first; tile < end; tile += step) {
        const TileRef tr = tile_ref(g, off, pre, tile);
        gemm_tile(g, tr, smem, acc, wm, wn, lane);
        const nvfp4::RowScale rs = nvfp4::row_scale(expert_scale(o, tr.e));
        for (int pass = 0; pass < kBM / kPassRows; ++pass) {
            if (wm == pass)
                stage_accumulators(c, acc, wn, lane);
            __syncthreads();
            epilogue(g, tr, pass, c, o, rs);
            __syncthreads();   // the next pass (or tile) overwrites the buffer
        }
    }
}

// ---------------------------------------------------------------------------
// Host side: validation (no HIP call before it passes) and launch.
// ---------------------------------------------------------------------------
bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

nvfp4_status_t make_gemm(const uint16_t* x, const uint16_t* w, int64_t tokens, int64_t hidden,
                         int64_t n, int64_t ld_x, int64_t ld_w, const int32_t* offsets,
                         int32_t num_experts, Gemm& g, int& grid)
{
    if (tokens < 0 || hidden < 0 || n < 0 || ld_x < hidden || ld_w < hidden || num_experts < 0)
        return NVFP4_ERROR_INVALID_VALUE;
    if ((offsets != nullptr) != (num_experts > 0))
        return NVFP4_ERROR_INVALID_VALUE;
    if (hidden % kBK != 0 || n % kBN != 0 || num_experts > kMaxExperts)
        return NVFP4_ERROR_UNSUPPORTED_SHAPE;
    if (tokens > INT32_MAX || hidden > INT32_MAX || n > INT32_MAX)
        return NVFP4_ERROR_UNSUPPORTED_SHAPE;
    const int experts = offsets != nullptr ? num_experts : 1;
    // byte extents of x and of the weight stack must be addressable with
    // int64 offsets, or no such buffers can exist
    if ((tokens > 1 && ld_x > INT64_MAX / 2 / tokens) ||
        (n > 0 && ld_w > INT64_MAX / 2 / (experts * n)))
        return NVFP4_ERROR_INVALID_VALUE;
    // upper bound of the tiles the kernel will find: every expert may end in
    // a partial row tile
    const int64_t bound = ((tokens + kBM - 1) / kBM + experts) * (n / kBN);
    if (bound > INT32_MAX)
        return NVFP4_ERROR_UNSUPPORTED_SHAPE;
    if (tokens > 0 && hidden > 0 && n > 0) {
        if (!x || !w)
            return NVFP4_ERROR_INVALID_VALUE;
        if (!aligned(x, 16) || !aligned(w, 16) || ld_x % 8 != 0 || ld_w % 8 != 0)
            return NVFP4_ERROR_MISALIGNED;
    }
    g.x = x;
    g.w = w;
    g.ld_x = ld_x;
    g.ld_w = ld_w;
    g.w_expert = n * ld_w;
    g.tokens = (int)tokens;
    g.k = (int)hidden;
    g.n = (int)n;
    g.offsets = offsets;
    g.experts = experts;
    const int64_t cap = kMi355xCUs;
    grid = (int)(bound < cap ? bound : cap);
    return NVFP4_SUCCESS;
}

nvfp4_status_t launched()
{
    return hipGetLastError() == hipSuccess ? NVFP4_SUCCESS : NVFP4_ERROR_LAUNCH;
}

}  // namespace

extern "C" {

nvfp4_status_t moe_l1_gemm_swiglu_nvfp4(const uint16_t* x, const uint16_t* w1, int64_t tokens,
                                        int64_t hidden, int64_t inter, int64_t ld_x,
                                        int64_t ld_w, const int32_t* expert_offsets,
                                        int32_t num_experts, const float* gs, uint8_t* packed,
                                        uint8_t* scales, float* swiglu_out, hipStream_t stream)
{
    if (inter < 0 || inter > INT64_MAX / 2)
        return NVFP4_ERROR_INVALID_VALUE;
    Gemm g;
    int grid = 0;
    nvfp4_status_t st = make_gemm(x, w1, tokens, hidden, 2 * inter, ld_x, ld_w, expert_offsets,
                                  num_experts, g, grid);
    if (st != NVFP4_SUCCESS)
        return st;
    if (tokens == 0 || inter == 0)
        return NVFP4_SUCCESS;
    if (hidden == 0)      // every accumulator is 0: not a supported problem
        return NVFP4_ERROR_UNSUPPORTED_SHAPE;
    if (!packed || !scales)
        return NVFP4_ERROR_INVALID_VALUE;
    if (!aligned(packed, 8) || (swiglu_out && !aligned(swiglu_out, 16)))
        return NVFP4_ERROR_MISALIGNED;
    FusedOut o{gs, packed, scales, swiglu_out};
    hipLaunchKernelGGL(moe_gemm_kernel<FusedOut>, dim3(grid), dim3(kThreads), 0, stream, g, o);
    return launched();
}

nvfp4_status_t moe_l1_gemm_bf16(const uint16_t* x, const uint16_t* w1, int64_t tokens,
                                int64_t hidden, int64_t n, int64_t ld_x, int64_t ld_w,
                                const int32_t* expert_offsets, int32_t num_experts, uint16_t* out,
                                int64_t ld_out, hipStream_t stream)
{
    Gemm g;
    int grid = 0;
    nvfp4_status_t st = make_gemm(x, w1, tokens, hidden, n, ld_x, ld_w, expert_offsets,
                                  num_experts, g, grid);
    if (st != NVFP4_SUCCESS)
        return st;
    if (ld_out < n || (tokens > 1 && ld_out > INT64_MAX / 2 / tokens))
        return NVFP4_ERROR_INVALID_VALUE;
    if (tokens == 0 || n == 0)
        return NVFP4_SUCCESS;
    if (hidden == 0)
        return NVFP4_ERROR_UNSUPPORTED_SHAPE;
    if (!out)
        return NVFP4_ERROR_INVALID_VALUE;
    if (!aligned(out, 16) || ld_out % 8 != 0)
        return NVFP4_ERROR_MISALIGNED;
    Bf16Out o{out, ld_out};
    hipLaunchKernelGGL(moe_gemm_kernel<Bf16Out>, dim3(grid), dim3(kThreads), 0, stream, g, o);
    return launched();
}

}  // extern "C"
