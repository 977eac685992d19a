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
// Decomposition: one workgroup of 8 waves per CU (two per SIMD) computes
// 256 x 256 output tiles; group G of 4 waves owns rows 128 G .. +128 and
// wave s of it columns 64 s .. +64, as 4 x 2 MFMA tiles of 32 x 32 (128
// accumulator registers per lane). The K loop stages 256 x 64 slices of x
// and w in LDS (double-buffered, the lower half of x triple-buffered;
// 16-byte chunks XOR-swizzled against bank conflicts). The slices arrive by
// buffer loads straight into LDS (buffer_load_dwordx4 ... lds, 16 bytes per
// lane on gfx950), so no register holds them on the way. The loop is a ping-pong: the two waves of
// each SIMD take turns issuing a slice's 32 MFMAs and reading the next
// slice's fragments (and issuing loads), so one wave feeds the SIMD's
// matrix core while the other waits on LDS and memory.
//
// What bounds it: a 256 x 256 tile does 128 FLOP per byte of operand slices,
// so the matrix-core peak would need about 19 TB/s of operands from L2, and
// a CU's vector memory path (about 64 bytes per clock) is busy for about
// 1024 of the 2048 clocks a slice's MFMAs take. The walk order is chosen
// for cache reuse (tiles of the same row group and expert run together on
// every XCD), and the loads are spread over the waves that are not issuing
// MFMAs. 256 x 256 is the largest tile the registers of 8 waves hold with
// their fragments (4 SIMDs x 2 waves x 32 KB of accumulators). The MFMA
// streams take about 90% of the K loop's clocks (about 2200-2250 clocks per
// slice against the 2048 of its MFMAs); the clock itself is held down by
// the board's power limit while the matrix cores are this busy.
//
// Tiles are enumerated per expert (ceil(rows_e / 256) row tiles each, from a
// prefix sum the workgroup builds once in LDS) and handed to a persistent,
// XCD-aware grid. The epilogue runs in four 64-row passes through an LDS
// buffer that overlays stage 1, while stage 0 takes the next tile's first
// slice.
#include "../../include/moe_nvfp4.h"
#include "nvfp4_device.hpp"

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr int kWave = 64;
constexpr int kBM = 256, kBN = 256, kBK = 64;
constexpr int kThreads = 512;                             // 8 waves, two per SIMD
constexpr int kWaveM = 128, kWaveN = 64;                  // group G rows 128 G, wave s columns 64 s
constexpr int kTM = kWaveM / 32, kTN = kWaveN / 32;       // 4 x 2 MFMA tiles per wave
constexpr int kKSteps = kBK / 16;                         // MFMA K steps per slice
constexpr int kMaxExperts = 512;
constexpr int kRowBytes = kBK * 2;                        // 128 bytes per staged row
constexpr int kRegionBytes = kBM * kRowBytes;             // 32 KB: one operand's slice
constexpr int kStageBytes = 2 * kRegionBytes;             // x slice, then w slice
constexpr int kDmaRows = kWave * 16 / kRowBytes;          // staged rows one LDS-DMA load fills (8)
constexpr int kPassRows = 64;                             // epilogue rows per pass
constexpr int kCPitch = kBN + 4;                          // floats per LDS row of the C buffer
constexpr int kCBytes = kPassRows * kCPitch * 4;          // 66,560 B
// The C buffer overlays stage 1 and the 1 KB after it, so that stage 0 can
// take the next tile's first slice during the epilogue. The lower half of
// the x slice (rows 128-255, group 1's) cycles through three slots: the
// lower-half regions of the two stages and one more after the C buffer.
constexpr int kHalfBytes = kRegionBytes / 2;              // 16 KB: 128 staged x rows
constexpr int kSlot2 = kStageBytes + kCBytes;
constexpr int kLdsBytes = kSlot2 + kHalfBytes;
static_assert(kCBytes >= kStageBytes, "the C buffer covers stage 1");

// LDS offset of lower-x-half slot k (0, 1, 2).
__device__ __forceinline__ uint32_t xbot_slot(int k)
{
    return k == 2 ? (uint32_t)kSlot2 : (uint32_t)(k * kStageBytes + kHalfBytes);
}
constexpr int kMi355xCUs = 256;
constexpr int kXcds = 8;
constexpr int64_t kMaxPitch = int64_t(1) << 22;            // elements; 256 rows < 2^31 bytes

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

template <int v>
struct Int {
    static constexpr int value = v;
};

// Staged rows are 128 bytes (8 chunks of 16) with no padding: an LDS-DMA
// load writes 1 KB contiguously. Logical chunk c of row r sits in slot
// c ^ swz(r). One LDS cycle serves 16 lanes of a 16-byte read; a fragment
// read has those lanes on 16 consecutive rows at one logical chunk, and
// (r % 2, c ^ swz(r)) then takes 16 different values: 16 different 4-bank
// groups of the 64 banks, no conflicts.
__device__ __forceinline__ int swz(int r) { return (r >> 1) & 7; }

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

// Tile prefix in LDS: off[e] and pre[e] = row tiles of experts 0..e-1
// (thread t counts experts 2t and 2t + 1; Hillis-Steele scan over the
// threads). Returns the total number of row tiles. off[e] is the offset
// clamped to [0, tokens] and raised to the largest offset before it (a
// running maximum, also by Hillis-Steele). Valid offsets are non-decreasing,
// so neither step changes them. Offsets that break the rules then still give
// disjoint row ranges inside [0, tokens): every access stays inside x, w1 and
// the outputs, and the row tiles number at most ceil(tokens / 256) + E, the
// bound the host checks against INT32_MAX.
static_assert(2 * kThreads >= kMaxExperts + 1, "two offsets per thread in the tile prefix");
__device__ int build_tile_prefix(const Gemm& g, int* off, int* pre, int* part)
{
    const int t = threadIdx.x;
    const int E = g.experts;
    for (int i = t; i <= E; i += kThreads) {
        const int o = g.offsets != nullptr ? g.offsets[i] : (i == 0 ? 0 : g.tokens);
        off[i] = min(max(o, 0), g.tokens);
    }
    __syncthreads();
    for (int d = 1; d <= E; d <<= 1) {
        const int i0 = t, i1 = t + kThreads;
        const int a0 = i0 <= E && i0 >= d ? off[i0 - d] : 0;
        const int a1 = i1 <= E && i1 >= d ? off[i1 - d] : 0;
        __syncthreads();
        if (i0 <= E)
            off[i0] = max(off[i0], a0);
        if (i1 <= E)
            off[i1] = max(off[i1], a1);
        __syncthreads();
    }
    const int e0 = 2 * t, e1 = 2 * t + 1;
    const int c0 = e0 < E ? (max(off[e0 + 1] - off[e0], 0) + kBM - 1) / kBM : 0;
    const int c1 = e1 < E ? (max(off[e1 + 1] - off[e1], 0) + kBM - 1) / kBM : 0;
    part[t] = c0 + c1;
    __syncthreads();
    for (int d = 1; d < kThreads; d <<= 1) {
        const int v = t >= d ? part[t - d] : 0;
        __syncthreads();
        part[t] += v;
        __syncthreads();
    }
    if (e0 < E)
        pre[e0 + 1] = part[t] - c1;
    if (e1 < E)
        pre[e1 + 1] = part[t];
    if (t == 0)
        pre[0] = 0;
    __syncthreads();
    return pre[E];
}

// Walk order: tiles are taken column-major within groups of kGroupRows row
// tiles (row tile = group base + i % rows, column tile = i / rows for the
// group's i-th tile). The 32 consecutive tiles one XCD runs together then
// cover 8 row tiles x 4 column tiles and share their x and w slices in that
// XCD's L2, where a row-major walk has each workgroup stream its own w
// slice. A bijection of [0, row_tiles * nt). Measured on the 8-expert
// problem: groups of 8 rows beat 4 and 16 by 3%, and 2 by 7%.
constexpr int kGroupRows = 8;

__device__ __forceinline__ void tile_coords(int tile, int row_tiles, int nt, int& mt, int& ct)
{
    const int group = tile / (kGroupRows * nt);
    const int first = group * kGroupRows;
    const int rows = min(kGroupRows, row_tiles - first);
    const int i = tile - group * kGroupRows * nt;
    mt = first + i % rows;
    ct = i / rows;
}

__device__ __forceinline__ TileRef tile_ref(const Gemm& g, const int* off, const int* pre,
                                            int row_tiles, int tile)
{
    const int nt = g.n / kBN;
    int mt, ct;
    tile_coords(tile, row_tiles, nt, mt, ct);
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
    r.n0 = uniform(ct * kBN);
    return r;
}

// A tile's operand windows as buffer resources (base and size in SGPRs):
// x rows row0 .. row0 + rows and w rows n0 .. n0 + 256 of expert e. A row
// of x past a partial tile lies outside its window, and the hardware range
// check returns zeros for it (those rows are computed, never stored). The
// range check covers the VGPR offset (plus the instruction's immediate),
// not the SGPR offset, so a lane keeps the whole row offset of each of its
// 8 x rows in VGPRs, and the SGPR offset only carries the K position within
// the row. Every w row lies inside its window: one VGPR offset (chunk t % 8
// of row t / 8), with the row step in the SGPR offset. Windows are at most
// 256 rows of pitch < 2^22 elements: under 2^31 bytes.
//
// The loads of a slice are split by group (see gemm_tile): wave s of group 0
// loads w rows 64 s .. +64 (8 loads), wave s of group 1 loads x rows
// 32 s .. +32 of the upper half and 128 + 32 s .. +32 of the lower half
// (4 loads each).
struct TileSrc {
    u32x4 x, w;              // buffer descriptors (SGPRs)
    int vx[8];               // group 1: x row offsets of this lane, upper-half loads 0-3, lower 4-7
    int vw[2];               // group 0: w offsets (row within the 8-row group) for even / odd loads
    int row_w;               // bytes of one w row
};

// A raw buffer descriptor over [base, base + bytes): base address, stride 0,
// the size for the range check, and the same format word as
// __builtin_amdgcn_make_buffer_rsrc takes. Wave-uniform, kept in SGPRs.
__device__ __forceinline__ u32x4 window(const uint16_t* base, int bytes)
{
    const uint64_t a = (uint64_t)(uintptr_t)base;
    return u32x4{(uint32_t)uniform((int)(uint32_t)a), (uint32_t)uniform((int)(uint32_t)(a >> 32)),
                 (uint32_t)uniform(bytes), 0x00020000u};
}

// A load instruction fills 8 staged rows r0 .. r0 + 8 (r0 a multiple of 8;
// 1 KB of LDS, lane l at byte 16 l): lane l loads row r0 + l / 8, logical
// chunk (l % 8) ^ swz(row) = (l % 8) ^ (4 ((r0 / 8) % 2) + l / 16). The x
// loads of wave s (group 1) start at rows 32 s + 8 i and 128 + 32 s + 8 i
// (i = 0..3), the w loads of wave s (group 0) at 64 s + 8 j (j = 0..7):
// r0 / 8 has the parity of i, resp. j.
__device__ __forceinline__ TileSrc tile_src(const Gemm& g, const TileRef& tr, int s)
{
    TileSrc t;
    t.x = window(g.x + (int64_t)tr.row0 * g.ld_x, tr.rows * (int)g.ld_x * 2);
    t.w = window(g.w + (int64_t)tr.e * g.w_expert + (int64_t)tr.n0 * g.ld_w, kBN * (int)g.ld_w * 2);
    const int l = threadIdx.x & (kWave - 1);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int c = (l & 7) ^ (4 * (i & 1) + (l >> 4));
        const int r0 = 128 * (i >> 2) + 32 * s + 8 * (i & 3);
        t.vx[i] = (r0 + (l >> 3)) * (int)g.ld_x * 2 + 16 * c;
        if (i < 2)
            t.vw[i] = (l >> 3) * (int)g.ld_w * 2 + 16 * c;
    }
    t.row_w = (int)g.ld_w * 2;
    return t;
}

// The 32-bit LDS address of a pointer into LDS. The cast from a generic
// pointer costs 64-bit arithmetic and a null check, so callers take it once
// per slice and add 32-bit row offsets: per load it also kept eight 64-bit
// row offsets live in SGPR pairs (2.8% slower, 36 instead of 9 SGPRs
// spilled to VGPR lanes).
__device__ __forceinline__ uint32_t lds_addr(const uint8_t* p)
{
    return (uint32_t)uniform((int)(uint32_t)(uintptr_t)(const __attribute__((address_space(3))) uint8_t*)p);
}

// 16 bytes per lane from the buffer straight into LDS at lds + 16 lane. By
// inline assembly: the compiler would otherwise wait for every such load
// before any later LDS read, since it cannot tell that they fill the other
// stage. The caller waits (vmcnt(0)) before the stage is read.
__device__ __forceinline__ void load_lds16(const u32x4& rsrc, uint32_t lds, int voff, int soff)
{
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
                 :: "s"(lds), "v"(voff), "s"(rsrc), "s"(soff) : "memory");
}

// Load jj (0..7) of group 0 wave s's share of the w slice at K offset k0
// into the stage at LDS address `base`: staged w rows 64 s + 8 jj .. +8.
static_assert(kDmaRows == 8, "the swizzle and offsets assume 8-row loads");
__device__ __forceinline__ void load_w_one(const TileSrc& src, uint32_t base, int k0, int s, int jj)
{
    const int row = 64 * s + 8 * jj;
    load_lds16(src.w, base + kRegionBytes + row * kRowBytes, src.vw[jj & 1],
               uniform(row * src.row_w + 2 * k0));
}

// Load i (0..3) of group 1 wave s's share of one half of the x slice at K
// offset k0: x rows 128 half + 32 s + 8 i .. +8 of the tile, staged at rows
// 32 s + 8 i .. +8 from LDS address `base` (the start of the half's 128
// rows: the stage for the upper half, a slot for the lower; the swizzle
// depends on the row modulo 16 only).
__device__ __forceinline__ void load_x_one(const TileSrc& src, uint32_t base, int k0, int s,
                                           int half, int i)
{
    const int row = 32 * s + 8 * i;
    load_lds16(src.x, base + row * kRowBytes, src.vx[4 * half + i], uniform(2 * k0));
}

__device__ __forceinline__ void load_w(const TileSrc& src, uint32_t base, int k0, int s)
{
#pragma unroll
    for (int jj = 0; jj < 8; ++jj)
        load_w_one(src, base, k0, s, jj);
}

__device__ __forceinline__ void load_x(const TileSrc& src, uint32_t base, int k0, int s, int half)
{
#pragma unroll
    for (int i = 0; i < 4; ++i)
        load_x_one(src, base, k0, s, half, i);
}

// The wave's MFMA operands for a whole staged slice: for each 16-deep K
// step kk, 4 A fragments (rows 128 G + 32 t + lane % 32) and 2 B fragments
// (columns 64 s + 32 t + lane % 32), each 8 K values starting at
// 8 (2 kk + lane / 32). 24 reads of 16 bytes per lane, 96 registers.
struct SliceFrags {
    bf16x8 a[kKSteps][kTM], b[kKSteps][kTN];
};

// A lane's byte offset of K step kk within a staged row group: rows
// 32 t + lane % 32 (+ a multiple of 32), so swz depends on the lane only,
// and chunk 2 kk + lane / 32 sits in slot (2 kk) ^ (lane / 32 ^ swz).
struct FragOffset {
    int row, c0;
    __device__ __forceinline__ explicit FragOffset(int lane)
        : row((lane & 31) * kRowBytes), c0((lane >> 5) ^ swz(lane & 31)) {}
    __device__ __forceinline__ int at(int kk) const { return row + (((2 * kk) ^ c0) << 4); }
};

// A fragments of K step kk from the wave's 128 staged x rows at `xrows`.
__device__ __forceinline__ void read_a(SliceFrags& f, const uint8_t* xrows, int kk,
                                       const FragOffset& fo)
{
#pragma unroll
    for (int t = 0; t < kTM; ++t)
        f.a[kk][t] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(
                                                    xrows + 32 * t * kRowBytes + fo.at(kk)));
}

__device__ __forceinline__ void read_b(SliceFrags& f, const uint8_t* stage, int s, int kk,
                                       const FragOffset& fo)
{
#pragma unroll
    for (int t = 0; t < kTN; ++t)
        f.b[kk][t] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(
                                                    stage + kRegionBytes + (kWaveN * s + 32 * t) * kRowBytes + fo.at(kk)));
}

constexpr int kSliceMfmas = kKSteps * kTM * kTN;             // 32

// MFMA n of a slice: K step n / 8, row tile (n % 8) / kTN, column tile n % kTN.
__device__ __forceinline__ void mma_one(f32x16 (&acc)[kTM][kTN], const SliceFrags& f, int n)
{
    const int kk = n / (kTM * kTN), i = n % (kTM * kTN);
    acc[i / kTN][i % kTN] =
        __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.a[kk][i / kTN], f.b[kk][i % kTN], acc[i / kTN][i % kTN], 0, 0, 0);
}

// The slice's 32 MFMAs back to back (about 1024 cycles of the SIMD's matrix
// core).
__device__ __forceinline__ void mma_slice(f32x16 (&acc)[kTM][kTN], const SliceFrags& f)
{
#pragma unroll
    for (int n = 0; n < kSliceMfmas; ++n)
        mma_one(acc, f, n);
    __builtin_amdgcn_sched_barrier(0);
}

// A workgroup barrier that orders nothing by itself: the waits a phase needs
// are written out before it. (__syncthreads() would also wait for every
// outstanding load, the loader waves' LDS-DMA loads of the next slice
// included.) The memory clobber keeps LDS accesses on their side of it.
__device__ __forceinline__ void phase_barrier()
{
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_barrier" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
}

__device__ __forceinline__ void wait_lds_reads() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }
__device__ __forceinline__ void wait_loads() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// The K loop of one tile, as a ping-pong between the two waves of each SIMD.
// Group 0 (waves 0-3) and group 1 (waves 4-7) hold the tile's upper and
// lower 128 rows; wave w and wave w + 4 run on the same SIMD. Both groups
// run the same loop, read a slice's fragments | barrier | issue its 32
// MFMAs | barrier, group 1 one phase behind group 0:
//
//   phase 2j         group 0 reads slice j      group 1 computes slice j - 1
//   phase 2j + 1     group 0 computes slice j   group 1 reads slice j
//
// (group 1 idles through phase 0, group 0 through the last phase), so each
// SIMD's matrix core runs one wave's MFMAs while the other wave's LDS reads
// are in flight, and a barrier costs a few cycles instead of the drift
// between four waves that all compute. Slice j sits in stage j % 2, its
// lower x half in slot j % 3 of a ring of three.
//
// The LDS-DMA loads are issued in the read phases, two after each K step's
// fragment reads: a load can stall the issuing wave for tens of cycles
// while the CU's vector memory path (about 64 bytes per clock, so about
// 1024 clocks per 64 KB slice) works through the loads before it, which a
// read phase has time for and an MFMA stream has not, and the LDS reads
// proceed meanwhile. They are spread over both groups' read phases, 32
// loads each, by what each group reads: group 0 reads x rows 0-127 and all
// of w, group 1 rows 128-255 and all of w.
//   * phase 2j: group 0 loads w of slice j + 1 into stage (j + 1) % 2 (both
//     groups read the w there, of slice j - 1, in phases 2j - 2 and 2j - 1).
//     Wave s of group 0 loads exactly the w rows its own B fragments read
//     (64 s .. +64), so it waits for them only in phase 2j + 2, after its x
//     fragment reads and before its w ones; group 1's wave s reads them in
//     phase 2j + 3, past the barrier. No MFMA phase of group 0 waits.
//   * phase 2j + 1: group 1 loads both x halves of slice j + 2: the upper
//     half into stage j % 2 (group 0 read the one there in phase 2j), the
//     lower half into slot (j + 2) % 3 of a three-slot ring (it read the
//     one there itself in phase 2j - 1). It waits for slice j + 1's halves
//     at the end of the same read phase, before the barrier, so no MFMA
//     phase waits for loads. (With the lower half double-buffered like the
//     rest, its window was one phase shorter and group 1 waited for it at
//     the end of its MFMA phases, about 85 clocks each.)
// Each wave waits for its own reads before the barrier that closes its read
// phase, so a stage part is free when the next barrier has passed; waits for
// loads use the exact in-order count of loads issued after them (or wait for
// all at the end of the K loop). Every wave runs 2 + 2 K / 64 barriers
// (s_barrier counts arrivals, not places in the code). Ends after the last
// slice's MFMAs have issued, with every LDS read and load complete.
__device__ __forceinline__ void load_slice0(const TileSrc& src, uint32_t stages, int grp, int s)
{
    if (grp == 0) {
        load_w(src, stages, 0, s);
    } else {
        load_x(src, stages, 0, s, 0);
        load_x(src, stages + xbot_slot(0), 0, s, 1);
    }
}

__device__ __forceinline__ void gemm_tile(const Gemm& g, const TileRef& tr, uint8_t* smem,
                                          f32x16 (&acc)[kTM][kTN], int grp, int s, int lane)
{
#pragma unroll
    for (int tm = 0; tm < kTM; ++tm)
#pragma unroll
        for (int tn = 0; tn < kTN; ++tn)
            acc[tm][tn] = f32x16{};
    const int slices = g.k / kBK;
    const bool g0 = grp == 0;
    const TileSrc src = tile_src(g, tr, s);
    const uint32_t stages = lds_addr(smem);
    // slice 0 was issued by load_slice0 (group 0 its w, group 1 its two x
    // halves, while the previous tile's epilogue ran); group 1 adds both x
    // halves of slice 1 and waits for slice 0's (8 loads after them)
    if (g0) {
        wait_loads();
    } else if (slices > 1) {
        load_x(src, stages + kStageBytes, kBK, s, 0);
        load_x(src, stages + xbot_slot(1), kBK, s, 1);
        asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
    } else {
        wait_loads();
    }
    phase_barrier();                                       // slice 0 is staged
    if (!g0)
        phase_barrier();                                   // group 1 idles through phase 0
    const FragOffset fo(lane);
    int slot = 0;                                          // j % 3: lower x half of slice j
    for (int j = 0; j < slices; ++j) {
        const uint32_t cur = uniform((j & 1) * kStageBytes), nxt = uniform(((j + 1) & 1) * kStageBytes);
        const bool next = j + 1 < slices, more = j + 2 < slices;
        const uint8_t* stage = smem + cur;
        const int slot2 = slot == 0 ? 2 : slot - 1;        // (j + 2) % 3
        SliceFrags f;
        if (g0) {
            // x fragments, two w loads of slice j + 1 after each K step's;
            // then this wave's own w rows of slice j (8 loads were issued
            // after them), and the w fragments
#pragma unroll
            for (int kk = 0; kk < kKSteps; ++kk) {
                read_a(f, stage, kk, fo);
                if (next) {
                    load_w_one(src, stages + nxt, (j + 1) * kBK, s, 2 * kk);
                    load_w_one(src, stages + nxt, (j + 1) * kBK, s, 2 * kk + 1);
                }
            }
            if (next)
                asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
            else
                wait_loads();
#pragma unroll
            for (int kk = 0; kk < kKSteps; ++kk)
                read_b(f, stage, s, kk, fo);
        } else {
            // each K step's fragments, then two loads of slice j + 2: its
            // lower x half into slot (j + 2) % 3 after steps 0 and 1, its
            // upper half into stage j % 2 after steps 2 and 3
            const uint8_t* xrows = smem + xbot_slot(slot);
#pragma unroll
            for (int kk = 0; kk < kKSteps; ++kk) {
                read_a(f, xrows, kk, fo);
                read_b(f, stage, s, kk, fo);
                if (more) {
                    if (kk < 2) {
                        load_x_one(src, stages + xbot_slot(slot2), (j + 2) * kBK, s, 1, 2 * kk);
                        load_x_one(src, stages + xbot_slot(slot2), (j + 2) * kBK, s, 1, 2 * kk + 1);
                    } else {
                        load_x_one(src, stages + cur, (j + 2) * kBK, s, 0, 2 * kk - 4);
                        load_x_one(src, stages + cur, (j + 2) * kBK, s, 0, 2 * kk - 3);
                    }
                }
            }
        }
        wait_lds_reads();
        if (!g0) {
            // both x halves of slice j + 1 (8 loads were issued after them)
            if (more)
                asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
            else
                wait_loads();
        }
        phase_barrier();
        mma_slice(acc, f);
        phase_barrier();
        slot = slot == 2 ? 0 : slot + 1;
    }
    if (g0)
        phase_barrier();                                   // group 0 idles through the last phase
}

// Epilogue pass p holds the tile rows of MFMA row tile p of every wave:
// C buffer row r is tile row 128 (r / 32) + 32 p + r % 32. All 8 waves
// write their tile p (no branch, and 32 accumulators per lane per pass):
// row 32 G + 8 (i / 4) + 4 (lane / 32) + i % 4, column 64 s + 32 tn +
// lane % 32 (the v_mfma_f32_32x32x16 result layout) for wave s of group G.
__device__ __forceinline__ int pass_row(int pass, int r)
{
    return kWaveM * (r >> 5) + 32 * pass + (r & 31);
}

template <int kPass>
__device__ __forceinline__ void stage_accumulators(float* c, const f32x16 (&acc)[kTM][kTN], int grp,
                                                   int s, int lane)
{
#pragma unroll
    for (int tn = 0; tn < kTN; ++tn)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int row = 32 * grp + (i >> 2) * 8 + (lane >> 5) * 4 + (i & 3);
            const int col = kWaveN * s + 32 * tn + (lane & 31);
            c[row * kCPitch + col] = acc[kPass][tn][i];
        }
}

// ---- SwiGLU of FP32 values -------------------------------------------------
// silu(g) u = g u sigma(g), sigma(g) = 1 / (1 + e^-|g|) for g >= 0 and
// e^-|g| / (1 + e^-|g|) for g < 0, with a = |g| clamped to 300 (beyond it
// sigma is 1 to binary32 precision, or so small that g u sigma(g) rounds to
// zero for any FP32 g and u: |g u| < 2^256 and e^-300 < 2^-432).
// e^-a = 2^(-a log2 e): log2 e = kL2eHi + kL2eLo (kL2eHi = RN(log2 e)); the
// product -a kL2eHi is split into its rounded value p and exact error (fma),
// so e^-a = 2^p 2^t with t = perr - a kL2eLo, |t| < 2e-4, and 2^t = 1 + t ln 2
// to better than 2e-8 relative. 2^p is formed as 2^(p + k) 2^-k with k the
// multiple of 64 that puts p + k in (-64, 0] (p + k is exact), so that
// v_exp_f32 and the sigmoid stay in the normal range down to g = -300;
// v_exp_f32 and v_rcp_f32 are about 1 ulp each: about 4 ulp in all. The
// product g u (sigma 2^k) 2^-k is formed in binary64 (g u exact, one rounding,
// an exact power-of-two scaling) and rounded once to binary32, so neither
// g u nor a tiny sigma leaves the range on the way: y has sigma's relative
// error down into the binary32 subnormals, and a zero keeps the sign of g u.
__device__ __forceinline__ float swiglu_f32(float g, float u)
{
    const float kL2eHi = 0x1.715476p+0f;
    const float kL2eLo = 0x1.4ae0bep-26f;
    const float kLn2 = 0x1.62e430p-1f;
    const float a = __builtin_fminf(__builtin_fabsf(g), 300.0f);
    const float p = -a * kL2eHi;
    const float perr = __builtin_fmaf(-a, kL2eHi, -p);
    const float t = __builtin_fmaf(-a, kL2eLo, perr);
    const int k = (int)(-p * 0.015625f) * 64;
    const float es = __builtin_amdgcn_exp2f(p + (float)k) * __builtin_fmaf(t, kLn2, 1.0f);
    const float r = __builtin_amdgcn_rcpf(1.0f + __builtin_ldexpf(es, -k));
    const bool neg = g < 0.0f;
    const float ss = neg ? es * r : r;          // sigma(g) 2^kk
    const int kk = neg ? k : 0;
    return (float)__builtin_ldexp((double)g * (double)u * (double)ss, -kk);
}

// swiglu_f32 for |g| < 44: there -p / 64 < 1, so k = 0, every shift is by
// zero and p + 0 = p (a zero p included: exp2(+0) = exp2(-0)); this is the
// same arithmetic with those steps left out, so the results are identical.
__device__ __forceinline__ float swiglu_f32_small(float g, float u)
{
    const float kL2eHi = 0x1.715476p+0f;
    const float kL2eLo = 0x1.4ae0bep-26f;
    const float kLn2 = 0x1.62e430p-1f;
    const float a = __builtin_fabsf(g);
    const float p = -a * kL2eHi;
    const float perr = __builtin_fmaf(-a, kL2eHi, -p);
    const float t = __builtin_fmaf(-a, kL2eLo, perr);
    const float es = __builtin_amdgcn_exp2f(p) * __builtin_fmaf(t, kLn2, 1.0f);
    const float r = __builtin_amdgcn_rcpf(1.0f + es);
    const float ss = g < 0.0f ? es * r : r;
    return (float)((double)g * (double)u * (double)ss);
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
// outputs); thread t takes block t % 8 of rows t / 8 and t / 8 + 32.
__device__ __forceinline__ void fused_block(const Gemm& g, const TileRef& tr, int pass,
                                            const float* c, const FusedOut& o,
                                            const nvfp4::RowScale& rs, int row, int bl)
{
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
    // the largest gate magnitude (a NaN gate is dropped by the max, and gives
    // NaN on either path)
    float gmax = 0.0f;
#pragma unroll
    for (int j = 0; j < 8; ++j)
        gmax = __builtin_fmaxf(gmax, __builtin_fmaxf(__builtin_fabsf(v[j]), __builtin_fabsf(v[16 + j])));
    if (gmax < 44.0f) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            y[j] = swiglu_f32_small(v[j], v[8 + j]);
            y[8 + j] = swiglu_f32_small(v[16 + j], v[24 + j]);
        }
    } else {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            y[j] = swiglu_f32(v[j], v[8 + j]);
            y[8 + j] = swiglu_f32(v[16 + j], v[24 + j]);
        }
    }
    uint32_t sf;
    const uint2 q = nvfp4::quantize16<true, false>(y, nvfp4::block_amax(y), rs, sf);
    const int trow = pass_row(pass, row);
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

__device__ __forceinline__ void epilogue(const Gemm& g, const TileRef& tr, int pass,
                                         const float* c, const FusedOut& o,
                                         const nvfp4::RowScale& rs, int tid)
{
#pragma unroll
    for (int j = 0; j < kPassRows * 8 / kThreads; ++j)
        fused_block(g, tr, pass, c, o, rs, (tid >> 3) + (kThreads / 8) * j, tid & 7);
}

// BF16 epilogue of one pass: thread t writes 16-byte chunks t + 256 j
// (j = 0..7) of the 64 x 256 pass, chunk q = row q / 32, columns 8 (q % 32).
__device__ __forceinline__ void epilogue(const Gemm&, const TileRef& tr, int pass, const float* c,
                                         const Bf16Out& o, const nvfp4::RowScale&, int tid)
{
#pragma unroll
    for (int j = 0; j < kPassRows * kBN / 8 / kThreads; ++j) {
        const int q = tid + kThreads * j;
        const int row = q >> 5;
        const int col = 8 * (q & 31);
        const float4 f0 = *reinterpret_cast<const float4*>(c + row * kCPitch + col);
        const float4 f1 = *reinterpret_cast<const float4*>(c + row * kCPitch + col + 4);
        const u32x4 w = {pack_bf16x2(f0.x, f0.y), pack_bf16x2(f0.z, f0.w), pack_bf16x2(f1.x, f1.y),
                         pack_bf16x2(f1.z, f1.w)};
        const int trow = pass_row(pass, row);
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
// (one per CU, dealt round-robin to the 8 XCDs), each round of gridDim.x
// consecutive tiles of the walk order is split into 8 runs, run x going to
// XCD x's workgroups: the workgroups of one XCD work on neighbouring tiles
// (sharing x and w slices in that XCD's L2), and the 8 XCDs work on the same
// row groups of the same expert at the same time (sharing them in the
// Infinity Cache). Giving each XCD a contiguous eighth of the whole walk
// instead put the XCDs on different experts, whose weights do not fit the
// cache together: 9% slower.
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
    const int grp = wave >> 2, s = wave & 3;               // waves w and w + 4 share a SIMD
    float* c = reinterpret_cast<float*>(smem + kStageBytes);
    const uint32_t stages = lds_addr(smem);
    int first = blockIdx.x;
    if (gridDim.x % kXcds == 0)
        first = (blockIdx.x % kXcds) * (gridDim.x / kXcds) + blockIdx.x / kXcds;
    f32x16 acc[kTM][kTN];
    TileRef next_tr{};
    if (first < tiles) {
        next_tr = tile_ref(g, off, pre, row_tiles, first);
        load_slice0(tile_src(g, next_tr, s), stages, grp, s);
    }
    for (int tile = first; tile < tiles; tile += gridDim.x) {
        const TileRef tr = next_tr;
        gemm_tile(g, tr, smem, acc, grp, s, lane);
        // the expert's scale, consumed here: a wait for it placed after the
        // loads below would wait for them too
        float gs = expert_scale(o, tr.e);
        asm volatile("" : "+v"(gs));
        const nvfp4::RowScale rs = nvfp4::row_scale(gs);
        // the next tile's slice 0 into stage 0, free now that every wave has
        // passed the K loop's last barrier; it lands during this epilogue
        if (tile + (int)gridDim.x < tiles) {
            next_tr = tile_ref(g, off, pre, row_tiles, tile + gridDim.x);
            load_slice0(tile_src(g, next_tr, s), stages, grp, s);
        }
        // the thread index taken afresh per tile: the epilogue's addresses
        // are then computed here, not hoisted out of the tile loop, where
        // they would stay live through the K loop and crowd its registers
        int tid = threadIdx.x;
        asm volatile("" : "+v"(tid));
        const int el = tid & (kWave - 1);
        static_assert(kBM / kPassRows == kTM && kPassRows == 2 * 32, "one MFMA row tile per pass");
        auto pass = [&](auto p) {
            stage_accumulators<decltype(p)::value>(c, acc, grp, s, el);
            __syncthreads();
            epilogue(g, tr, decltype(p)::value, c, o, rs, tid);
            __syncthreads();   // the next pass (or tile) overwrites the buffer
        };
        pass(Int<0>{});
        pass(Int<1>{});
        pass(Int<2>{});
        pass(Int<3>{});
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
    // a tile's operand window (256 rows) is addressed with 32-bit offsets
    if (ld_x >= kMaxPitch || ld_w >= kMaxPitch)
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
