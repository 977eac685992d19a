// libmoe_nvfp4.so: HIP kernels for gfx950 and the C ABI declared in
// include/moe_nvfp4.h.
//
// Kernels: the fused SwiGLU + NVFP4 quantize and the standalone quantize
// (quantize_tiles_kernel), the dequantize, the global-scale pre-pass
// (amax_tiles_kernel and two small helpers), the compact BF16 SwiGLU pass,
// and the paged KV-cache write (quantize_paged_kernel) and read (the
// dequantize with a slot indirection). The grouped GEMM with the fused
// epilogue is in moe_gemm.hip.
//
// Work decomposition: one lane owns one NVFP4 block of 16 output values; one
// wave64 owns a "tile" of 64 consecutive blocks of one row, so the row index
// and its base addresses are wave-uniform (scalar registers). Tiles are
// numbered row-major and handed to waves with a grid-stride loop: the
// quantize, paged-write, pre-pass and compact kernels walk them with a
// persistent grid sized per kernel (workgroup waves and workgroups per CU
// measured on MI355X), the dequantize with one tile per wave.
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
constexpr int kWavesPerBlock = 4;                  // dequantize workgroups
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
typedef float f32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

// Streaming (read-once / write-once) accesses: non-temporal hint.
__device__ __forceinline__ u32x4 ld_stream(const u32x4* p) { return __builtin_nontemporal_load(p); }
__device__ __forceinline__ u32x2 ld_stream(const u32x2* p) { return __builtin_nontemporal_load(p); }
__device__ __forceinline__ void st_stream(f32x4 v, f32x4* p) { __builtin_nontemporal_store(v, p); }

// Orders this wave's LDS accesses (stores before the loads that follow and
// vice versa). LDS operations of one wave execute in order, so a compiler
// barrier plus a wavefront-scope fence is enough; no s_barrier is needed
// because each wave owns its staging area.
__device__ __forceinline__ void wave_lds_sync()
{
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    __builtin_amdgcn_wave_barrier();
}

// LDS slot of 16-byte word w of a staged tile: one pad slot after every 16
// words. Global memory is read (or written) one word per lane with
// consecutive lanes on consecutive words; each lane works on the P (2 or 4)
// consecutive words of its own block. With the padding both patterns hit 8
// (or 16) distinct 16-byte bank groups per LDS cycle, and a lane's own block
// is contiguous, so its P accesses share one address plus immediate offsets.
constexpr int kStageSlots(int P) { return kTileBlocks * P + kTileBlocks * P / 16; }

__device__ __forceinline__ int lds_slot(int w) { return w + (w >> 4); }

struct Tile {
    int row;
    int blk0;   // first block of the tile within the row
    int nblk;   // blocks in this tile (64, fewer in a row's last tile)
};

__device__ __forceinline__ Tile tile_at(int tile, const Geometry& geo)
{
    Tile t;
    t.row = uniform(tile / geo.cpr);
    t.blk0 = uniform((tile - t.row * geo.cpr) * kTileBlocks);
    t.nblk = uniform(min(kTileBlocks, geo.bpr - t.blk0));
    return t;
}

// ---------------------------------------------------------------------------
// Quantize kernels (fused SwiGLU + NVFP4, and plain BF16 -> NVFP4).
// A block's input is P words: 4 for the fused input [g0..7][u0..7][g8..15]
// [u8..15] (64 bytes), 2 for plain BF16 (32 bytes). Each wave walks its tiles
// with a stride of the whole grid and keeps one tile in flight: it issues the
// coalesced loads of the next tile, computes the staged tile from LDS (each
// lane its own block), stores it, and then stages the next tile.
// ---------------------------------------------------------------------------
// Coalesced loads of a tile: instruction j reads word j*64 + lane. In a
// row's last, partial tile the lanes past the end re-read the last word
// (clamped, no branch), so every load and LDS store is unconditional and the
// compiler can wait for exactly the loads it needs.
template <int P>
__device__ __forceinline__ void load_tile(u32x4 (&v)[P], const uint16_t* in, int64_t ld,
                                          const Tile& t, int lane)
{
    const u32x4* src = reinterpret_cast<const u32x4*>(in + (int64_t)t.row * ld) + t.blk0 * P;
    const int last = t.nblk * P - 1;
#pragma unroll
    for (int j = 0; j < P; ++j)
        v[j] = ld_stream(src + min(j * kWave + lane, last));
}

template <int P>
__device__ __forceinline__ void stage_tile(u32x4* lds, const u32x4 (&v)[P], int lane)
{
#pragma unroll
    for (int j = 0; j < P; ++j)
        lds[lds_slot(j * kWave + lane)] = v[j];
}

// Buffer resource over `bytes` bytes at `base` (raw, stride 0). Stores at an
// offset past `bytes` are discarded by the hardware's range check, which is
// how lanes without data of a kind skip a store without a branch.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_over(void* base, int bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(base, (short)0, bytes, 0x00020000);
}

constexpr int kOffRange = 0x7ffffff0;   // a store offset past any tile's output
constexpr int kOutStorePolicy = 17;     // output stores: sc0 sc1 (system scope; measured fastest)

// Writes one tile's quantized output: block b's 8 packed bytes and its scale
// byte (lanes past a partial tile's end carry block b = nblk - 1 again).
// Wide path - every row's block count a multiple of 16, packed and scales
// 16-byte aligned: the 8*nblk + nblk bytes go through the wave's LDS area
// (packed at 0, scales at 512) and leave as 16-byte lane stores, lane L
// writing LDS bytes [16L, 16L + 16): lanes 0..31 the packed bytes, lanes
// 32..63 the scale bytes, each through a buffer resource that spans exactly
// that tile's bytes of its kind, so the other lanes' stores (and, in a
// partial tile, the lanes past the data) fall out of range and are dropped.
// Narrow path: 8-byte and 1-byte lane stores straight from registers.
// With keep == false (a paged write whose slot is skipped) nothing is
// stored: the wide path's windows are empty, so the hardware drops every
// store without a branch.
template <bool kWide>
__device__ __forceinline__ void store_tile_outputs(uint8_t* lds_bytes, uint2 q, uint32_t sf,
                                                   const Tile& t, int b, int lane,
                                                   const Geometry& geo, uint8_t* packed,
                                                   uint8_t* scales, bool keep = true)
{
    const int64_t tb = (int64_t)t.row * geo.bpr + t.blk0;   // first block of the tile
    if constexpr (!kWide) {
        if (keep) {
            *reinterpret_cast<uint2*>(packed + (tb + b) * 8) = q;
            scales[tb + b] = (uint8_t)sf;
        }
    } else {
        wave_lds_sync();
        reinterpret_cast<u32x2*>(lds_bytes)[b] = u32x2{q.x, q.y};
        lds_bytes[kTileBlocks * 8 + b] = (uint8_t)sf;
        wave_lds_sync();
        const u32x4 d = reinterpret_cast<const u32x4*>(lds_bytes)[lane];
        const bool scale_lane = lane >= kWave / 2;
        const int off = (lane & (kWave / 2 - 1)) * 16;
        __builtin_amdgcn_raw_buffer_store_b128(d, buffer_over(packed + tb * 8, keep ? t.nblk * 8 : 0),
                                               scale_lane ? kOffRange : off, 0, kOutStorePolicy);
        __builtin_amdgcn_raw_buffer_store_b128(d, buffer_over(scales + tb, keep ? t.nblk : 0),
                                               scale_lane ? off : kOffRange, 0, kOutStorePolicy);
    }
}

// Grouped wide store, for a wave that walks its tiles in groups of G
// consecutive ones (walk_tiles). A group's scale bytes are adjacent in memory
// (a row's last tile is followed by the next row's first), so they gather in
// the wave's scale window in LDS (`win`, 64 * G bytes, kept across the
// group) and leave as one piece of up to 64 * G bytes with the group's last
// tile, or with the grid's last tile, instead of one 64-byte piece per tile.
// Every tile runs the same instructions: the scale store of a tile that does
// not close its group has an empty range and is dropped. Lanes 32.. hold the
// window's 16-byte words (lanes past it re-read its words; their stores fall
// out of range), lanes 0..31 the tile's packed bytes as in store_tile_outputs.
struct ScaleWindow {
    int64_t first;   // block index of the window's first scale byte
    int n;           // scale bytes gathered so far
};

template <int G>
__device__ __forceinline__ void store_tile_outputs_grouped(uint8_t* lds_bytes, uint8_t* win,
                                                           uint2 q, uint32_t sf, const Tile& t,
                                                           int tile, int b, int lane,
                                                           const Geometry& geo, uint8_t* packed,
                                                           uint8_t* scales, ScaleWindow& ws)
{
    const int64_t tb = (int64_t)t.row * geo.bpr + t.blk0;   // first block of the tile
    const bool opens = tile % G == 0;
    const bool closes = tile % G == G - 1 || tile + 1 >= geo.tiles;
    const int at = opens ? 0 : ws.n;
    ws.first = opens ? tb : ws.first;
    wave_lds_sync();
    reinterpret_cast<u32x2*>(lds_bytes)[b] = u32x2{q.x, q.y};
    win[at + b] = (uint8_t)sf;
    wave_lds_sync();
    const bool scale_lane = lane >= kWave / 2;
    const int off = (lane & (kWave / 2 - 1)) * 16;
    const u32x4* src = scale_lane ? reinterpret_cast<const u32x4*>(win) + (lane & (4 * G - 1))
                                  : reinterpret_cast<const u32x4*>(lds_bytes) + lane;
    const u32x4 d = *src;
    __builtin_amdgcn_raw_buffer_store_b128(d, buffer_over(packed + tb * 8, t.nblk * 8),
                                           scale_lane ? kOffRange : off, 0, kOutStorePolicy);
    __builtin_amdgcn_raw_buffer_store_b128(d, buffer_over(scales + ws.first,
                                                          closes ? at + t.nblk : 0),
                                           scale_lane ? off : kOffRange, 0, kOutStorePolicy);
    ws.n = at + t.nblk;
}

// Block values from its staged words. kWaves is the workgroup size in waves
// and kBlocksPerCU the persistent grid's workgroups per CU (what LDS allows).
struct FusedBlock {
    static constexpr int P = 4;
    // 8 waves per CU (2 per SIMD) keep enough loads in flight; measured on
    // the prefill shape, 12 or 16 waves per CU are 4-6% slower and 4 waves
    // per CU 25% slower.
    static constexpr int kWaves = 8;
    static constexpr int kBlocksPerCU = 1;   // 64 KB sigma table + 8 x 4.25 KB staging
    static constexpr bool kSigmaTable = true;
    // element quotients: guarded fast path (full-significand FP32 values)
    static constexpr bool kFastQuotient = true;
    // Consecutive tiles per wave with wide stores (their scale bytes leave
    // as one piece). Measured on the prefill shape: 2 and 4 are 1.5-1.7%
    // slower than 1 and 8 is 6% slower; the walk's read order matters more
    // here than the size of the scale pieces.
    static constexpr int kScaleGroup = 1;
    // The block's 16 values y = silu(gate) * up = (gate * up) * sigma(gate)
    // and their largest magnitude, with sigma from the table in LDS: all 16
    // table reads are issued before the first product, so that their
    // latencies overlap. Each value is swiglu_product of the binary32 g u.
    // Its amax (NaN-propagating) is finite unless some g u left the binary32
    // range (only gates or ups of magnitude near 2^64 and beyond make one)
    // or an input is not finite; such blocks take swiglu, with g u in
    // binary64, for every value (lanes diverge; waves without such a block
    // skip it).
    __device__ static __forceinline__ float block(const u32x4 (&c)[4], float (&y)[16],
                                                  const uint8_t* sig)
    {
        const uint32_t gw[8] = {c[0].x, c[0].y, c[0].z, c[0].w, c[2].x, c[2].y, c[2].z, c[2].w};
        const uint32_t uw[8] = {c[1].x, c[1].y, c[1].z, c[1].w, c[3].x, c[3].y, c[3].z, c[3].w};
        double e[16];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            uint32_t o = nvfp4::sigma_offsets(gw[i]);
            // keep o whole: one shift-or builds it, then one mask and one
            // shift split it (the compiler would otherwise rebuild each half)
            asm("" : "+v"(o));
            e[2 * i] = *reinterpret_cast<const double*>(sig + (o & 0xffffu));
            e[2 * i + 1] = *reinterpret_cast<const double*>(sig + (o >> 16));
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            y[2 * i] = nvfp4::swiglu_product(nvfp4::bf16_lo(gw[i]) * nvfp4::bf16_lo(uw[i]),
                                             e[2 * i]);
            y[2 * i + 1] = nvfp4::swiglu_product(nvfp4::bf16_hi(gw[i]) * nvfp4::bf16_hi(uw[i]),
                                                 e[2 * i + 1]);
        }
        float amax = nvfp4::block_amax(y);
        if (!(amax < __builtin_inff())) {
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                y[2 * i] = nvfp4::swiglu(nvfp4::bf16_lo(gw[i]), nvfp4::bf16_lo(uw[i]), e[2 * i]);
                y[2 * i + 1] = nvfp4::swiglu(nvfp4::bf16_hi(gw[i]), nvfp4::bf16_hi(uw[i]),
                                             e[2 * i + 1]);
            }
            amax = nvfp4::block_amax(y);
        }
        return amax;
    }
};

struct PlainBlock {
    static constexpr int P = 2;
    static constexpr int kWaves = 4;
    static constexpr int kBlocksPerCU = 3;   // 12 waves per CU: measured best (8: -9%, 24: -7%)
    static constexpr bool kSigmaTable = false;
    // element quotients: exact path only (BF16 values often sit on a tie)
    static constexpr bool kFastQuotient = false;
    // 128-byte scale pieces: 1.5% faster than 1 tile on 65536 x 3072
    // (4 tiles: level with 1; 8 tiles: 3% slower).
    static constexpr int kScaleGroup = 2;
    __device__ static __forceinline__ float block(const u32x4 (&c)[2], float (&y)[16],
                                                  const uint8_t*)
    {
        const uint32_t w[8] = {c[0].x, c[0].y, c[0].z, c[0].w, c[1].x, c[1].y, c[1].z, c[1].w};
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            y[2 * i] = nvfp4::bf16_lo(w[i]);
            y[2 * i + 1] = nvfp4::bf16_hi(w[i]);
        }
        return nvfp4::block_amax(y);
    }
};

// Where a wave's next group of G consecutive tiles comes from. Both
// schedules hand out the same groups to a workgroup: group q of workgroup
// blk is q = blk * kWaves + w + k * stride for w < kWaves and k = 0, 1, ...
// (stride = gridDim * kWaves), and a wave starts on its own first group
// (w = its index). StaticWalk then gives each wave every stride-th group from
// there on. WorkgroupQueue lets the workgroup's waves take the groups from a
// counter in LDS in that order instead, one group per claim, so that waves
// that run faster take more of them: without it the eight waves of a
// workgroup finish up to 10 us apart on the prefill shape.
struct StaticWalk {
    int stride;
    __device__ __forceinline__ void start() {}
    template <int G>
    __device__ __forceinline__ int next(int tile) const
    {
        return tile % G == G - 1 ? tile + (stride - 1) * G + 1 : tile + 1;
    }
};

template <int kWaves>
struct WorkgroupQueue {
    int* counter;   // LDS, kWaves at start (set in the workgroup's set-up)
    int stride;     // gridDim * kWaves
    int lane;
    int pending;    // a claim made one group ahead (valid in lane 0)
    // Claims the workgroup's next group number (one LDS atomic from lane 0).
    // The result is read a group later (next), so the atomic's latency is
    // hidden behind a tile's work.
    __device__ __forceinline__ int claim() const
    {
        int n = 0;
        if (lane == 0)
            n = __hip_atomic_fetch_add(counter, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        return n;
    }
    __device__ __forceinline__ void start() { pending = claim(); }
    template <int G>
    __device__ __forceinline__ int next(int tile)
    {
        if (tile % G != G - 1)
            return tile + 1;
        const int n = uniform(pending);
        pending = claim();
        return ((n / kWaves) * stride + (int)blockIdx.x * kWaves + n % kWaves) * G;
    }
};

// A wave's walk over its tiles: groups of G consecutive tiles, the first
// group starting at `tile` (a multiple of G), the next ones from `sched`.
// The caller has tile < geo.tiles, and runs `setup` (setup(0), then
// setup(1)) itself on waves without a tile so that every wave reaches its
// barrier once. The walk keeps one tile
// in flight and calls op(tile, t, b, y, amax) with each lane's block b of
// tile t, its 16 values y and their largest magnitude. Loop invariant: tile
// t is staged in LDS and no loads are in flight. Each pass issues the loads
// of the next tile first, computes tile t from LDS and runs op, then stages
// the next tile; op may store (its stores are the only memory operations
// younger than those loads, so the wait before staging does not wait for
// them) and may use the wave's LDS area between the two LDS syncs of the
// pass.
template <class Block, int G = 1, class Sched, class Setup, class Op>
__device__ __forceinline__ void walk_tiles(const uint16_t* in, int64_t ld_in, const Geometry& geo,
                                           int tile, Sched& sched, int lane, u32x4* lds,
                                           const uint8_t* sig, Setup&& setup, Op&& op)
{
    constexpr int P = Block::P;
    Tile t = tile_at(tile, geo);
    u32x4 v[P];
    // the workgroup's one-time set-up (LDS tables, ending in a barrier) runs
    // while the first tile's loads are in flight: phase 0 issues its global
    // loads ahead of the tile's, phase 1 writes the tables and syncs
    setup(0);
    load_tile<P>(v, in, ld_in, t, lane);
    setup(1);
    sched.start();
    stage_tile<P>(lds, v, lane);
    // Keeps the prologue's staging out of the loop: were the compiler to
    // merge it with the loop's own staging at the loop head, the merged
    // wait would have to drain every outstanding memory operation, this
    // tile's stores included (vmcnt counts stores too), on every pass.
    wave_lds_sync();
    for (;;) {
        const int next = sched.template next<G>(tile);
        const bool has_next = next < geo.tiles;
        Tile tn = t;
        if (has_next) {
            tn = tile_at(next, geo);
            load_tile<P>(v, in, ld_in, tn, lane);
        }
        wave_lds_sync();
        // In a partial tile the lanes past its end redo the tile's last block
        // (same values, same output bytes to the same place): no lane is
        // masked, so there is no branch around op's stores (a branch would
        // make the wait before the next staging also wait for them).
        const int b = min(lane, t.nblk - 1);
        u32x4 c[P];
#pragma unroll
        for (int k = 0; k < P; ++k)
            c[k] = lds[lds_slot(b * P + k)];
        float y[16];
        const float amax = Block::block(c, y, sig);
        op(tile, t, b, y, amax);
        if (!has_next)
            break;
        wave_lds_sync();
        stage_tile<P>(lds, v, lane);
        tile = next;
        t = tn;
    }
}

// ---- per-expert lookups, batched ---------------------------------------------
// With experts every tile needs its row's expert (and that expert's global
// scale). For up to kLdsExperts experts the kernels copy expert_offsets and
// gs into LDS once per workgroup; then every 64 tiles each lane of a wave
// looks up the expert of one of the wave's next 64 tiles (tile + lane *
// stride) with a branch-free binary search in LDS and prepares that tile's
// scale constants, and each tile reads its lane's values with v_readlane.
// LDS reads count against lgkmcnt, not vmcnt, so the lookups never wait for
// the tile loads or stores in flight. More experts fall back to a scalar
// search per tile.
constexpr int kLdsExperts = 1024;

struct ExpertTable {
    int32_t off[kLdsExperts];   // expert_offsets[0 .. E-1]
    float gs[kLdsExperts];      // gs[e], or 1.0 without gs
};

template <int kThreadsPerBlock>
__device__ __forceinline__ void fill_expert_table(ExpertTable& tab, const int32_t* offsets,
                                                  const float* gs, int num_experts)
{
    for (int i = threadIdx.x; i < num_experts; i += kThreadsPerBlock) {
        tab.off[i] = offsets[i];
        tab.gs[i] = gs != nullptr ? gs[i] : 1.0f;
    }
}

// Largest e < num_experts with off[e] <= row (off[0] = 0 <= row): binary
// lifting over powers of two, the same number of steps on every lane.
__device__ __forceinline__ int lds_expert_of(const int32_t* off, int num_experts, int row)
{
    int lo = 0;
    for (int step = 1 << (31 - __builtin_clz(num_experts)); step > 0; step >>= 1) {
        const int i = lo + step;
        if (i < num_experts && off[min(i, num_experts - 1)] <= row)
            lo = i;
    }
    return lo;
}

// Lane j holds the expert (and scale constants) of the wave's j-th tile
// from tile0 on (tile0 opens a group of G; see walk_tiles); tiles past the
// end get the last row's.
struct ExpertBatch {
    int e;
    float gs, k, rk;
    template <int G = 1>
    __device__ __forceinline__ void refill(const ExpertTable& tab, int num_experts, int tile0,
                                           int stride, const Geometry& geo, int lane)
    {
        const int tj = tile0 + (lane / G) * G * stride + lane % G;
        const int row = tj < geo.tiles ? tj / geo.cpr : geo.rows - 1;
        e = lds_expert_of(tab.off, num_experts, row);
        const nvfp4::RowScale r = nvfp4::row_scale(tab.gs[e]);
        gs = r.gs;
        k = r.k;
        rk = r.rk;
    }
    __device__ __forceinline__ int expert(int j) const { return __builtin_amdgcn_readlane(e, j); }
    __device__ __forceinline__ nvfp4::RowScale scale(int j) const
    {
        nvfp4::RowScale r;
        r.gs = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(gs), j));
        r.k = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(k), j));
        r.rk = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(rk), j));
        r.pow2 = (__float_as_uint(r.gs) & 0x007fffffu) == 0;
        return r;
    }
};

// sigma(g) = 1 / (1 + e^-g) for the table's gates (generated by
// gen_sigma_table.py with 150-digit arithmetic): one binary64 per entry, low
// word first, positive magnitudes m = 0 .. kSigSpan - 1, then the negative
// ones. The LDS table is a plain copy of it.
__device__ const uint32_t kSigmaBits[] __attribute__((aligned(16))) = {
#include "sigma_table.inc"
};
static_assert(sizeof(kSigmaBits) == nvfp4::kSigFloats * 4, "one binary64 per entry");

// Copies the sigmoid table (fused input only) from kSigmaBits into the
// workgroup's LDS: 64 KB, eight 16-byte loads per thread, served by L2 after
// the first workgroups. Every wave of the workgroup takes part, so all of them
// reach the barrier. Two phases: load() issues the global loads into
// registers, store() writes them to LDS. A kernel issues load() before its
// first tile's loads: the wait before store() then covers only the table's
// own (L2) loads, which are older, and not the tile's HBM loads behind them
// (the memory counter retires loads in order).
template <class Block>
struct SigmaCopy {
    static constexpr int kThreadsPerBlock = Block::kWaves * kWave;
    static constexpr int kWords = Block::kSigmaTable ? nvfp4::kSigFloats / 4 : 0;   // 16-byte words
    static constexpr int kFull = kWords / kThreadsPerBlock;
    static constexpr int kRest = kWords - kFull * kThreadsPerBlock;
    static_assert(kRest < kThreadsPerBlock, "one more word for some threads");
    u32x4 v[kFull + 1];

    __device__ __forceinline__ void load()
    {
        if constexpr (Block::kSigmaTable) {
            const u32x4* src = reinterpret_cast<const u32x4*>(kSigmaBits);
#pragma unroll
            for (int k = 0; k < kFull; ++k)
                v[k] = src[k * kThreadsPerBlock + threadIdx.x];
            if (kRest > 0 && threadIdx.x < kRest)
                v[kFull] = src[kFull * kThreadsPerBlock + threadIdx.x];
        }
    }
    __device__ __forceinline__ void store(float* sig) const
    {
        if constexpr (Block::kSigmaTable) {
            u32x4* dst = reinterpret_cast<u32x4*>(sig);
#pragma unroll
            for (int k = 0; k < kFull; ++k)
                dst[k * kThreadsPerBlock + threadIdx.x] = v[k];
            if (kRest > 0 && threadIdx.x < kRest)
                dst[kFull * kThreadsPerBlock + threadIdx.x] = v[kFull];
        }
    }
};

template <class Block, bool kWide>
__global__ __launch_bounds__(Block::kWaves * kWave) void quantize_tiles_kernel(
    const uint16_t* __restrict__ in, int64_t ld_in, Geometry geo,
    const float* __restrict__ gs, const int32_t* __restrict__ offsets, int num_experts,
    uint8_t* __restrict__ packed, uint8_t* __restrict__ scales,
    float* __restrict__ values_out)
{
    constexpr int kWaves = Block::kWaves;
    constexpr int G = kWide ? Block::kScaleGroup : 1;
    __shared__ u32x4 stage[kWaves][kStageSlots(Block::P)];
    __shared__ u32x4 win[kWaves][4 * G];
    __shared__ __attribute__((aligned(16))) float sig[Block::kSigmaTable ? nvfp4::kSigFloats : 1];
    __shared__ ExpertTable tab;
    __shared__ int queue;
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = uniform(threadIdx.x / kWave);
    u32x4* lds = stage[wave];
    const int cols = geo.bpr * 16;
    const int tile = (blockIdx.x * kWaves + wave) * G;
    const int stride = gridDim.x * kWaves;
    const bool lds_experts = offsets != nullptr && num_experts <= kLdsExperts;
    // the fused kernel without experts shares its groups through an LDS queue
    // (see WorkgroupQueue; measured on the prefill shape: 4% faster). The
    // standalone quantize, whose waves carry little compute, keeps the static
    // walk (the queue measured 0.8% slower there).
    const bool queued = Block::kSigmaTable && offsets == nullptr;
    SigmaCopy<Block> table;
    auto setup = [&](int phase) {
        if (phase == 0) {
            table.load();
            return;
        }
        table.store(sig);
        if (lds_experts)
            fill_expert_table<kWaves * kWave>(tab, offsets, gs, num_experts);
        if (queued && threadIdx.x == 0)
            queue = kWaves;
        if (Block::kSigmaTable || lds_experts)
            __syncthreads();
    };
    if (tile >= geo.tiles) {
        setup(0);
        setup(1);
        return;
    }
    // Without experts the global scale (and its reciprocal) is the same for
    // every row: computed once here instead of per tile.
    nvfp4::RowScale rs = nvfp4::row_scale(gs != nullptr ? gs[0] : 1.0f);
    ExpertBatch batch;
    ScaleWindow ws{0, 0};
    int n = 0;   // tiles done by this wave
    auto body = [&](int tile_index, const Tile& t, int b, const float (&y)[16], float amax) {
        if (lds_experts) {
            const int j = n & (kWave - 1);
            if (j == 0)
                batch.refill<G>(tab, num_experts, tile_index, stride, geo, lane);
            rs = batch.scale(j);
            ++n;
        } else if (offsets != nullptr) {
            rs = nvfp4::row_scale(nvfp4::row_global_scale(gs, offsets, num_experts, t.row));
        }
        uint32_t sf;
        const uint2 q = nvfp4::quantize16<Block::kFastQuotient>(y, amax, rs, sf);
        if constexpr (kWide)
            store_tile_outputs_grouped<G>(reinterpret_cast<uint8_t*>(lds),
                                          reinterpret_cast<uint8_t*>(win[wave]), q, sf, t,
                                          tile_index, b, lane, geo, packed, scales, ws);
        else
            store_tile_outputs<false>(reinterpret_cast<uint8_t*>(lds), q, sf, t, b, lane, geo,
                                      packed, scales);
        if (values_out != nullptr) {
            f32x4* dst = reinterpret_cast<f32x4*>(values_out + (int64_t)t.row * cols) +
                         (t.blk0 + b) * 4;
#pragma unroll
            for (int i = 0; i < 4; ++i)
                dst[i] = f32x4{y[4 * i], y[4 * i + 1], y[4 * i + 2], y[4 * i + 3]};
        }
    };
    // With experts each wave keeps its own sequence, which the per-lane
    // expert lookahead (64 tiles ahead) relies on.
    if (queued) {
        WorkgroupQueue<kWaves> q{&queue, stride, lane, 0};
        walk_tiles<Block, G>(in, ld_in, geo, tile, q, lane, lds,
                             reinterpret_cast<const uint8_t*>(sig), setup, body);
    } else {
        StaticWalk w{stride};
        walk_tiles<Block, G>(in, ld_in, geo, tile, w, lane, lds,
                             reinterpret_cast<const uint8_t*>(sig), setup, body);
    }
}

// ---------------------------------------------------------------------------
// Compact SwiGLU output, the first pass of the two-pass variant (SwiGLU to
// BF16, then nvfp4_quantize): y = silu(gate) * up exactly as the fused
// kernel computes it, rounded to BF16 (round to nearest even, by
// v_cvt_pk_bf16_f32) and written as [rows][ld_out] BF16. A lane's block is
// 32 output bytes; the wave transposes its tile through LDS and writes it as
// two coalesced 1 KB stores, through a buffer resource spanning the tile's
// bytes so that a partial tile's surplus lanes are dropped.
// ---------------------------------------------------------------------------
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi)
{
    const bf16x2 b = __builtin_convertvector(f32x2{lo, hi}, bf16x2);
    return __builtin_bit_cast(uint32_t, b);
}

// ---------------------------------------------------------------------------
// Paged KV-cache write: the standalone quantize of a row of BF16 values
// (keys or values of one token, all heads), stored in cache row
// slots[row] instead of row `row`. A slot outside [0, num_slots) (a padding
// token's -1) is skipped. The slot is wave-uniform (one row per tile): one
// scalar load per tile.
// ---------------------------------------------------------------------------
template <bool kWide>
__global__ __launch_bounds__(PlainBlock::kWaves * kWave) void quantize_paged_kernel(
    const uint16_t* __restrict__ in, int64_t ld_in, Geometry geo, const float* __restrict__ gs,
    const int64_t* __restrict__ slots, int64_t num_slots, uint8_t* __restrict__ packed,
    uint8_t* __restrict__ scales)
{
    constexpr int kWaves = PlainBlock::kWaves;
    __shared__ u32x4 stage[kWaves][kStageSlots(PlainBlock::P)];
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = uniform(threadIdx.x / kWave);
    const int tile = blockIdx.x * kWaves + wave;
    if (tile >= geo.tiles)
        return;
    const nvfp4::RowScale rs = nvfp4::row_scale(gs != nullptr ? gs[0] : 1.0f);
    StaticWalk walk{(int)gridDim.x * kWaves};
    walk_tiles<PlainBlock>(in, ld_in, geo, tile, walk, lane, stage[wave], nullptr,
                           [](int) {}, [&](int, const Tile& t, int b, const float (&y)[16], float amax) {
        const int64_t slot = slots[t.row];
        const bool keep = slot >= 0 && slot < num_slots;
        Tile o = t;
        o.row = keep ? (int)slot : 0;
        uint32_t sf;
        const uint2 q = nvfp4::quantize16<PlainBlock::kFastQuotient>(y, amax, rs, sf);
        store_tile_outputs<kWide>(reinterpret_cast<uint8_t*>(stage[wave]), q, sf, o, b, lane, geo,
                                  packed, scales, keep);
    });
}

__global__ __launch_bounds__(FusedBlock::kWaves * kWave) void swiglu_bf16_kernel(
    const uint16_t* __restrict__ in, int64_t ld_in, Geometry geo, uint16_t* __restrict__ out,
    int64_t ld_out)
{
    using Block = FusedBlock;
    constexpr int kWaves = Block::kWaves;
    __shared__ u32x4 stage[kWaves][kStageSlots(Block::P)];
    __shared__ __attribute__((aligned(16))) float sig[nvfp4::kSigFloats];
    __shared__ int queue;
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = uniform(threadIdx.x / kWave);
    u32x4* lds = stage[wave];
    const int tile = blockIdx.x * kWaves + wave;
    SigmaCopy<Block> table;
    auto setup = [&](int phase) {
        if (phase == 0) {
            table.load();
            return;
        }
        table.store(sig);
        if (threadIdx.x == 0)
            queue = kWaves;
        __syncthreads();
    };
    if (tile >= geo.tiles) {
        setup(0);
        setup(1);
        return;
    }
    WorkgroupQueue<kWaves> walk{&queue, (int)gridDim.x * kWaves, lane, 0};
    walk_tiles<Block>(in, ld_in, geo, tile, walk, lane, lds,
                      reinterpret_cast<const uint8_t*>(sig), setup,
                      [&](int, const Tile& t, int b, const float (&y)[16], float) {
        u32x4 w[2];
#pragma unroll
        for (int h = 0; h < 2; ++h)
            w[h] = u32x4{pack_bf16x2(y[8 * h], y[8 * h + 1]), pack_bf16x2(y[8 * h + 2], y[8 * h + 3]),
                         pack_bf16x2(y[8 * h + 4], y[8 * h + 5]), pack_bf16x2(y[8 * h + 6], y[8 * h + 7])};
        wave_lds_sync();
        lds[lds_slot(2 * b)] = w[0];
        lds[lds_slot(2 * b + 1)] = w[1];
        wave_lds_sync();
        const __amdgpu_buffer_rsrc_t rsrc =
            buffer_over(out + (int64_t)t.row * ld_out + t.blk0 * 16, t.nblk * 32);
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int k = j * kWave + lane;
            __builtin_amdgcn_raw_buffer_store_b128(lds[lds_slot(k)], rsrc, k * 16, 0,
                                                   kOutStorePolicy);
        }
    });
}

// ---------------------------------------------------------------------------
// Global-scale pre-pass of the two-level scaling: amax of the quantizer's
// input values (the SwiGLU outputs, or the BF16 values) over the rows of
// each expert (or of the whole tensor), then gs = amax / (6 * 448).
// Three launches: zero the accumulator, reduce, finalize. The reduction
// folds each tile's maximum into a per-workgroup LDS array (one slot per
// expert) and flushes it with one global atomic max per touched expert.
// The maxima are non-negative floats, whose order is that of their bit
// patterns as unsigned integers, so the atomics work on the bits.
// ---------------------------------------------------------------------------
constexpr int kMaxScaleGroups = 1024;    // experts per global-scale call (LDS slots)
constexpr float kFp4Fp8Max = 6.0f * 448.0f;

__device__ __forceinline__ float wave_max(float v)
{
#pragma unroll
    for (int o = kWave / 2; o > 0; o >>= 1)
        v = fmaxf(v, __shfl_xor(v, o));
    return v;
}

__global__ void fill_u32_kernel(uint32_t* __restrict__ p, int n, uint32_t value)
{
    for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x)
        p[i] = value;
}

template <class Block>
__global__ __launch_bounds__(Block::kWaves * kWave) void amax_tiles_kernel(
    const uint16_t* __restrict__ in, int64_t ld_in, Geometry geo,
    const int32_t* __restrict__ offsets, int groups, uint32_t* __restrict__ acc)
{
    constexpr int kWaves = Block::kWaves;
    static_assert(kMaxScaleGroups <= kLdsExperts, "experts of a global-scale call fit in LDS");
    __shared__ u32x4 stage[kWaves][kStageSlots(Block::P)];
    __shared__ __attribute__((aligned(16))) float sig[Block::kSigmaTable ? nvfp4::kSigFloats : 1];
    __shared__ uint32_t part[kMaxScaleGroups];
    __shared__ ExpertTable tab;
    __shared__ int queue;
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = uniform(threadIdx.x / kWave);
    const int tile = blockIdx.x * kWaves + wave;
    const int stride = gridDim.x * kWaves;
    // the SwiGLU pre-pass without experts shares its tiles through the LDS
    // queue, as the fused quantize does
    const bool queued = Block::kSigmaTable && offsets == nullptr;
    SigmaCopy<Block> table;
    auto setup = [&](int phase) {
        if (phase == 0) {
            table.load();
            return;
        }
        table.store(sig);
        for (int i = threadIdx.x; i < groups; i += kWaves * kWave)
            part[i] = 0u;
        if (offsets != nullptr)
            fill_expert_table<kWaves * kWave>(tab, offsets, nullptr, groups);
        if (threadIdx.x == 0)
            queue = kWaves;
        __syncthreads();
    };
    if (tile >= geo.tiles) {
        setup(0);
        setup(1);
    }
    if (tile < geo.tiles) {
        // Each lane keeps a running max over the wave's consecutive tiles of
        // one expert; the wave reduces it and folds it into the workgroup's
        // slot when the expert changes, and once at the end.
        float run = 0.0f;
        int cur = -1;
        ExpertBatch batch;
        int n = 0;
        auto flush = [&]() {
            const float m = wave_max(run);
            if (lane == 0)
                atomicMax(&part[cur], __float_as_uint(m));
        };
        auto body = [&](int tile_index, const Tile&, int, const float (&)[16], float amax) {
            int e = 0;
            if (offsets != nullptr) {
                const int j = n & (kWave - 1);
                if (j == 0)
                    batch.refill(tab, groups, tile_index, stride, geo, lane);
                e = batch.expert(j);
                ++n;
            }
            if (e != cur) {
                if (cur >= 0)
                    flush();
                cur = e;
                run = 0.0f;
            }
            run = fmaxf(run, amax);
        };
        if (queued) {
            WorkgroupQueue<kWaves> walk{&queue, stride, lane, 0};
            walk_tiles<Block>(in, ld_in, geo, tile, walk, lane, stage[wave],
                              reinterpret_cast<const uint8_t*>(sig), setup, body);
        } else {
            StaticWalk walk{stride};
            walk_tiles<Block>(in, ld_in, geo, tile, walk, lane, stage[wave],
                              reinterpret_cast<const uint8_t*>(sig), setup, body);
        }
        flush();
    }
    __syncthreads();
    for (int i = threadIdx.x; i < groups; i += kWaves * kWave) {
        const uint32_t m = part[i];
        if (m != 0u)
            atomicMax(&acc[i], m);
    }
}

// gs[e] = RN(amax[e] / 2688) (IEEE division) for a non-empty expert with a
// nonzero amax, 1.0 otherwise; then clamped to [kGsMin, kGsMax], the global
// scales the quantizers are exact for (outside it the remainders of their
// quotients can leave the normal binary32 range). acc holds the amax bits
// and may be the gs array itself.
constexpr float kGsMin = 0x1p-64f, kGsMax = 0x1p+64f;

__global__ void global_scale_kernel(const uint32_t* acc, float* gs, int n)
{
    for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) {
        const float a = __uint_as_float(acc[i]);
        const float g = a > 0.0f ? a / kFp4Fp8Max : 1.0f;
        gs[i] = __builtin_fminf(__builtin_fmaxf(g, kGsMin), kGsMax);
    }
}

// ---------------------------------------------------------------------------
// NVFP4 dequantize to FP32. A block's output is 4 words (64 bytes); each lane
// computes its block, the wave transposes the tile through LDS and writes it
// with coalesced stores.
// ---------------------------------------------------------------------------
// kPaged: output row r reads cache row slots[r] (a paged KV-cache read); a
// slot outside [0, num_slots) gives a row of zeros.
template <bool kPaged>
__global__ __launch_bounds__(kThreads) void nvfp4_dequantize_kernel(
    const uint8_t* __restrict__ packed, const uint8_t* __restrict__ scales, Geometry geo,
    const float* __restrict__ gs, const int32_t* __restrict__ offsets, int num_experts,
    float* __restrict__ out, const int64_t* __restrict__ slots, int64_t num_slots)
{
    constexpr int P = 4;
    __shared__ f32x4 stage[kWavesPerBlock][kStageSlots(P)];
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = uniform(threadIdx.x / kWave);
    f32x4* lds = stage[wave];
    const int cols = geo.bpr * 16;
    for (int tile = blockIdx.x * kWavesPerBlock + wave; tile < geo.tiles;
         tile += gridDim.x * kWavesPerBlock) {
        const Tile t = tile_at(tile, geo);
        const int nwords = t.nblk * P;
        const float g_s = nvfp4::row_global_scale(gs, offsets, num_experts, t.row);
        int64_t src_row = t.row;
        bool valid = true;
        if constexpr (kPaged) {
            const int64_t slot = slots[t.row];
            valid = slot >= 0 && slot < num_slots;
            src_row = valid ? slot : 0;
        }
        const int64_t ib = src_row * geo.bpr + t.blk0 + lane;
        wave_lds_sync();
        if (lane < t.nblk) {
            float v[16];
            if (valid) {
                const u32x2 pv = ld_stream(reinterpret_cast<const u32x2*>(packed) + ib);
                const uint32_t sf = __builtin_nontemporal_load(scales + ib);
                nvfp4::dequantize16(make_uint2(pv.x, pv.y), sf, g_s, v);
            } else {
#pragma unroll
                for (int k = 0; k < 16; ++k)
                    v[k] = 0.0f;
            }
#pragma unroll
            for (int k = 0; k < P; ++k)
                lds[lds_slot(lane * P + k)] = f32x4{v[4 * k], v[4 * k + 1], v[4 * k + 2], v[4 * k + 3]};
        }
        wave_lds_sync();
        f32x4* dst = reinterpret_cast<f32x4*>(out + (int64_t)t.row * cols) + t.blk0 * P;
#pragma unroll
        for (int j = 0; j < P; ++j)
            if (j * kWave + lane < nwords)
                st_stream(lds[lds_slot(j * kWave + lane)], dst + j * kWave + lane);
    }
}

// ---------------------------------------------------------------------------
// Host side: validation (no HIP call before it passes) and launch.
// ---------------------------------------------------------------------------
bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

// rows rows of pitch ld BF16 elements (rows, ld >= 0): the byte extent must be
// addressable with int64 offsets, or no such buffer can exist.
bool extent_ok(int64_t rows, int64_t ld) { return rows <= 1 || ld <= INT64_MAX / 2 / rows; }

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

// Persistent grid for the pipelined quantize kernels: enough workgroups to
// fill MI355X (256 CUs) at the occupancy the kernel's LDS and registers
// allow, never more than the tiles need.
constexpr int kMi355xCUs = 256;
template <class Block>
dim3 persistent_grid_for(const Geometry& g, int group = 1)
{
    const int64_t per_block = (int64_t)Block::kWaves * group;   // tiles a workgroup starts on
    const int64_t want = ((int64_t)g.tiles + per_block - 1) / per_block;
    const int64_t cap = (int64_t)kMi355xCUs * Block::kBlocksPerCU;
    return dim3((unsigned)(want < cap ? want : cap));
}

// The 16-byte store path needs every tile's output to start 16-byte aligned.
bool wide_stores(const Geometry& g, const uint8_t* packed, const uint8_t* scales)
{
    return g.bpr % 16 == 0 && aligned(packed, 16) && aligned(scales, 16);
}

template <class Block>
void launch_quantize(const Geometry& g, const uint16_t* in, int64_t ld, const float* gs,
                     const int32_t* offsets, int32_t num_experts, uint8_t* packed,
                     uint8_t* scales, float* values_out, hipStream_t stream)
{
    const dim3 block(Block::kWaves * kWave);
    if (wide_stores(g, packed, scales))
        hipLaunchKernelGGL((quantize_tiles_kernel<Block, true>),
                           persistent_grid_for<Block>(g, Block::kScaleGroup), block, 0, stream, in,
                           ld, g, gs, offsets, (int)num_experts, packed, scales, values_out);
    else
        hipLaunchKernelGGL((quantize_tiles_kernel<Block, false>), persistent_grid_for<Block>(g),
                           block, 0, stream, in, ld, g, gs, offsets, (int)num_experts, packed,
                           scales, values_out);
}

nvfp4_status_t launched()
{
    return hipGetLastError() == hipSuccess ? NVFP4_SUCCESS : NVFP4_ERROR_LAUNCH;
}

// Arguments of the global-scale calls beyond the input's: the scale groups
// (experts, or the whole tensor), at most kMaxScaleGroups, and 4-byte
// aligned outputs.
nvfp4_status_t check_scale_outputs(int32_t num_experts, const float* amax, const float* gs)
{
    if (!gs)
        return NVFP4_ERROR_INVALID_VALUE;
    if (num_experts > kMaxScaleGroups)
        return NVFP4_ERROR_UNSUPPORTED_SHAPE;
    if (!aligned(gs, 4) || (amax && !aligned(amax, 4)))
        return NVFP4_ERROR_MISALIGNED;
    return NVFP4_SUCCESS;
}

// Zero the accumulator (amax, or gs itself without amax), reduce the tiles
// (skipped for an empty input), write gs.
template <class Block>
nvfp4_status_t launch_global_scale(const Geometry* g, const uint16_t* in, int64_t ld,
                                   const int32_t* offsets, int32_t num_experts, float* amax,
                                   float* gs, hipStream_t stream)
{
    const int groups = offsets != nullptr ? num_experts : 1;
    uint32_t* acc = reinterpret_cast<uint32_t*>(amax != nullptr ? amax : gs);
    const dim3 small((groups + 255) / 256);
    hipLaunchKernelGGL(fill_u32_kernel, small, dim3(256), 0, stream, acc, groups, 0u);
    nvfp4_status_t st = launched();
    if (st == NVFP4_SUCCESS && g != nullptr) {
        hipLaunchKernelGGL((amax_tiles_kernel<Block>), persistent_grid_for<Block>(*g),
                           dim3(Block::kWaves * kWave), 0, stream, in, ld, *g, offsets, groups,
                           acc);
        st = launched();
    }
    if (st == NVFP4_SUCCESS) {
        hipLaunchKernelGGL(global_scale_kernel, small, dim3(256), 0, stream, acc, gs, groups);
        st = launched();
    }
    return st;
}

}  // namespace

extern "C" {

nvfp4_status_t nvfp4_quantize(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld_x,
                              const float* gs, const int32_t* expert_offsets,
                              int32_t num_experts, uint8_t* packed, uint8_t* scales,
                              hipStream_t stream)
{
    if (rows < 0 || cols < 0 || ld_x < cols || !extent_ok(rows, ld_x))
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
    if (!aligned(x, 16) || ld_x % 8 != 0 || !aligned(packed, 8))
        return NVFP4_ERROR_MISALIGNED;
    Geometry g;
    if ((st = make_geometry(rows, cols, g)) != NVFP4_SUCCESS)
        return st;
    launch_quantize<PlainBlock>(g, x, ld_x, gs, expert_offsets, num_experts, packed, scales,
                                nullptr, stream);
    return launched();
}

nvfp4_status_t swiglu_nvfp4_quantize(const uint16_t* gate_up, int64_t rows, int64_t inter,
                                     int64_t ld_in, const float* gs,
                                     const int32_t* expert_offsets, int32_t num_experts,
                                     uint8_t* packed, uint8_t* scales, float* swiglu_out,
                                     hipStream_t stream)
{
    if (rows < 0 || inter < 0 || inter > INT64_MAX / 2 || ld_in < 2 * inter ||
        !extent_ok(rows, ld_in))
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
    if (!aligned(gate_up, 16) || ld_in % 8 != 0 || !aligned(packed, 8) ||
        (swiglu_out && !aligned(swiglu_out, 16)))
        return NVFP4_ERROR_MISALIGNED;
    Geometry g;
    if ((st = make_geometry(rows, inter, g)) != NVFP4_SUCCESS)
        return st;
    launch_quantize<FusedBlock>(g, gate_up, ld_in, gs, expert_offsets, num_experts, packed,
                                scales, swiglu_out, stream);
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
    hipLaunchKernelGGL(nvfp4_dequantize_kernel<false>, grid_for(g), dim3(kThreads), 0, stream,
                       packed, scales, g, gs, expert_offsets, (int)num_experts, out,
                       (const int64_t*)nullptr, (int64_t)0);
    return launched();
}

nvfp4_status_t nvfp4_global_scale(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld_x,
                                  const int32_t* expert_offsets, int32_t num_experts,
                                  float* amax, float* gs, hipStream_t stream)
{
    if (rows < 0 || cols < 0 || ld_x < cols || !extent_ok(rows, ld_x))
        return NVFP4_ERROR_INVALID_VALUE;
    if (cols % 16 != 0)
        return NVFP4_ERROR_UNSUPPORTED_SHAPE;
    nvfp4_status_t st = check_experts(expert_offsets, num_experts);
    if (st == NVFP4_SUCCESS)
        st = check_scale_outputs(num_experts, amax, gs);
    if (st != NVFP4_SUCCESS)
        return st;
    Geometry g;
    const bool empty = rows == 0 || cols == 0;
    if (!empty) {
        if (!x)
            return NVFP4_ERROR_INVALID_VALUE;
        if (!aligned(x, 16) || ld_x % 8 != 0)
            return NVFP4_ERROR_MISALIGNED;
        if ((st = make_geometry(rows, cols, g)) != NVFP4_SUCCESS)
            return st;
    }
    return launch_global_scale<PlainBlock>(empty ? nullptr : &g, x, ld_x, expert_offsets,
                                           num_experts, amax, gs, stream);
}

nvfp4_status_t swiglu_nvfp4_global_scale(const uint16_t* gate_up, int64_t rows, int64_t inter,
                                         int64_t ld_in, const int32_t* expert_offsets,
                                         int32_t num_experts, float* amax, float* gs,
                                         hipStream_t stream)
{
    if (rows < 0 || inter < 0 || inter > INT64_MAX / 2 || ld_in < 2 * inter ||
        !extent_ok(rows, ld_in))
        return NVFP4_ERROR_INVALID_VALUE;
    if (inter % 16 != 0)
        return NVFP4_ERROR_UNSUPPORTED_SHAPE;
    nvfp4_status_t st = check_experts(expert_offsets, num_experts);
    if (st == NVFP4_SUCCESS)
        st = check_scale_outputs(num_experts, amax, gs);
    if (st != NVFP4_SUCCESS)
        return st;
    Geometry g;
    const bool empty = rows == 0 || inter == 0;
    if (!empty) {
        if (!gate_up)
            return NVFP4_ERROR_INVALID_VALUE;
        if (!aligned(gate_up, 16) || ld_in % 8 != 0)
            return NVFP4_ERROR_MISALIGNED;
        if ((st = make_geometry(rows, inter, g)) != NVFP4_SUCCESS)
            return st;
    }
    return launch_global_scale<FusedBlock>(empty ? nullptr : &g, gate_up, ld_in, expert_offsets,
                                           num_experts, amax, gs, stream);
}

nvfp4_status_t swiglu_bf16(const uint16_t* gate_up, int64_t rows, int64_t inter, int64_t ld_in,
                           uint16_t* out, int64_t ld_out, hipStream_t stream)
{
    if (rows < 0 || inter < 0 || inter > INT64_MAX / 2 || ld_in < 2 * inter || ld_out < inter ||
        !extent_ok(rows, ld_in) || !extent_ok(rows, ld_out))
        return NVFP4_ERROR_INVALID_VALUE;
    if (inter % 16 != 0)
        return NVFP4_ERROR_UNSUPPORTED_SHAPE;
    if (rows == 0 || inter == 0)
        return NVFP4_SUCCESS;
    if (!gate_up || !out)
        return NVFP4_ERROR_INVALID_VALUE;
    if (!aligned(gate_up, 16) || ld_in % 8 != 0 || !aligned(out, 16) ||
        ld_out % 8 != 0)
        return NVFP4_ERROR_MISALIGNED;
    Geometry g;
    nvfp4_status_t st = make_geometry(rows, inter, g);
    if (st != NVFP4_SUCCESS)
        return st;
    hipLaunchKernelGGL(swiglu_bf16_kernel, persistent_grid_for<FusedBlock>(g),
                       dim3(FusedBlock::kWaves * kWave), 0, stream, gate_up, ld_in, g, out, ld_out);
    return launched();
}

nvfp4_status_t nvfp4_quantize_paged(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld_x,
                                    const float* gs, const int64_t* slot_mapping,
                                    int64_t num_slots, uint8_t* packed_cache,
                                    uint8_t* scales_cache, hipStream_t stream)
{
    if (rows < 0 || cols < 0 || ld_x < cols || !extent_ok(rows, ld_x) || num_slots < 0)
        return NVFP4_ERROR_INVALID_VALUE;
    if (cols % 16 != 0 || num_slots > INT32_MAX)
        return NVFP4_ERROR_UNSUPPORTED_SHAPE;
    if (rows == 0 || cols == 0 || num_slots == 0)
        return NVFP4_SUCCESS;   // nothing to write (every slot is out of range)
    if (!x || !slot_mapping || !packed_cache || !scales_cache)
        return NVFP4_ERROR_INVALID_VALUE;
    if (!aligned(x, 16) || ld_x % 8 != 0 || !aligned(packed_cache, 8) ||
        !aligned(slot_mapping, 8))
        return NVFP4_ERROR_MISALIGNED;
    Geometry g;
    nvfp4_status_t st = make_geometry(rows, cols, g);
    if (st != NVFP4_SUCCESS)
        return st;
    const dim3 grid = persistent_grid_for<PlainBlock>(g);
    const dim3 block(PlainBlock::kWaves * kWave);
    if (wide_stores(g, packed_cache, scales_cache))
        hipLaunchKernelGGL(quantize_paged_kernel<true>, grid, block, 0, stream, x, ld_x, g, gs,
                           slot_mapping, num_slots, packed_cache, scales_cache);
    else
        hipLaunchKernelGGL(quantize_paged_kernel<false>, grid, block, 0, stream, x, ld_x, g, gs,
                           slot_mapping, num_slots, packed_cache, scales_cache);
    return launched();
}

nvfp4_status_t nvfp4_dequantize_paged(const uint8_t* packed_cache, const uint8_t* scales_cache,
                                      int64_t num_slots, const int64_t* slots, int64_t rows,
                                      int64_t cols, const float* gs, float* out,
                                      hipStream_t stream)
{
    if (rows < 0 || cols < 0 || num_slots < 0)
        return NVFP4_ERROR_INVALID_VALUE;
    if (cols % 16 != 0 || num_slots > INT32_MAX)
        return NVFP4_ERROR_UNSUPPORTED_SHAPE;
    if (rows == 0 || cols == 0)
        return NVFP4_SUCCESS;
    if (!slots || !out || (num_slots > 0 && (!packed_cache || !scales_cache)))
        return NVFP4_ERROR_INVALID_VALUE;
    if (!aligned(packed_cache, 8) || !aligned(out, 16) || !aligned(slots, 8))
        return NVFP4_ERROR_MISALIGNED;
    Geometry g;
    nvfp4_status_t st = make_geometry(rows, cols, g);
    if (st != NVFP4_SUCCESS)
        return st;
    hipLaunchKernelGGL(nvfp4_dequantize_kernel<true>, grid_for(g), dim3(kThreads), 0, stream,
                       packed_cache, scales_cache, g, gs, (const int32_t*)nullptr, 0, out, slots,
                       num_slots);
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
