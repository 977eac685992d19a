"""Seeded synthetic inputs shaped like the MoE L1 epilogue workloads.

This module only draws random numbers and lays them out: it holds none of the
quantization or SwiGLU arithmetic, imports neither the HIP binding nor the
oracle, and is the one piece both sides share. Every generator is
deterministic in its seed (NumPy PCG64). Values are drawn in float64, rounded
to float32 and then to BF16 with round-to-nearest-even; BF16 tensors are
returned as ``uint16`` bit patterns.

Workloads (rows x interleaved BF16 columns):

* ``standalone``  128 x 256 plain BF16, N(0,1), with injected edge blocks
  (zero, -0, tiny, subnormal-scale, saturating, exact E2M1 and FP8 ties).
* ``fused_small`` 512 x 4096 interleaved [gate x8, up x8, ...] (I = 2048),
  gate and up ~ N(0, 1.5).
* ``decode``      8192 x 4096 (I = 2048), gate/up = 2 * Student-t(3), 1 % of
  elements x100, 2 % of output blocks with all 32 feeding inputs +0.0.
* ``prefill``     65536 x 6144 (I = 3072), gate/up ~ N(0,1) times a per-row
  lognormal(0,1) factor; generated in 4096-row chunks so any chunk can be
  regenerated alone.
* ``ragged``      131072 x 4096 (I = 2048), 256 experts with Zipf(1.1) row
  counts (rows grouped by expert, int32 offsets[257]), N(0,1) times a
  per-expert lognormal(0,1) factor.
* ``moe_gemm``    inputs of the MoE L1 grouped GEMM: activations
  x[tokens][hidden] ~ N(0,1), weights w1[E][2I][hidden] ~ N(0, 1/hidden)
  (so the accumulators are about N(0,1)), Zipf(1.1) expert row counts;
  ``exact=True`` draws x from multiples of 1/8 in [-2, 2] and w1 from
  multiples of 1/16 in [-1, 1], whose FP32 sums are exact in any order.
"""
from __future__ import annotations

import hashlib
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

CHUNK_ROWS = 4096


def _workers() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def _run_chunks(fn, n: int) -> None:
    """Run fn(k) for k in range(n) on a thread pool (NumPy's generators and
    array arithmetic release the GIL); results must not depend on order."""
    if n <= 1:
        for k in range(n):
            fn(k)
        return
    with ThreadPoolExecutor(max_workers=_workers()) as ex:
        list(ex.map(fn, range(n)))


# ---- layout helpers (no method arithmetic) -----------------------------------
def to_bf16_bits(a) -> np.ndarray:
    """float64/float32 -> float32 (RNE) -> BF16 bits (RNE). Finite inputs."""
    f = np.ascontiguousarray(a, dtype=np.float32)
    b = f.view(np.uint32)
    r = (b + np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(bits) -> np.ndarray:
    b = np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32)


def interleave(gate: np.ndarray, up: np.ndarray) -> np.ndarray:
    """gate, up [rows][I] -> [rows][2I] laid out [gate x8, up x8, ...]."""
    rows, inter = gate.shape
    assert up.shape == gate.shape and inter % 8 == 0
    g = gate.reshape(rows, inter // 8, 8)
    u = up.reshape(rows, inter // 8, 8)
    return np.stack([g, u], axis=2).reshape(rows, 2 * inter)


def sha256(a: np.ndarray) -> str:
    return hashlib.sha256(np.ascontiguousarray(a).tobytes()).hexdigest()


@dataclass
class Workload:
    name: str
    x: np.ndarray                  # uint16 BF16 bits, [rows][cols]
    fused: bool                    # True: interleaved gate/up input
    offsets: np.ndarray | None = None   # int32 [E+1] expert row offsets
    meta: dict = field(default_factory=dict)

    @property
    def rows(self) -> int:
        return self.x.shape[0]

    @property
    def out_cols(self) -> int:
        """Quantized columns: I for the fused path, cols for the plain one."""
        return self.x.shape[1] // 2 if self.fused else self.x.shape[1]


# ---- standalone quantize (128 x 256) ----------------------------------------
_TIES = [0.25, 0.75, 1.25, 1.75, 2.25, 2.5, 2.75, 3.25, 3.5, 3.75, 4.75, 5.0,
         5.25, 5.75, 6.0, 0.5]
_HALF_STEPS = [0.0, 0.5, 1.0, 1.5, 2.0, 2.5, 3.0, 3.5, 4.0, 4.5, 5.0, 5.5, 6.0,
               -6.0, -0.5, -3.5]


def _block_with_amax(rng, amax: float, sign: float = 1.0) -> np.ndarray:
    v = rng.uniform(-0.9, 0.9, 16) * amax
    v[rng.integers(16)] = sign * amax
    return v


def standalone_blocks(rng) -> list[tuple[str, np.ndarray]]:
    """The injected edge blocks of the standalone workload, 16 values each."""
    out: list[tuple[str, np.ndarray]] = []
    out += [("zero", np.zeros(16)), ("zero", np.zeros(16))]
    out += [("negzero", np.full(16, -0.0)), ("negzero", np.full(16, -0.0))]
    out += [("tiny", rng.standard_normal(16) * 1e-3) for _ in range(4)]
    for m in range(1, 8):                       # amax = 3m/256
        out.append(("subnormal_scale", _block_with_amax(rng, 3.0 * m / 256.0)))
    out.append(("subnormal_scale", _block_with_amax(rng, 0.006)))
    out.append(("subnormal_scale", _block_with_amax(rng, 0.0908203125, -1.0)))
    for a in (1440.0, 1488.0, 2688.0, 2784.0, 2816.0, 3072.0, 10240.0):
        out.append(("large", _block_with_amax(rng, a, -1.0 if a == 2816.0 else 1.0)))
    ties = np.array(_TIES)
    signs = np.where(rng.random(16) < 0.5, -1.0, 1.0)
    for d in (1.0, 1.25, 3.0 / 512.0):
        out.append(("e2m1_ties", ties * d))
        out.append(("e2m1_ties", -ties * d))
        out.append(("e2m1_ties", ties * d * signs))
    out.append(("half_steps", np.array(_HALF_STEPS)))
    out.append(("half_steps", -np.array(_HALF_STEPS)))
    for a in (6.375, 7.125, 11.625):
        out.append(("fp8_ties", _block_with_amax(rng, a)))
    return out


def standalone(seed: int = 1, rows: int = 128, cols: int = 256) -> Workload:
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((rows, cols))
    nb = cols // 16
    blocks = standalone_blocks(rng)
    slots = rng.choice(rows * nb, size=len(blocks), replace=False)
    kinds = {}
    for (kind, vals), s in zip(blocks, slots):
        r, b = divmod(int(s), nb)
        x[r, 16 * b:16 * b + 16] = vals
        kinds[(r, b)] = kind
    return Workload("standalone", to_bf16_bits(x), fused=False,
                    meta={"seed": seed, "injected": kinds})


# ---- fused workloads ----------------------------------------------------------
def fused_normal(rows: int, inter: int, seed: int, sigma: float = 1.5) -> Workload:
    rng = np.random.default_rng(seed)
    g = rng.normal(0.0, sigma, (rows, inter))
    u = rng.normal(0.0, sigma, (rows, inter))
    return Workload("fused_normal", to_bf16_bits(interleave(g, u)), fused=True,
                    meta={"seed": seed, "sigma": sigma})


def fused_small(seed: int = 2) -> Workload:
    w = fused_normal(512, 2048, seed, 1.5)
    w.name = "fused_small"
    return w


def decode(seed: int = 3, rows: int = 8192, inter: int = 2048) -> Workload:
    rng = np.random.default_rng(seed)
    g = 2.0 * rng.standard_t(3.0, (rows, inter))
    u = 2.0 * rng.standard_t(3.0, (rows, inter))
    g[rng.random((rows, inter)) < 0.01] *= 100.0
    u[rng.random((rows, inter)) < 0.01] *= 100.0
    zero_blocks = rng.random((rows, inter // 16)) < 0.02
    zmask = np.repeat(zero_blocks, 16, axis=1)
    g[zmask] = 0.0
    u[zmask] = 0.0
    return Workload("decode", to_bf16_bits(interleave(g, u)), fused=True,
                    meta={"seed": seed, "zero_blocks": int(zero_blocks.sum())})


def prefill_chunk(k: int, seed: int = 4, inter: int = 3072,
                  total_rows: int = 65536) -> np.ndarray:
    """Rows [4096k, 4096k + 4096) of the prefill workload (BF16 bits)."""
    n_chunks = (total_rows + CHUNK_ROWS - 1) // CHUNK_ROWS
    ss = np.random.SeedSequence(seed).spawn(n_chunks)[k]
    rng = np.random.default_rng(ss)
    nrows = min(CHUNK_ROWS, total_rows - k * CHUNK_ROWS)
    f = rng.lognormal(0.0, 1.0, (nrows, 1))
    g = rng.standard_normal((nrows, inter)) * f
    u = rng.standard_normal((nrows, inter)) * f
    return to_bf16_bits(interleave(g, u))


def prefill(seed: int = 4, rows: int = 65536, inter: int = 3072) -> Workload:
    n_chunks = (rows + CHUNK_ROWS - 1) // CHUNK_ROWS
    x = np.empty((rows, 2 * inter), np.uint16)

    def fill(k):
        x[k * CHUNK_ROWS:(k + 1) * CHUNK_ROWS] = prefill_chunk(k, seed, inter, rows)

    _run_chunks(fill, n_chunks)
    return Workload("prefill", x, fused=True, meta={"seed": seed})


def ragged_offsets(seed: int = 5, rows: int = 131072, experts: int = 256,
                   s: float = 1.1) -> np.ndarray:
    """Zipf(s) expert sizes: counts ~ multinomial(rows, p_k ~ k^-s), expert
    ids permuted, rows grouped by expert -> int32 offsets[experts + 1]."""
    rng = np.random.default_rng(np.random.SeedSequence(seed).spawn(2)[0])
    p = np.arange(1, experts + 1, dtype=np.float64) ** (-s)
    p /= p.sum()
    counts = rng.multinomial(rows, p)
    counts = counts[rng.permutation(experts)]
    off = np.zeros(experts + 1, np.int64)
    np.cumsum(counts, out=off[1:])
    return off.astype(np.int32)


def ragged(seed: int = 5, rows: int = 131072, inter: int = 2048,
           experts: int = 256) -> Workload:
    off = ragged_offsets(seed, rows, experts)
    ss_vals = np.random.SeedSequence(seed).spawn(2)[1]
    n_chunks = (rows + CHUNK_ROWS - 1) // CHUNK_ROWS
    children = ss_vals.spawn(n_chunks + 1)
    factors = np.random.default_rng(children[0]).lognormal(0.0, 1.0, experts)
    row_expert = np.repeat(np.arange(experts), np.diff(off.astype(np.int64)))
    x = np.empty((rows, 2 * inter), np.uint16)

    def fill(k):
        r0, r1 = k * CHUNK_ROWS, min(rows, (k + 1) * CHUNK_ROWS)
        rng = np.random.default_rng(children[k + 1])
        f = factors[row_expert[r0:r1]][:, None]
        g = rng.standard_normal((r1 - r0, inter)) * f
        u = rng.standard_normal((r1 - r0, inter)) * f
        x[r0:r1] = to_bf16_bits(interleave(g, u))

    _run_chunks(fill, n_chunks)
    return Workload("ragged", x, fused=True, offsets=off,
                    meta={"seed": seed, "experts": experts})


@dataclass
class GemmWorkload:
    x: np.ndarray            # BF16 bits [tokens][hidden]
    w1: np.ndarray           # BF16 bits [experts][2 inter][hidden]
    offsets: np.ndarray      # int32 [experts + 1]
    inter: int


def moe_gemm(seed: int = 6, tokens: int = 32768, hidden: int = 7168, inter: int = 3072,
             experts: int = 8, exact: bool = False) -> GemmWorkload:
    off = ragged_offsets(seed, tokens, experts)
    ss = np.random.SeedSequence(seed).spawn(3)
    n = 2 * inter
    x = np.empty((tokens, hidden), np.uint16)
    w = np.empty((experts, n, hidden), np.uint16)
    xc = ss[1].spawn((tokens + CHUNK_ROWS - 1) // CHUNK_ROWS)
    wc = ss[2].spawn(experts)

    def draw(rng, shape, std, den, top):
        if exact:
            return rng.integers(-top, top + 1, shape).astype(np.float64) / den
        return rng.standard_normal(shape) * std

    def fill_x(k):
        r0, r1 = k * CHUNK_ROWS, min(tokens, (k + 1) * CHUNK_ROWS)
        x[r0:r1] = to_bf16_bits(draw(np.random.default_rng(xc[k]), (r1 - r0, hidden), 1.0, 8, 16))

    def fill_w(e):
        w[e] = to_bf16_bits(draw(np.random.default_rng(wc[e]), (n, hidden),
                                 1.0 / np.sqrt(hidden), 16, 16))

    _run_chunks(fill_x, len(xc))
    _run_chunks(fill_w, experts)
    return GemmWorkload(x, w, off, inter)


# ---- small edge-case generators ----------------------------------------------
@dataclass
class KvWorkload:
    x: np.ndarray            # BF16 bits [tokens][heads * head_dim]
    slots: np.ndarray        # int64 [tokens]: cache row of each token, -1 for padding
    num_slots: int
    heads: int
    head_dim: int


def kv_cache(seed: int = 7, tokens: int = 65536, heads: int = 8, head_dim: int = 128,
             num_slots: int = 131072, pad_fraction: float = 0.01) -> KvWorkload:
    """Keys (or values) of `tokens` new tokens for a paged NVFP4 KV cache. Each
    head's values are N(0, 1) times a per-head lognormal(0, 1) scale (heads
    differ in range). The tokens take distinct slots drawn at random from the
    cache's `num_slots`, in random order; a `pad_fraction` of them are
    padding (slot -1)."""
    rng = np.random.default_rng(seed)
    scale = rng.lognormal(0.0, 1.0, heads).astype(np.float32)
    x = rng.standard_normal((tokens, heads, head_dim), dtype=np.float32) * scale[None, :, None]
    slots = rng.choice(num_slots, size=tokens, replace=False).astype(np.int64)
    slots[rng.random(tokens) < pad_fraction] = -1
    return KvWorkload(to_bf16_bits(x.reshape(tokens, heads * head_dim)), slots, num_slots, heads,
                      head_dim)


def random_plain(rows: int, cols: int, seed: int, scale: float = 1.0) -> np.ndarray:
    rng = np.random.default_rng(seed)
    return to_bf16_bits(rng.standard_normal((rows, cols)) * scale)


def random_fused(rows: int, inter: int, seed: int, scale: float = 1.0) -> np.ndarray:
    rng = np.random.default_rng(seed)
    g = rng.standard_normal((rows, inter)) * scale
    u = rng.standard_normal((rows, inter)) * scale
    return to_bf16_bits(interleave(g, u))


def random_offsets(rows: int, experts: int, seed: int, empty: int = 0) -> np.ndarray:
    """Sorted expert offsets with some forced-empty experts (edge cases)."""
    rng = np.random.default_rng(seed)
    cuts = np.sort(rng.integers(0, rows + 1, experts - 1))
    off = np.concatenate([[0], cuts, [rows]]).astype(np.int64)
    if empty:
        # collapse a few experts to zero rows (always the first and the last)
        picks = set(int(e) for e in rng.choice(experts, size=empty, replace=False))
        for e in sorted(picks | {0, experts - 1}):
            if e < experts - 1:
                off[e + 1] = off[e]
            else:
                off[e] = rows
        off = np.maximum.accumulate(off)
    return off.astype(np.int32)


CONFIGS = {
    "standalone": standalone,
    "fused_small": fused_small,
    "decode": decode,
    "prefill": prefill,
    "ragged": ragged,
}
