"""NumPy front end of the CPU oracle (``liboracle_nvfp4.so``).

TEST INFRASTRUCTURE ONLY. The oracle is the plain definition of NVFP4 block
quantization and of the fused SwiGLU + NVFP4 quantize step; the GPU library
is checked against it. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package. It shares no
code with the HIP path and never imports it.

Every function takes and returns host NumPy arrays. BF16 tensors travel as
``uint16`` bit patterns. ``gs_rows`` is one FP32 global scale per row (None
means 1.0); :func:`rows_global_scale` expands per-expert scales to rows.
"""
from __future__ import annotations

import ctypes as C
import os

import numpy as np

from . import build as _build

_LIB = None

_u8p = C.POINTER(C.c_uint8)
_u16p = C.POINTER(C.c_uint16)
_i32p = C.POINTER(C.c_int32)
_f32p = C.POINTER(C.c_float)
_i64 = C.c_int64


def lib():
    """Load the oracle library, building it with gcc if it is missing."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(_build.LIB):
            _build.build()
        L = C.CDLL(_build.LIB)
        L.oracle_bf16_to_f32.argtypes = [C.c_uint16]
        L.oracle_bf16_to_f32.restype = C.c_float
        L.oracle_swiglu.argtypes = [C.c_float, C.c_float]
        L.oracle_swiglu.restype = C.c_float
        L.oracle_fp8_e4m3_encode.argtypes = [C.c_float]
        L.oracle_fp8_e4m3_encode.restype = C.c_uint8
        L.oracle_fp8_e4m3_decode.argtypes = [C.c_uint8]
        L.oracle_fp8_e4m3_decode.restype = C.c_float
        L.oracle_e2m1_index.argtypes = [C.c_int]
        L.oracle_e2m1_index.restype = C.c_int
        L.oracle_e2m1_decode.argtypes = [C.c_uint8]
        L.oracle_e2m1_decode.restype = C.c_float
        L.oracle_quantize_block.argtypes = [_f32p, C.c_float, _u8p, _u8p, _f32p, _f32p]
        L.oracle_quantize_block.restype = None
        L.oracle_fp8_encode_array.argtypes = [_f32p, _i64, _u8p]
        L.oracle_swiglu_rows.argtypes = [_u16p, _i64, _i64, _i64, _f32p]
        L.oracle_swiglu_bf16_rows.argtypes = [_u16p, _i64, _i64, _i64, _u16p]
        L.oracle_swiglu_f32_rows.argtypes = [_f32p, _i64, _i64, _i64, _f32p]
        L.oracle_f32_to_bf16_array.argtypes = [_f32p, _i64, _u16p]
        L.oracle_quantize_f32_rows.argtypes = [_f32p, _i64, _i64, _i64, _f32p,
                                               _u8p, _u8p, _f32p, _f32p]
        L.oracle_quantize_bf16_rows.argtypes = [_u16p, _i64, _i64, _i64, _f32p,
                                                _u8p, _u8p]
        L.oracle_swiglu_quantize_rows.argtypes = [_u16p, _i64, _i64, _i64, _f32p,
                                                  _u8p, _u8p, _f32p, _f32p, _f32p]
        L.oracle_dequantize_rows.argtypes = [_u8p, _u8p, _i64, _i64, _f32p, _f32p]
        L.oracle_group_amax.argtypes = [_f32p, _i64, _i64, _i32p, C.c_int32, _f32p]
        L.oracle_num_threads.argtypes = []
        L.oracle_num_threads.restype = C.c_int
        L.oracle_set_num_threads.argtypes = [C.c_int]
        L.oracle_set_num_threads.restype = None
        _LIB = L
    return _LIB


def _p(a, t):
    return None if a is None else a.ctypes.data_as(t)


def _check(rc, what):
    if rc != 0:
        raise ValueError("oracle %s rejected its arguments" % what)


def _rows_gs(gs_rows, rows):
    if gs_rows is None:
        return None
    g = np.ascontiguousarray(gs_rows, dtype=np.float32)
    if g.shape != (rows,):
        raise ValueError("gs_rows must have one value per row")
    return g


def num_threads() -> int:
    return int(lib().oracle_num_threads())


def set_num_threads(n: int) -> None:
    lib().oracle_set_num_threads(int(n))


# ---- scalar primitives ------------------------------------------------------
def bf16_to_f32(bits: int) -> float:
    return float(lib().oracle_bf16_to_f32(int(bits)))


def swiglu_scalar(g: float, u: float) -> float:
    return float(lib().oracle_swiglu(float(g), float(u)))


def fp8_encode_scalar(v: float) -> int:
    return int(lib().oracle_fp8_e4m3_encode(float(v)))


def fp8_decode(code: int) -> float:
    return float(lib().oracle_fp8_e4m3_decode(int(code)))


def e2m1_index(half_step: int) -> int:
    return int(lib().oracle_e2m1_index(int(half_step)))


def e2m1_decode(nibble: int) -> float:
    return float(lib().oracle_e2m1_decode(int(nibble)))


def quantize_block(x, gs: float = 1.0):
    """One 16-value block -> (packed[8] uint8, sf, bsf, v[16])."""
    xb = np.ascontiguousarray(x, dtype=np.float32)
    assert xb.shape == (16,)
    packed = np.zeros(8, np.uint8)
    sf = np.zeros(1, np.uint8)
    bsf = np.zeros(1, np.float32)
    v = np.zeros(16, np.float32)
    lib().oracle_quantize_block(_p(xb, _f32p), C.c_float(gs), _p(packed, _u8p),
                                _p(sf, _u8p), _p(bsf, _f32p), _p(v, _f32p))
    return packed, int(sf[0]), float(bsf[0]), v


# ---- array drivers ----------------------------------------------------------
def fp8_encode(v: np.ndarray) -> np.ndarray:
    a = np.ascontiguousarray(v, dtype=np.float32).reshape(-1)
    out = np.empty(a.shape, np.uint8)
    _check(lib().oracle_fp8_encode_array(_p(a, _f32p), a.size, _p(out, _u8p)),
           "fp8_encode")
    return out.reshape(np.shape(v))


def swiglu(gate_up: np.ndarray) -> np.ndarray:
    """Interleaved BF16 [rows][2I] ([gate x8, up x8, ...]) -> FP32 [rows][I]."""
    x = np.ascontiguousarray(gate_up, dtype=np.uint16)
    rows, two_i = x.shape
    inter = two_i // 2
    y = np.empty((rows, inter), np.float32)
    _check(lib().oracle_swiglu_rows(_p(x, _u16p), rows, inter, two_i, _p(y, _f32p)),
           "swiglu")
    return y


def swiglu_f32(acc: np.ndarray) -> np.ndarray:
    """FP32 [rows][2I] interleaved accumulators -> FP32 SwiGLU [rows][I]."""
    a = np.ascontiguousarray(acc, dtype=np.float32)
    rows, two_i = a.shape
    inter = two_i // 2
    y = np.empty((rows, inter), np.float32)
    _check(lib().oracle_swiglu_f32_rows(_p(a, _f32p), rows, inter, two_i, _p(y, _f32p)),
           "swiglu_f32")
    return y


def moe_l1_gemm(x: np.ndarray, w1: np.ndarray, offsets=None, rows=None) -> np.ndarray:
    """The MoE L1 grouped GEMM in float64: acc[t][n] = sum_k x[t][k] w1[e(t)][n][k]
    with BF16 bit patterns x [tokens][hidden] and w1 [E][n][hidden], e(t) the
    expert holding row t (offsets [E+1]; None: one expert). Every product of
    two BF16 values is exact in float64 and the sums carry about 1e-16
    relative error. ``rows``: only these token rows (in that order)."""
    xs = np.asarray(x, np.uint16)
    ws = np.asarray(w1, np.uint16)
    if ws.ndim == 2:
        ws = ws[None]
    t_all = np.arange(xs.shape[0]) if rows is None else np.asarray(rows)
    if offsets is None:
        e_of = np.zeros(t_all.size, np.int64)
    else:
        e_of = np.searchsorted(np.asarray(offsets, np.int64), t_all, side="right") - 1
    out = np.empty((t_all.size, ws.shape[1]), np.float64)
    for e in np.unique(e_of):
        sel = np.nonzero(e_of == e)[0]
        xf = (xs[t_all[sel]].astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        wf = (ws[e].astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        out[sel] = xf @ wf.T
    return out


def f32_to_bf16(x: np.ndarray) -> np.ndarray:
    """FP32 values -> BF16 bit patterns (uint16), round to nearest even."""
    a = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(a.shape, np.uint16)
    _check(lib().oracle_f32_to_bf16_array(_p(a, _f32p), a.size, _p(out, _u16p)), "f32_to_bf16")
    return out


def swiglu_bf16(gate_up: np.ndarray) -> np.ndarray:
    """Interleaved BF16 [rows][2I] -> compact BF16 [rows][I] (bit patterns):
    the SwiGLU values rounded to BF16, the first pass of the two-pass variant."""
    x = np.ascontiguousarray(gate_up, dtype=np.uint16)
    rows, two_i = x.shape
    inter = two_i // 2
    out = np.empty((rows, inter), np.uint16)
    _check(lib().oracle_swiglu_bf16_rows(_p(x, _u16p), rows, inter, two_i, _p(out, _u16p)),
           "swiglu_bf16")
    return out


def quantize_f32(x: np.ndarray, gs_rows=None, diag: bool = False):
    """FP32 [rows][cols] -> packed [rows][cols/2], scales [rows][cols/16]
    (+ bsf [rows][cols/16] and v [rows][cols] when diag)."""
    a = np.ascontiguousarray(x, dtype=np.float32)
    rows, cols = a.shape
    packed = np.empty((rows, cols // 2), np.uint8)
    scales = np.empty((rows, cols // 16), np.uint8)
    bsf = np.empty((rows, cols // 16), np.float32) if diag else None
    v = np.empty((rows, cols), np.float32) if diag else None
    g = _rows_gs(gs_rows, rows)
    _check(lib().oracle_quantize_f32_rows(_p(a, _f32p), rows, cols, cols, _p(g, _f32p),
                                          _p(packed, _u8p), _p(scales, _u8p),
                                          _p(bsf, _f32p), _p(v, _f32p)),
           "quantize_f32")
    return (packed, scales, bsf, v) if diag else (packed, scales)


def quantize_bf16(x: np.ndarray, gs_rows=None):
    """BF16 bits [rows][cols] -> packed [rows][cols/2], scales [rows][cols/16]."""
    a = np.ascontiguousarray(x, dtype=np.uint16)
    rows, cols = a.shape
    packed = np.empty((rows, cols // 2), np.uint8)
    scales = np.empty((rows, cols // 16), np.uint8)
    g = _rows_gs(gs_rows, rows)
    _check(lib().oracle_quantize_bf16_rows(_p(a, _u16p), rows, cols, cols,
                                           _p(g, _f32p), _p(packed, _u8p),
                                           _p(scales, _u8p)),
           "quantize_bf16")
    return packed, scales


def swiglu_quantize(gate_up: np.ndarray, gs_rows=None, diag: bool = False):
    """Fused path definition: interleaved BF16 [rows][2I] ->
    (packed [rows][I/2], scales [rows][I/16], swiglu FP32 [rows][I]
    [, bsf [rows][I/16], v [rows][I]])."""
    x = np.ascontiguousarray(gate_up, dtype=np.uint16)
    rows, two_i = x.shape
    inter = two_i // 2
    packed = np.empty((rows, inter // 2), np.uint8)
    scales = np.empty((rows, inter // 16), np.uint8)
    y = np.empty((rows, inter), np.float32)
    bsf = np.empty((rows, inter // 16), np.float32) if diag else None
    v = np.empty((rows, inter), np.float32) if diag else None
    g = _rows_gs(gs_rows, rows)
    _check(lib().oracle_swiglu_quantize_rows(_p(x, _u16p), rows, inter, two_i,
                                             _p(g, _f32p), _p(packed, _u8p),
                                             _p(scales, _u8p), _p(y, _f32p),
                                             _p(bsf, _f32p), _p(v, _f32p)),
           "swiglu_quantize")
    return (packed, scales, y, bsf, v) if diag else (packed, scales, y)


def dequantize(packed: np.ndarray, scales: np.ndarray, gs_rows=None) -> np.ndarray:
    p = np.ascontiguousarray(packed, dtype=np.uint8)
    s = np.ascontiguousarray(scales, dtype=np.uint8)
    rows = p.shape[0]
    cols = p.shape[1] * 2
    if s.shape != (rows, cols // 16):
        raise ValueError("scales shape does not match packed")
    out = np.empty((rows, cols), np.float32)
    g = _rows_gs(gs_rows, rows)
    _check(lib().oracle_dequantize_rows(_p(p, _u8p), _p(s, _u8p), rows, cols,
                                        _p(g, _f32p), _p(out, _f32p)),
           "dequantize")
    return out


def quantize_paged(x: np.ndarray, slots, packed_cache: np.ndarray, scales_cache: np.ndarray,
                   gs: float | None = None):
    """Paged KV-cache write ("2026-05-28_STATUS.md": KV cache infra with a
    paged cache, FP4 quantize in the compressor; "Priority 7: NVFP4-2 FP4 KV
    pipeline"). Row r of the BF16 input is quantized exactly as
    quantize_bf16 does (one global scale for all rows) and its bytes replace
    cache row slots[r]; a slot outside [0, num_slots) skips the row. The
    caches are updated in place and returned. Rows are visited one by one so
    that the slot rule reads as written (no NumPy fancy indexing, whose
    negative indices would wrap)."""
    packed, scales = quantize_bf16(x, None if gs is None else np.full(x.shape[0], gs, np.float32))
    num_slots = packed_cache.shape[0]
    for r in range(x.shape[0]):
        slot = int(slots[r])
        if 0 <= slot < num_slots:
            packed_cache[slot, :] = packed[r]
            scales_cache[slot, :] = scales[r]
    return packed_cache, scales_cache


def dequantize_paged(packed_cache: np.ndarray, scales_cache: np.ndarray, slots,
                     gs: float | None = None) -> np.ndarray:
    """Paged KV-cache read: row r is the dequantize of cache row slots[r], or
    zeros for a slot outside [0, num_slots)."""
    num_slots, half = packed_cache.shape
    out = np.zeros((len(slots), 2 * half), np.float32)
    for r in range(len(slots)):
        slot = int(slots[r])
        if 0 <= slot < num_slots:
            out[r] = dequantize(packed_cache[slot:slot + 1], scales_cache[slot:slot + 1],
                                None if gs is None else np.full(1, gs, np.float32))[0]
    return out


def group_amax(y: np.ndarray, offsets: np.ndarray) -> np.ndarray:
    a = np.ascontiguousarray(y, dtype=np.float32)
    o = np.ascontiguousarray(offsets, dtype=np.int32)
    groups = o.size - 1
    out = np.empty(groups, np.float32)
    _check(lib().oracle_group_amax(_p(a, _f32p), a.shape[0], a.shape[1],
                                   _p(o, _i32p), groups, _p(out, _f32p)),
           "group_amax")
    return out


def expert_global_scale(amax: np.ndarray) -> np.ndarray:
    """Two-level NVFP4 global scale per expert: gs_e = RN32(amax_e / (6*448))
    (one IEEE binary32 division), so that the largest block scale of the
    expert lands on the FP8 maximum 448 ("NVFP4-1.1_APPROACH_PART_2.md", the
    l2_global_scale parameter of the fused kernel; the per-expert
    amax / (6 * 448) recipe of the ragged grouped MoE workload). An empty or
    all-zero expert gets 1.0 (its value is never used)."""
    a = np.asarray(amax, dtype=np.float32)
    with np.errstate(under="ignore"):
        gs = a / np.float32(6.0 * 448.0)          # binary32 IEEE division
    return np.where(a > 0, gs, np.float32(1.0)).astype(np.float32)


def rows_global_scale(gs: np.ndarray, offsets: np.ndarray, rows: int) -> np.ndarray:
    """Expand per-expert scales to one value per row (row r belongs to expert
    e when offsets[e] <= r < offsets[e+1])."""
    o = np.asarray(offsets, dtype=np.int64)
    g = np.asarray(gs, dtype=np.float32)
    out = np.empty(rows, np.float32)
    for e in range(o.size - 1):
        out[o[e]:o[e + 1]] = g[e]
    return out
