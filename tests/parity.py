"""Acceptance rules for comparing the HIP path with the CPU oracle.

Standalone quantize and dequantize: bit-exact.

Fused SwiGLU + NVFP4 (both sides round a binary64 SwiGLU value to binary32,
so a value sitting on a rounding boundary may fall either way):
  1. SwiGLU: |y_gpu - y_ref| <= max(2e-6 |y_ref|, 2^-149) with equal sign
     bits. The absolute term is one step of the binary32 subnormal grid: for
     results below 2^-126 a relative bound cannot be met by two roundings
     (and the GPU's FP32 product g u may itself be subnormal there).
  2. A scale byte may differ only when the oracle's block scale before the
     FP8 cast lies within 1e-6 (relative) of an FP8 rounding midpoint; the
     block's 16 codes are then exempt as well.
  3. A code may differ only when the oracle's 2 min(|s|, 6) lies within 1e-6
     (relative) of a half-integer (a half-step rounding boundary).
  4. Exempt mismatches are at most 1e-5 of the elements; others: none.
  5. Zero tolerance: the oracle quantizer applied to the GPU's own FP32
     SwiGLU values reproduces the GPU's bytes exactly.

Compact SwiGLU pass (BF16 output of the two-pass variant): BF16 bits equal,
except where the oracle's FP32 SwiGLU lies within the SwiGLU tolerance
(max(2e-6 relative, 2^-149)) of a BF16 rounding midpoint; exempt mismatches
at most 1e-4 of the elements. The second pass is
the standalone quantize: bit-exact on the GPU's own BF16 values.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

import oracle

SWIGLU_RTOL = 2e-6
SWIGLU_ABS = 2.0 ** -149          # one binary32 subnormal step
BOUNDARY_RTOL = 1e-6
EXEMPT_FRACTION = 1e-5
BF16_EXEMPT_FRACTION = 1e-4


def nibbles(packed: np.ndarray) -> np.ndarray:
    """[rows][cols/2] bytes -> [rows][cols] codes (even element = low nibble)."""
    p = np.asarray(packed, np.uint8)
    out = np.empty((p.shape[0], p.shape[1] * 2), np.uint8)
    out[:, 0::2] = p & 15
    out[:, 1::2] = p >> 4
    return out


def assert_bytes_equal(what, got, want):
    got = np.asarray(got)
    want = np.asarray(want)
    assert got.shape == want.shape, (what, got.shape, want.shape)
    bad = np.argwhere(got != want)
    if bad.size:
        idx = tuple(bad[0])
        raise AssertionError("%s: %d mismatches; first at %s: got %s want %s"
                             % (what, len(bad), idx, got[idx], want[idx]))


_FP8 = np.array([oracle.fp8_decode(c) for c in range(0x7F)], np.float64)
_FP8_MID = (_FP8[:-1] + _FP8[1:]) / 2


def near_fp8_midpoint(bsf: np.ndarray) -> np.ndarray:
    """bsf within BOUNDARY_RTOL (relative) of a midpoint between two
    consecutive finite E4M3 values (where the FP8 cast changes its result)."""
    b = np.asarray(bsf, np.float64)
    i = np.searchsorted(_FP8_MID, b)
    lo = _FP8_MID[np.clip(i - 1, 0, _FP8_MID.size - 1)]
    hi = _FP8_MID[np.clip(i, 0, _FP8_MID.size - 1)]
    return (np.abs(b - lo) <= BOUNDARY_RTOL * lo) | (np.abs(b - hi) <= BOUNDARY_RTOL * hi)


def near_half_step_boundary(v: np.ndarray) -> np.ndarray:
    v = np.asarray(v, np.float64)
    b = np.floor(v) + 0.5
    return np.abs(v - b) <= BOUNDARY_RTOL * b


@dataclass
class FusedReport:
    elements: int
    swiglu_bad: int
    scale_mismatch: int
    scale_exempt: int
    code_mismatch: int
    code_exempt: int
    requant_mismatch: int

    def ok(self) -> bool:
        return (self.swiglu_bad == 0 and self.scale_mismatch == self.scale_exempt
                and self.code_mismatch == self.code_exempt and self.requant_mismatch == 0
                and self.code_exempt <= EXEMPT_FRACTION * self.elements)


def check_swiglu(y_gpu: np.ndarray, y_ref: np.ndarray) -> int:
    yg = np.asarray(y_gpu, np.float64)
    yr = np.asarray(y_ref, np.float64)
    # the sign bit is the code's sign bit: it must agree also for zeros and
    # for the subnormal values that the absolute term admits
    with np.errstate(invalid="ignore"):
        close = np.abs(yg - yr) <= np.maximum(SWIGLU_RTOL * np.abs(yr), SWIGLU_ABS)
    same = yg == yr                                  # infinities included
    ok = (close | same) & (np.signbit(yg) == np.signbit(yr))
    return int(np.count_nonzero(~ok))


def fused_report(packed, scales, y_gpu, ref_packed, ref_scales, ref_y, ref_bsf, ref_v,
                 gs_rows=None) -> FusedReport:
    codes, ref_codes = nibbles(packed), nibbles(ref_packed)
    n = codes.size
    sbad = scales != ref_scales
    sexempt = sbad & near_fp8_midpoint(ref_bsf)
    block_exempt = np.repeat(sexempt, 16, axis=1)
    cbad = codes != ref_codes
    cexempt = cbad & (block_exempt | near_half_step_boundary(ref_v))
    swiglu_bad = check_swiglu(y_gpu, ref_y) if y_gpu is not None else 0
    requant = 0
    if y_gpu is not None:
        rp, rs = oracle.quantize_f32(np.asarray(y_gpu, np.float32), gs_rows)
        requant = int(np.count_nonzero(rp != packed) + np.count_nonzero(rs != scales))
    return FusedReport(n, swiglu_bad, int(sbad.sum()), int(sexempt.sum()),
                       int(cbad.sum()), int(cexempt.sum()), requant)


def assert_fused_ok(rep: FusedReport, what: str):
    assert rep.ok(), "%s: %s" % (what, rep)


def near_bf16_midpoint(y_ref: np.ndarray) -> np.ndarray:
    """FP32 y within SWIGLU_RTOL (relative) of the midpoint between the two
    BF16 values around it (where the BF16 rounding changes its result)."""
    y = np.ascontiguousarray(y_ref, np.float32)
    mid = ((y.view(np.uint32) & np.uint32(0xFFFF0000)) | np.uint32(0x8000)).view(np.float32)
    yd = y.astype(np.float64)
    with np.errstate(invalid="ignore"):     # inf / NaN y: never a midpoint
        return np.abs(yd - mid.astype(np.float64)) <= np.maximum(SWIGLU_RTOL * np.abs(yd),
                                                                 SWIGLU_ABS)


@dataclass
class Bf16Report:
    elements: int
    mismatch: int
    exempt: int

    def ok(self) -> bool:
        return (self.mismatch == self.exempt
                and self.exempt <= max(2, BF16_EXEMPT_FRACTION * self.elements))


def bf16_report(got_bits, ref_bits, y_ref) -> Bf16Report:
    got = np.ascontiguousarray(got_bits, np.uint16)
    ref = np.ascontiguousarray(ref_bits, np.uint16)
    yr = np.ascontiguousarray(y_ref, np.float32)
    assert got.shape == ref.shape == yr.shape
    bad = got != ref
    exempt = bad & near_bf16_midpoint(yr)
    return Bf16Report(int(got.size), int(bad.sum()), int(exempt.sum()))
