"""Exact-rational restatement of NVFP4 block quantization, for pinning the
oracle on small inputs.

This is deliberately a different construction from the C oracle: every value
is a ``fractions.Fraction``; every binary32 rounding is the textbook
round-to-nearest-even of an exact rational; the FP8 scale is found by a
nearest search over the finite E4M3 values that PyTorch's ``float8_e4m3fn``
decodes (ties to the even code); the E2M1 magnitude is a nearest search over
the OCP E2M1 grid (ties to the even index). Pure Python, so only for small
inputs.
"""
from __future__ import annotations

import bisect
import math
from fractions import Fraction as F

import torch

HALF = F(1, 2)


def rn32(q: F) -> F:
    """Round an exact rational to the nearest binary32 (ties to even),
    including the subnormal range. Overflow is not expected here."""
    if q == 0:
        return F(0)
    sign = -1 if q < 0 else 1
    a = abs(q)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    while F(2) ** e > a:
        e -= 1
    while F(2) ** (e + 1) <= a:
        e += 1
    e = max(e, -126)                      # subnormals share the 2^-149 spacing
    ulp = F(2) ** (e - 23)
    n = a / ulp
    fl = n.numerator // n.denominator
    rem = n - fl
    if rem > HALF or (rem == HALF and fl % 2 == 1):
        fl += 1
    r = fl * ulp
    assert r < F(2) ** 128, "binary32 overflow"
    return sign * r


def round_half_even_int(q: F) -> int:
    fl = q.numerator // q.denominator
    rem = q - fl
    if rem > HALF or (rem == HALF and fl % 2 == 1):
        fl += 1
    return fl


# Finite non-negative E4M3 values, decoded by PyTorch (codes 0x00..0x7e).
_FP8_VALUES = [F(float(v)) for v in
               torch.arange(0, 0x7F, dtype=torch.uint8).view(torch.float8_e4m3fn)
               .to(torch.float64).tolist()]
assert all(_FP8_VALUES[i] < _FP8_VALUES[i + 1] for i in range(len(_FP8_VALUES) - 1))

# OCP E2M1: sign bit, 2 exponent bits (bias 1), 1 mantissa bit.
E2M1_GRID = [F(0), F(1, 2), F(1), F(3, 2), F(2), F(3), F(4), F(6)]


def fp8_value(code: int) -> F:
    return _FP8_VALUES[code]


def fp8_encode(v: F) -> int:
    """Nearest finite E4M3 value to v >= 0, ties to the even code; values at
    or above the largest finite value (448) saturate to it."""
    if v >= _FP8_VALUES[-1]:
        return len(_FP8_VALUES) - 1
    i = bisect.bisect_left(_FP8_VALUES, v)
    if _FP8_VALUES[i] == v:
        return i
    lo, hi = i - 1, i
    dlo, dhi = v - _FP8_VALUES[lo], _FP8_VALUES[hi] - v
    if dlo < dhi:
        return lo
    if dhi < dlo:
        return hi
    return lo if lo % 2 == 0 else hi


def e2m1_nearest_index(m: F) -> int:
    """Nearest E2M1 magnitude index to m in [0, 6], ties to the even index."""
    best = None
    for i, g in enumerate(E2M1_GRID):
        d = abs(m - g)
        if best is None or d < best[0] or (d == best[0] and i % 2 == 0):
            best = (d, i)
    return best[1]


def quantize_block(xs, gs: float = 1.0):
    """16 binary32 values -> (packed bytes list, scale code, bsf, v list)."""
    assert len(xs) == 16
    X = [F(float(x)) for x in xs]
    G = F(float(gs))
    amax = max(abs(x) for x in X)
    k = rn32(6 * G)
    bsf = rn32(amax / k)
    sf = fp8_encode(bsf)
    denom = rn32(fp8_value(sf) * G)
    codes, vs = [], []
    for x, xf in zip(X, xs):
        if denom == 0:
            v = F(0)
        else:
            s = rn32(x / denom)
            v = 2 * min(abs(s), F(6))
        hs = round_half_even_int(v)
        idx = e2m1_nearest_index(F(hs, 2))
        neg = math.copysign(1.0, float(xf)) < 0
        codes.append((8 if neg else 0) | idx)
        vs.append(v)
    packed = [codes[2 * i] | (codes[2 * i + 1] << 4) for i in range(8)]
    return packed, sf, bsf, vs


def dequant_value(nibble: int, sf: int, gs: float) -> F:
    """RN32(RN32(e2m1 * scale) * gs) from the format definitions."""
    sign = -1 if nibble & 8 else 1
    t = rn32(sign * E2M1_GRID[nibble & 7] * fp8_value(sf))
    return rn32(t * F(float(gs)))
