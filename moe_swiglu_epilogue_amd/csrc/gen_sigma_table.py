"""Writes sigma_table.inc, the sigmoid table of the fused SwiGLU kernels.

sigma(g) = 1 / (1 + e^-g) for every BF16 gate g whose magnitude has an
exponent field in 103..134 (2^-24 <= |g| < 256: all 32 * 128 = 4096
magnitudes), for g > 0 (entries 0..4095) and g < 0 (entries 4096..8191),
magnitude index m = (BF16 magnitude bits) - (103 << 7).

Main table, 8 bytes per entry:
* for every gate above -64, a pair of binary32 numbers, hi = sigma rounded
  toward zero and lo = RN(sigma - hi). hi + lo carries sigma to about 2^-47
  relative; both are normal numbers (sigma(-64) is about 2^-92) and lo >= 0,
  so a kernel can form (g u) sigma as fma(g u, hi, (g u) lo) with one final
  rounding, both terms with the sign of g u (a zero keeps its sign, an
  infinite product stays infinite);
* for the gates at or below -64 (negative magnitudes with exponent field 133
  or 134: the last 256 entries) the pair (+inf, +inf): there sigma drops
  from 2^-92 to about 2^-368, through and below the binary32 normal range,
  where a pair would lose precision. The marker makes the kernel's pair
  product infinite or NaN, which sends the block to its binary64 path.

Wide table, after the main one: the binary64 nearest to sigma for those 256
gates, in the same order. Its last entry, read for every gate at or below
-255 (the index saturates there), holds 2^-1000 instead of sigma(-255): for
such gates the SwiGLU value rounds to a zero with the sign of g u in binary32
(|y| is below 2^-231 for g = -255 and any BF16 up; below that gate
sigma < e^-256 and |g u| < 2^256), and any entry under 2^-406 gives that
zero.

Each sigma is evaluated with 150 significant decimal digits (Python's
decimal module: exp and division correctly rounded at that precision; enough
to resolve 1 - sigma(255) = e^-255, about 1.8e-111). sigma of a nonzero
binary number is transcendental, so it is never a representable value or a
rounding midpoint; the distance to both is checked.

The table holds 32-bit words: (hi, lo) bit patterns per main entry, then
each binary64 bit pattern low word first (the little-endian layout of a
double).

Run from the repository root:
    python moe_swiglu_epilogue_amd/csrc/gen_sigma_table.py
"""
import os
import struct
from decimal import Decimal, localcontext
from fractions import Fraction

import numpy as np

EXP_LO, EXP_HI = 103, 134
SPAN = (EXP_HI - EXP_LO + 1) * 128          # 4096 magnitudes
OUT = os.path.join(os.path.dirname(os.path.abspath(__file__)), "sigma_table.inc")
CLAMP_ENTRY = 2.0 ** -1000      # the last negative entry (gates <= -255)
WIDE_FIRST = 3840               # first negative index stored as binary64: gate -64


def bf16_magnitude(m: int) -> float:
    bits = ((EXP_LO << 7) + m) << 16
    return struct.unpack("<f", struct.pack("<I", bits))[0]


def sigma_decimal(g: float) -> Decimal:
    with localcontext() as ctx:
        ctx.prec = 150
        return Decimal(1) / (Decimal(1) + (-Decimal(g)).exp())


def round_binary32(d) -> np.float32:
    """Nearest binary32 of d (a Decimal or a Fraction), with a check that d is
    not near a tie."""
    q = Fraction(d)
    if q < 0:
        return -round_binary32(-q)
    c = np.float32(float(d))
    cands = sorted({c, np.nextafter(c, np.float32(np.inf)), np.nextafter(c, np.float32(0))},
                   key=lambda x: abs(Fraction(float(x)) - q))
    best, second = cands[0], cands[1]
    gap = abs(Fraction(float(second)) - q) - abs(Fraction(float(best)) - q)
    # the 150-digit value is within 1e-149 * q of sigma: a gap far above that
    # makes the rounding exact
    assert gap > q * Fraction(1, 10 ** 140), (d, best, second)
    return best


def truncate_binary32(d) -> np.float32:
    """The largest binary32 not above d (d >= 0), with a check that d is not
    near a binary32 value."""
    q = Fraction(d)
    c = np.float32(float(d))
    while Fraction(float(c)) > q:
        c = np.nextafter(c, np.float32(0))
    while Fraction(float(np.nextafter(c, np.float32(np.inf)))) <= q:
        c = np.nextafter(c, np.float32(np.inf))
    up = np.nextafter(c, np.float32(np.inf))
    gap = min(q - Fraction(float(c)), Fraction(float(up)) - q)
    assert q == 0 or c == 0 or gap > q * Fraction(1, 10 ** 140), (d, c)
    return c


def round_binary64(d) -> float:
    """Nearest binary64 of the Decimal d > 0, with a check that d is not near
    a rounding midpoint."""
    q = Fraction(d)
    c = float(d)
    cands = sorted({c, float(np.nextafter(c, np.inf)), float(np.nextafter(c, 0.0))},
                   key=lambda x: abs(Fraction(x) - q))
    best, second = cands[0], cands[1]
    gap = abs(Fraction(second) - q) - abs(Fraction(best) - q)
    assert gap > q * Fraction(1, 10 ** 140), (d, best, second)
    return best


def is_wide(sign: float, m: int) -> bool:
    return sign < 0 and m >= WIDE_FIRST


INF_BITS = 0x7F800000


def table_bits() -> list:
    """32-bit words of the main table (positive gates first), then of the
    wide table."""
    main, wide = [], []
    for sign in (1.0, -1.0):
        for m in range(SPAN):
            sigma = sigma_decimal(sign * bf16_magnitude(m))
            if is_wide(sign, m):
                main += [INF_BITS, INF_BITS]
                v = CLAMP_ENTRY if m == SPAN - 1 else round_binary64(sigma)
                wide += list(struct.unpack("<II", struct.pack("<d", v)))
            else:
                hi = truncate_binary32(sigma)
                lo = round_binary32(Fraction(sigma) - Fraction(float(hi)))
                assert lo >= 0 and hi >= np.float32(2.0 ** -126)
                assert lo == 0 or lo >= np.float32(2.0 ** -126)
                main += [int(np.array(v, np.float32).view(np.uint32)) for v in (hi, lo)]
    assert len(main) == 4 * SPAN and len(wide) == 2 * (SPAN - WIDE_FIRST)
    return main + wide


def render(bits: list) -> str:
    lines = ["// Generated by gen_sigma_table.py: sigma(g) = 1 / (1 + e^-g), two 32-bit words per",
             "// entry. Entries 0..4095: g = +a, 4096..8191: g = -a, a = the BF16 magnitude with bits",
             "// (103 << 7) + index. Gates above -64: binary32 hi = RZ(sigma), lo = RN(sigma - hi);",
             "// entries 7936..8191 (gates <= -64): +inf, +inf. Then 256 binary64 RN64(sigma) for",
             "// those gates, low word first; the last one (g = -255, read for every gate at or",
             "// below it) is 2^-1000. Do not edit.",
             ]
    for i in range(0, len(bits), 8):
        lines.append(" ".join("0x%08xu," % b for b in bits[i:i + 8]))
    return "\n".join(lines) + "\n"


def main() -> None:
    text = render(table_bits())
    with open(OUT, "w") as f:
        f.write(text)
    print(OUT)


if __name__ == "__main__":
    main()
