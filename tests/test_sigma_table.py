"""The sigmoid table of the fused SwiGLU kernels (csrc/sigma_table.inc): it is
what its generator writes, and its values are sigma(g) = 1 / (1 + e^-g)
correctly rounded to binary32, checked against float64 arithmetic and
against the function's exact properties. CPU only."""
import importlib.util
import os
import struct

import numpy as np

CSRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                    "moe_swiglu_epilogue_amd", "csrc")


def _gen():
    spec = importlib.util.spec_from_file_location("gen_sigma_table",
                                                  os.path.join(CSRC, "gen_sigma_table.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def _table():
    bits = []
    with open(os.path.join(CSRC, "sigma_table.inc")) as f:
        for line in f:
            if line.startswith("0x"):
                bits += [int(t.rstrip("u,"), 16) for t in line.split()]
    return np.array(bits, np.uint32)


def _gates():
    a = ((((103 << 7) + np.arange(4096)).astype(np.uint32)) << 16).view(np.float32)
    a = a.astype(np.float64)
    return np.concatenate([a, -a])


def test_committed_table_is_the_generators_output():
    gen = _gen()
    with open(os.path.join(CSRC, "sigma_table.inc")) as f:
        assert f.read() == gen.render(gen.table_bits())


def test_table_against_float64():
    """Within 1 ulp of the float64 sigmoid everywhere, and equal to its
    rounding wherever the float64 value lies clear of a binary32 midpoint
    (float64's own error is below 1e-15 relative)."""
    t = _table()
    assert t.size == 8192
    g = _gates()
    with np.errstate(over="ignore"):
        s64 = 1.0 / (1.0 + np.exp(-g))
    ref = s64.astype(np.float32)
    tf = t.view(np.float32)
    d = t.view(np.int32).astype(np.int64) - ref.view(np.int32).astype(np.int64)
    assert np.abs(d).max() <= 1
    # distance of the float64 value from the nearest binary32 midpoint
    lo = np.where(ref.astype(np.float64) <= s64, ref, np.nextafter(ref, np.float32(0)))
    hi = np.nextafter(lo, np.float32(np.inf))
    mid = (lo.astype(np.float64) + hi.astype(np.float64)) / 2
    clear = np.abs(s64 - mid) > 1e-14 * s64
    # the rest (256) are small gates, where sigma = 1/2 + g/4 - g^3/48 + ...
    # sits next to a midpoint by construction; the 1-ulp bound covers them
    assert clear.sum() >= 7900
    assert np.array_equal(tf[clear], ref[clear])


def test_table_exact_properties():
    tf = _table().view(np.float32).astype(np.float64)
    pos, neg = tf[:4096], tf[4096:]
    # the smallest magnitude, 2^-24: sigma = 1/2 +- 2^-26 rounds to 1/2 on both sides
    assert pos[0] == 0.5 and neg[0] == 0.5
    # monotone: increasing in g
    assert np.all(np.diff(pos) >= 0) and np.all(np.diff(neg) <= 0)
    assert np.all(pos >= 0.5) and np.all(neg <= 0.5) and np.all(neg >= 0)
    # sigma(g) + sigma(-g) = 1, up to the two roundings
    ulp = np.spacing(pos.astype(np.float32)).astype(np.float64)
    assert np.all(np.abs(pos + neg - 1.0) <= ulp)
    # the largest magnitudes: sigma(+255) rounds to 1, sigma(-255) (about 1.8e-111) to 0
    assert pos[-1] == 1.0 and neg[-1] == 0.0
    # subnormal binary32 results for g in (-103.3, -87.3), zero below
    g = _gates()[4096:]
    sub = neg[(neg > 0) & (neg < 2.0 ** -126)]
    assert sub.size > 0
    assert np.all(neg[g < -104.0] == 0.0)
    # sigma(1) = 1 / (1 + 1/e): 0.7310585786300049 -> binary32 0x3f3b26a8
    one = (127 - 103) * 128
    assert struct.pack("<f", np.float32(pos[one])) == struct.pack("<I", 0x3f3b26a8)


def _nearest_binary32(q):
    """The binary32 nearest to the rational q (> 0), and the distance from q
    to the nearest binary32 midpoint."""
    from fractions import Fraction
    c = np.float32(float(q))
    cands = [c, np.nextafter(c, np.float32(np.inf)), np.nextafter(c, np.float32(0))]
    best = min(cands, key=lambda x: abs(Fraction(float(x)) - q))
    mids = [(Fraction(float(best)) + Fraction(float(n))) / 2
            for n in (np.nextafter(best, np.float32(np.inf)), np.nextafter(best, np.float32(0)))]
    return best, min(abs(q - m) for m in mids)


def test_small_gates_exact_by_series():
    """For |g| <= 2^-6, sigma(g) = 1/2 + tanh(g/2)/2 = 1/2 + g/4 - g^3/48
    + g^5/480 - 17 g^7/80640 + 31 g^9/1451520 - ..., an alternating series
    whose remainder is below 2.2e-6 |g|^11. Summed exactly in rationals, it
    fixes the correctly rounded binary32 of every such entry (including the
    ones next to a midpoint, where float64 cannot decide), independently of
    the generator's decimal arithmetic."""
    from fractions import Fraction
    t = _table().view(np.float32)
    g = _gates()
    coef = [(1, Fraction(1, 4)), (3, Fraction(-1, 48)), (5, Fraction(1, 480)),
            (7, Fraction(-17, 80640)), (9, Fraction(31, 1451520))]
    checked = 0
    for i in np.nonzero(np.abs(g) <= 2.0 ** -6)[0]:
        x = Fraction(float(g[i]))
        q = Fraction(1, 2) + sum(c * x ** k for k, c in coef)
        bound = Fraction(22, 10 ** 7) * abs(x) ** 11
        best, margin = _nearest_binary32(q)
        assert margin > bound, i                      # the series decides the rounding
        assert t[i] == best, (i, float(g[i]), t[i], best)
        checked += 1
    assert checked == 2 * (18 * 128 + 1)   # exponents 103..120 and 2^-6, both signs
