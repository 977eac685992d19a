"""The sigmoid table of the fused SwiGLU kernels (csrc/sigma_table.inc): it is
what its generator writes, and each entry is RN64(sigma(g)), the binary64
value nearest to sigma(g) = 1 / (1 + e^-g), for the BF16 gates with exponent
field 103..134 (positive gates first), except the last negative one (the gate
-255, read for every gate at or below it), which holds 2^-1000.
Checked against float64 arithmetic, against the exact Taylor series of the
sigmoid near 0, against an exact-rational series for e^-|g| across the whole
range, and against the sigmoid's exact properties. CPU only."""
import importlib.util
import os
import struct
from fractions import Fraction

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
    """The 8192 binary64 entries: g > 0 (0..4095), then g < 0."""
    bits = []
    with open(os.path.join(CSRC, "sigma_table.inc")) as f:
        for line in f:
            if line.startswith("0x"):
                bits += [int(t.rstrip("u,"), 16) for t in line.split()]
    w = np.array(bits, np.uint32)
    assert w.size == 2 * 8192
    return w.view(np.float64)


def _gates():
    a = ((((103 << 7) + np.arange(4096)).astype(np.uint32)) << 16).view(np.float32)
    a = a.astype(np.float64)
    return np.concatenate([a, -a])


def _nearest_binary64(q):
    """The binary64 nearest to the rational q > 0, and the distance from q to
    the nearest binary64 rounding midpoint."""
    c = float(q)
    cands = [c, np.nextafter(c, np.inf), np.nextafter(c, 0.0)]
    best = min(cands, key=lambda x: abs(Fraction(float(x)) - q))
    mids = [(Fraction(float(best)) + Fraction(float(n))) / 2
            for n in (np.nextafter(best, np.inf), np.nextafter(best, 0.0))]
    return float(best), min(abs(q - m) for m in mids)


FIX = 600                                  # fixed-point fraction bits of _exp_neg


def _exp_neg(x: Fraction):
    """e^-x for 0 <= x <= 256 as an exact rational with a relative error
    bound: e^-x = (e^-(x/2^k))^(2^k), the inner value by its alternating
    Taylor series, then squared k times, all in integers scaled by 2^FIX
    (every product truncated, so each step adds at most one unit of 2^-FIX;
    the truncated series' remainder is below its first omitted term, and a
    squaring doubles the relative error and adds one unit relative to the
    result, which stays above e^-256 > 2^-370)."""
    k = 9
    y = x / 2 ** k                         # at most 1/2, a dyadic rational
    one = 1 << FIX
    s, t, n_terms = 0, one, 40
    for n in range(1, n_terms + 1):
        s += t
        t = -(abs(t) * y.numerator // (y.denominator * n)) if t > 0 else \
            abs(t) * y.numerator // (y.denominator * n)
    # |error| <= n_terms units (truncations) + |t| (the remainder) + 1; the
    # bound is carried as a float rounded up generously (it stays near 2^-220)
    rel = (n_terms + abs(t) + 1) / s * 1.01
    unit_rel = 2.0 ** (370 - FIX)              # one unit relative to any value >= 2^-370
    for _ in range(k):
        s = s * s >> FIX
        rel = (2 * rel + rel * rel + unit_rel) * 1.01
    return Fraction(s, one), Fraction(rel)


def test_committed_table_is_the_generators_output():
    gen = _gen()
    with open(os.path.join(CSRC, "sigma_table.inc")) as f:
        assert f.read() == gen.render(gen.table_bits())


def test_table_against_float64():
    """Every entry (the clamp entry aside) is within 4 ulp of the float64
    evaluation 1 / (1 + exp(-g)) (for g < 0: e^g / (1 + e^g), which keeps
    float64's relative accuracy down to the gate -255), and all are normal
    binary64 numbers."""
    t, g = _table(), _gates()
    e = np.exp(-np.abs(g))
    f64 = np.where(g > 0, 1.0 / (1.0 + e), e / (1.0 + e))
    body = np.ones(8192, bool)
    body[-1] = False
    assert np.all(np.abs(t[body] - f64[body]) <= 4 * np.spacing(f64[body]))
    assert np.all(t >= np.finfo(np.float64).tiny)


def test_small_gates_exact_by_series():
    """For |g| <= 2^-6, sigma(g) = 1/2 + tanh(g/2)/2 = 1/2 + g/4 - g^3/48
    + g^5/480 - 17 g^7/80640 + 31 g^9/1451520 - ..., an alternating series
    whose remainder is below 2.2e-6 |g|^11. Summed exactly in rationals, it
    fixes every such entry as the nearest binary64, independently of the
    generator's decimal arithmetic."""
    t, g = _table(), _gates()
    coef = [(1, Fraction(1, 4)), (3, Fraction(-1, 48)), (5, Fraction(1, 480)),
            (7, Fraction(-17, 80640)), (9, Fraction(31, 1451520))]
    checked = 0
    for i in np.nonzero(np.abs(g) <= 2.0 ** -6)[0]:
        x = Fraction(float(g[i]))
        q = Fraction(1, 2) + sum(c * x ** k for k, c in coef)
        bound = Fraction(22, 10 ** 7) * abs(x) ** 11
        want, margin = _nearest_binary64(q)
        assert margin > bound, i                      # the series decides the rounding
        assert t[i] == want, (i, float(g[i]), t[i], want)
        checked += 1
    assert checked == 2 * (18 * 128 + 1)   # exponents 103..120 and 2^-6, both signs


def test_entries_exact_by_exp_series():
    """Across the whole range (every 7th gate of each sign, and all gates at
    or below -64), each entry is the binary64 nearest to sigma, with e^-|g|
    from an exact-rational series: sigma(g) = 1 / (1 + e^-g) for g > 0 and
    e^-|g| / (1 + e^-|g|) for g < 0. Where the series' error bound cannot
    decide the rounding, the entry is still within half an ulp plus that
    bound."""
    t, g = _table(), _gates()
    idx = sorted(set(range(0, 8192 - 1, 7)) | set(range(8192 - 256, 8192 - 1)))
    decided = total = 0
    for i in idx:
        if abs(g[i]) <= 2.0 ** -6:
            continue                                   # the Taylor test above covers these
        total += 1
        e, rel = _exp_neg(Fraction(float(abs(g[i]))))
        sig = 1 / (1 + e) if g[i] > 0 else e / (1 + e)
        err = 2 * rel * sig                            # bound on |sig - sigma|
        got = Fraction(float(t[i]))
        ulp = Fraction(float(np.spacing(t[i])))
        assert abs(got - sig) <= ulp / 2 + err, (i, float(g[i]))
        want, margin = _nearest_binary64(sig)
        if margin > err:
            assert t[i] == want, (i, float(g[i]))
            decided += 1
    assert decided >= 0.99 * total


def test_table_exact_properties():
    t = _table()
    pos, neg = t[:4096], t[4096:]
    # the smallest magnitude, 2^-24: sigma = 1/2 +- 2^-26 + O(2^-77) rounds
    # to 1/2 +- 2^-26 exactly
    assert pos[0] == 0.5 + 2.0 ** -26 and neg[0] == 0.5 - 2.0 ** -26
    # monotone: increasing in g, within sigma's range
    assert np.all(np.diff(pos) >= 0) and np.all(np.diff(neg) < 0)
    assert np.all(pos > 0.5) and np.all(pos <= 1.0) and np.all(neg < 0.5) and np.all(neg > 0)
    # sigma(g) + sigma(-g) = 1: each entry within half an ulp (at most 2^-54
    # for entries in [1/4, 1]; less below), so the exact sum is within 2^-52
    # of 1
    for i in range(0, 4095, 13):
        s = Fraction(float(pos[i])) + Fraction(float(neg[i]))
        assert abs(s - 1) <= Fraction(1, 2 ** 52), i
    # sigma(1) = 1 / (1 + 1/e) = 0.73105857863000487925...: the nearest
    # binary64 prints as 0.7310585786300049
    one = (127 - 103) * 128
    assert repr(float(pos[one])) == "0.7310585786300049"
    # large gates: 1 - sigma(g) is below 2^-54 (half an ulp below 1) once
    # e^-g < 2^-54, i.e. g > 37.43: those entries are 1.0; up to g = 36.5
    # they are not
    g = _gates()[:4096]
    assert np.all(pos[g >= 37.5] == 1.0) and np.all(pos[g <= 36.5] < 1.0)
    # the clamp entry (the gate -255 and every gate below it) is 2^-1000;
    # the entry before it, sigma(-254) ~ 2^-366.4, is normal and larger
    assert neg[-1] == 2.0 ** -1000 and neg[-2] > 2.0 ** -370
    assert struct.pack("<d", neg[-1]) == struct.pack("<Q", (1023 - 1000) << 52)
