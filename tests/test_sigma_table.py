"""The sigmoid table of the fused SwiGLU kernels (csrc/sigma_table.inc): it is
what its generator writes; each main entry for a gate above -64 is the pair
hi = RZ(sigma) (toward zero), lo = RN(sigma - hi) >= 0 of normal binary32
values for sigma(g) = 1 / (1 + e^-g), each main entry for a gate at or below
-64 is the marker (+inf, +inf), and the wide table after the main one holds
RN64(sigma) for those gates (the last, read for gates at or below -255,
2^-1000).
Checked against float64 arithmetic, against the exact Taylor series of the
sigmoid near 0, against an exact-rational series for e^g at the binary64
entries, and against the sigmoid's exact properties. CPU only."""
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


WIDE = 8192 - 256          # first binary64 entry: the gate -64


def _words():
    bits = []
    with open(os.path.join(CSRC, "sigma_table.inc")) as f:
        for line in f:
            if line.startswith("0x"):
                bits += [int(t.rstrip("u,"), 16) for t in line.split()]
    w = np.array(bits, np.uint32)
    assert w.size == 2 * 8192 + 2 * 256
    return w


def _table():
    """(hi, lo) float32 arrays of the 7936 pair entries: g > 0 (0..4095), then
    g < 0 down to the gate -63.75 (4096..7935)."""
    t = _words().view(np.float32)
    return t[0::2][:WIDE], t[1::2][:WIDE]


def _wide():
    """The wide table: 256 binary64 entries, gates -64 .. -255."""
    return _words()[2 * 8192:].view(np.float64)


def test_marked_entries():
    """The main entries of the gates -64 .. -255 are (+inf, +inf)."""
    w = _words()[2 * WIDE:2 * 8192]
    assert np.all(w == 0x7F800000)


def _gates(n=WIDE):
    a = ((((103 << 7) + np.arange(4096)).astype(np.uint32)) << 16).view(np.float32)
    a = a.astype(np.float64)
    return np.concatenate([a, -a])[:n]


def _nearest_binary32(q):
    """The binary32 nearest to the rational q, and the distance from q to the
    nearest binary32 rounding midpoint."""
    if q < 0:
        b, m = _nearest_binary32(-q)
        return -b, m
    c = np.float32(float(q))
    cands = [c, np.nextafter(c, np.float32(np.inf)), np.nextafter(c, np.float32(0))]
    best = min(cands, key=lambda x: abs(Fraction(float(x)) - q))
    mids = [(Fraction(float(best)) + Fraction(float(n))) / 2
            for n in (np.nextafter(best, np.float32(np.inf)), np.nextafter(best, np.float32(0)))]
    return best, min(abs(q - m) for m in mids)


def _truncate_binary32(q):
    """The largest binary32 not above the rational q >= 0, and the distance
    from q to the nearest binary32 value."""
    c = np.float32(float(q))
    while Fraction(float(c)) > q:
        c = np.nextafter(c, np.float32(0))
    while Fraction(float(np.nextafter(c, np.float32(np.inf)))) <= q:
        c = np.nextafter(c, np.float32(np.inf))
    up = np.nextafter(c, np.float32(np.inf))
    return c, min(q - Fraction(float(c)), Fraction(float(up)) - q)


def test_committed_table_is_the_generators_output():
    gen = _gen()
    with open(os.path.join(CSRC, "sigma_table.inc")) as f:
        assert f.read() == gen.render(gen.table_bits())


def test_table_against_float64():
    """hi is the float64 sigmoid truncated to binary32 wherever the float64
    value lies clear of a binary32 value (float64's own error is below 1e-15
    relative), and within 1 ulp of it everywhere; hi + lo agrees with the
    float64 value to within 2^-47."""
    hi, lo = _table()
    g = _gates()
    s64 = 1.0 / (1.0 + np.exp(-g))
    near = s64.astype(np.float32)
    below = np.where(near.astype(np.float64) <= s64, near, np.nextafter(near, np.float32(0)))
    above = np.nextafter(below, np.float32(np.inf))
    d = hi.view(np.int32).astype(np.int64) - below.view(np.int32).astype(np.int64)
    assert np.abs(d).max() <= 1
    clear = (np.minimum(s64 - below.astype(np.float64), above.astype(np.float64) - s64)
             > 1e-14 * s64)
    # the rest are small gates, where sigma = 1/2 + g/4 - g^3/48 + ... sits
    # next to a binary32 value by construction (the series test pins them),
    # and gates above about 33, where sigma is within 1e-14 of 1 (pinned below)
    assert clear.sum() >= 6900
    assert np.array_equal(hi[clear], below[clear])
    # the pair: |hi + lo - sigma| <= 2^-48 sigma (lo rounded to 24 bits, lo
    # below 2^-23 sigma) plus float64's error; both halves normal
    pair = hi.astype(np.float64) + lo.astype(np.float64)
    assert np.all(np.abs(pair - s64) <= 2.0 ** -47 * s64)
    assert np.all(hi >= np.float32(2.0 ** -126)) and np.all((lo == 0) | (lo >= np.float32(2.0 ** -126)))
    # lo is the remainder: non-negative and below one ulp of hi
    assert np.all(lo >= 0) and not np.any(np.signbit(lo))
    assert np.all(lo.astype(np.float64) <= np.spacing(hi).astype(np.float64))


def test_small_gates_exact_by_series():
    """For |g| <= 2^-6, sigma(g) = 1/2 + tanh(g/2)/2 = 1/2 + g/4 - g^3/48
    + g^5/480 - 17 g^7/80640 + 31 g^9/1451520 - ..., an alternating series
    whose remainder is below 2.2e-6 |g|^11. Summed exactly in rationals, it
    fixes both halves of every such entry (including the hi values next to a
    midpoint, where float64 cannot decide), independently of the
    generator's decimal arithmetic."""
    hi, lo = _table()
    g = _gates()
    coef = [(1, Fraction(1, 4)), (3, Fraction(-1, 48)), (5, Fraction(1, 480)),
            (7, Fraction(-17, 80640)), (9, Fraction(31, 1451520))]
    checked = 0
    for i in np.nonzero(np.abs(g) <= 2.0 ** -6)[0]:
        x = Fraction(float(g[i]))
        q = Fraction(1, 2) + sum(c * x ** k for k, c in coef)
        bound = Fraction(22, 10 ** 7) * abs(x) ** 11
        want_hi, margin = _truncate_binary32(q)
        assert margin > bound, i                      # the series decides the truncation
        assert hi[i] == want_hi, (i, float(g[i]), hi[i], want_hi)
        want_lo, margin = _nearest_binary32(q - Fraction(float(want_hi)))
        assert margin > bound, i
        assert lo[i] == want_lo, (i, float(g[i]), lo[i], want_lo)
        checked += 1
    assert checked == 2 * (18 * 128 + 1)   # exponents 103..120 and 2^-6, both signs


def test_table_exact_properties():
    hi, lo = _table()
    h = hi.astype(np.float64)
    pos, neg = h[:4096], h[4096:]
    # the smallest magnitude, 2^-24: sigma = 1/2 +- 2^-26 + O(2^-75) truncates
    # to 1/2 and to 1/2 - 2^-25, and lo carries the 2^-26 on both sides
    assert pos[0] == 0.5 and neg[0] == 0.5 - 2.0 ** -25
    assert lo[0] == np.float32(2.0 ** -26) and lo[4096] == np.float32(2.0 ** -26)
    # monotone: increasing in g
    assert np.all(np.diff(pos) >= 0) and np.all(np.diff(neg) <= 0)
    assert np.all(pos >= 0.5) and np.all(neg < 0.5) and np.all(neg >= 0)
    # sigma(g) + sigma(-g) = 1: to the pairs' accuracy, in exact arithmetic
    for i in range(0, WIDE - 4096, 37):
        s = (Fraction(float(hi[i])) + Fraction(float(lo[i])) + Fraction(float(hi[4096 + i]))
             + Fraction(float(lo[4096 + i])))
        assert abs(s - 1) <= Fraction(1, 2 ** 46), i
    # the largest magnitude: sigma(+255) = 1 - 1.8e-111 is 1 - 2^-24 plus lo =
    # 2^-24
    assert pos[-1] == 1.0 - 2.0 ** -24 and lo[4095] == np.float32(2.0 ** -24)
    # sigma(1) = 1 / (1 + 1/e) = 0.7310585786300049, between the binary32
    # values 0x3f3b26a7 and 0x3f3b26a8: truncated, 0x3f3b26a7
    one = (127 - 103) * 128
    assert struct.pack("<f", np.float32(pos[one])) == struct.pack("<I", 0x3f3b26a7)
    # the pair entries end at the gate -63.75 (BF16 0xC27F), the binary64 ones
    # start at -64 (0xC280)
    a = ((((103 << 7) + np.arange(4096)).astype(np.uint32)) << 16).view(np.float32)
    assert a[WIDE - 4096 - 1] == np.float32(63.75) and a[WIDE - 4096] == np.float32(64.0)


def _exp_neg(x: Fraction, terms: int = 400):
    """e^-x for 0 <= x <= 256 as an exact rational with an error bound:
    e^-x = (e^-(x/2^k))^(2^k), the inner value by its alternating Taylor
    series (remainder below the first omitted term), then squared k times
    (the relative error grows by at most a factor 2^k * (1 + err))."""
    k = 9
    y = x / 2 ** k                         # at most 1/2
    s, t = Fraction(0), Fraction(1)
    for n in range(1, 40):
        s += t
        t = t * (-y) / n
    rel = abs(t) / s * 2                   # relative bound of the truncated series
    for _ in range(k):
        s = s * s
        rel = 2 * rel + rel * rel
    return s, rel


def test_wide_entries_exact():
    """The binary64 entries (gates -64 .. -254.x) are the binary64 values
    nearest to sigma(g) = e^g / (1 + e^g), computed here from an
    exact-rational series for e^-|g| (independent of the generator's decimal
    arithmetic) wherever its error bound decides the rounding; the last entry
    is 2^-1000."""
    wide = _wide()
    gates = -_gates(8192)[WIDE:]
    assert gates[0] == 64.0 and gates[-1] == 255.0
    assert wide[-1] == 2.0 ** -1000
    decided = 0
    for i in range(0, 255, 3):
        e, rel = _exp_neg(Fraction(float(gates[i])))
        sig = e / (1 + e)                   # sigma(-|g|)
        got = Fraction(float(wide[i]))
        ulp = Fraction(float(np.spacing(wide[i])))
        # the entry is within half an ulp of sigma, up to the series' error
        assert abs(got - sig) <= ulp / 2 + 2 * rel * sig, (i, float(gates[i]))
        if abs(abs(got - sig) - ulp / 2) > 2 * rel * sig:
            assert abs(got - sig) < ulp / 2, (i, float(gates[i]))
            decided += 1
    assert decided >= 80
    # against float64: sigma(-x) = exp(-x) / (1 + exp(-x)) within 4 ulp
    f64 = np.exp(-gates[:-1]) / (1.0 + np.exp(-gates[:-1]))
    assert np.all(np.abs(wide[:-1] - f64) <= 4 * np.spacing(f64))
    assert np.all(np.diff(wide[:-1]) < 0) and np.all(wide > 0)


def test_large_gates():
    """For g >= 18, 1 - sigma(g) = e^-g / (1 + e^-g) < 2^-25, so sigma
    truncates to 1 - 2^-24 and lo = RN(2^-24 - e^-g / (1 + e^-g)), which
    float64 fixes (its error is below 1e-23 absolute, far inside lo's
    rounding steps of at least 2^-48 here); above g = 40, lo = 2^-24."""
    hi, lo = _table()
    g = _gates()[:4096]
    big = g >= 18.0
    assert np.all(hi[:4096][big] == np.float32(1.0 - 2.0 ** -24))
    t = np.exp(-g[big])
    want = (2.0 ** -24 - t / (1.0 + t)).astype(np.float32)
    assert np.array_equal(lo[:4096][big], want)
    assert np.all(lo[:4096][g > 40.0] == np.float32(2.0 ** -24))
