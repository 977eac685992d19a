"""CPU proof of the division-free quotient used by the GPU quantizer.

The kernels compute RN(a / b) as q0 = RN(a * rb), rem = RN(q0 * b - a) (fma),
q = RN(q0 - rem * rb) (fma), with rb = RN(1 / b). This test runs the same
binary32 sequence on the CPU (IEEE fmaf, no contraction) and compares it with
the correctly rounded division a / b:

* exhaustively for every binary32 numerator mantissa against the 8 E4M3
  mantissas (1 + m/8) as divisors, at three relative exponent offsets - the
  quotient depends only on the mantissas and the exponent difference, so this
  covers every element quotient (and every amax / 6 block-scale quotient)
  when the global scale is a power of two;
* the same exhaustive set with the reciprocal rb moved one ulp down or up
  (a faithful reciprocal such as v_rcp_f32, used when the global scale is a
  power of two): the correction still gives the correctly rounded quotient;
* the sign of zero for +-0 numerators;
* a large random sample of arbitrary divisor mantissas (general global
  scales; every pair of significands is checked on the GPU by
  test_gpu_division_exhaustive.py);
* the remainder criterion that GPU check accepts quotients by, against IEEE
  division: it accepts RN(a / b) and rejects both binary32 neighbours, for
  random pairs and for quotients next to powers of two (where the gap below
  is half the gap above).
"""
import os
import subprocess

import pytest

SRC = r"""
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>
#include <stdlib.h>
static float u2f(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
static uint32_t f2u(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }
static float div_rn(float a, float b, float rb) {
    float q0 = a * rb;
    float rem = fmaf(q0, b, -a);
    return fmaf(rem, -rb, q0);
}
/* the acceptance criterion of the GPU's exhaustive check (divcheck.hip) */
static int correctly_rounded(float a, float b, float q) {
    float r = fmaf(-q, b, a);
    uint32_t qb = f2u(q);
    int e = (int)(qb >> 23) - 127;
    float half_gap = ldexpf(b, e - 24);
    if ((qb & 0x7fffffu) == 0u && r < 0.0f) half_gap *= 0.5f;
    float ar = fabsf(r);
    return ar < half_gap || (ar == half_gap && (qb & 1u) == 0u);
}
int main(int argc, char** argv) {
    long bad = 0, n = 0;
    /* exhaustive: 8 E4M3 mantissas, all numerator mantissas, 3 exponents,
       3 reciprocals */
    for (int m = 0; m < 8; ++m) {
        for (int eb = -1; eb <= 1; ++eb) {
            float b = ldexpf(1.0f + m / 8.0f, eb);
            float r0 = 1.0f / b;
            /* rb = RN(1/b), and its two neighbours (faithful reciprocals) */
            const float rbs[3] = {r0, nextafterf(r0, 0.0f), nextafterf(r0, INFINITY)};
            for (int k = 0; k < 3; ++k) {
                const float rb = rbs[k];
                #pragma omp parallel for reduction(+:bad,n)
                for (uint32_t mx = 0; mx < (1u << 23); ++mx)
                    for (uint32_t ex = 126; ex <= 128; ++ex) {
                        float a = u2f((ex << 23) | mx);
                        float q = div_rn(a, b, rb), r = a / b;
                        float qn = div_rn(-a, b, rb), rn = -a / b;
                        n += 2;
                        bad += (f2u(q) != f2u(r)) + (f2u(qn) != f2u(rn));
                    }
            }
        }
    }
    /* signed zeros */
    float b = 1.25f, rb = 1.0f / b;
    if (f2u(div_rn(0.0f, b, rb)) != f2u(0.0f) || f2u(div_rn(-0.0f, b, rb)) != f2u(-0.0f))
        bad += 1000000;
    /* rb == 0 (zero scale) gives a signed zero */
    if (f2u(div_rn(3.0f, 0.0f, 0.0f)) != f2u(0.0f) || f2u(div_rn(-3.0f, 0.0f, 0.0f)) != f2u(-0.0f))
        bad += 1000000;
    /* random divisor mantissas */
    long rbad = 0, rn_ = 0;
    srand(12345);
    int ndiv = atoi(argv[1]);
    for (int t = 0; t < ndiv; ++t) {
        uint32_t md = ((uint32_t)rand() ^ ((uint32_t)rand() << 15)) & 0x7fffffu;
        float bb = u2f((127u << 23) | md), rbb = 1.0f / bb;
        #pragma omp parallel for reduction(+:rbad,rn_)
        for (uint32_t mx = 0; mx < (1u << 23); mx += 3) {
            float a = u2f((127u << 23) | mx);
            rn_ += 1;
            rbad += f2u(div_rn(a, bb, rbb)) != f2u(a / bb);
        }
    }
    /* the criterion: accepts a / b, rejects its neighbours */
    long cbad = 0, cn = 0;
    srand(777);
    for (long t = 0; t < 20000000; ++t) {
        uint32_t ma = ((uint32_t)rand() ^ ((uint32_t)rand() << 15)) & 0x7fffffu;
        uint32_t mb = ((uint32_t)rand() ^ ((uint32_t)rand() << 15)) & 0x7fffffu;
        if (t % 4 == 0) ma = mb;                         /* quotient exactly 1 */
        if (t % 4 == 1) ma = (mb + (rand() & 7)) & 0x7fffffu;   /* just above or below 1 */
        float a = u2f((127u << 23) | ma), b = u2f((127u << 23) | mb), q = a / b;
        cn += 3;
        cbad += !correctly_rounded(a, b, q);
        cbad += correctly_rounded(a, b, nextafterf(q, INFINITY));
        cbad += correctly_rounded(a, b, nextafterf(q, 0.0f));
    }
    printf("%ld %ld %ld %ld %ld %ld\n", n, bad, rn_, rbad, cn, cbad);
    return 0;
}
"""


@pytest.mark.slow
def test_markstein_quotient_matches_ieee_division(tmp_path):
    c = tmp_path / "divproof.c"
    c.write_text(SRC)
    exe = tmp_path / "divproof"
    subprocess.run(["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
                    "-std=c11", str(c), "-o", str(exe), "-lm"], check=True)
    out = subprocess.run([str(exe), "256"], capture_output=True, text=True, check=True,
                         env={**os.environ, "OMP_NUM_THREADS": str(min(8, os.cpu_count() or 1))})
    n, bad, rn, rbad, cn, cbad = map(int, out.stdout.split())
    assert n == 8 * 3 * 3 * (1 << 23) * 3 * 2
    assert bad == 0, "exhaustive E4M3-mantissa check failed in %d cases" % bad
    assert rn > 0 and rbad == 0, "random-divisor check failed in %d of %d cases" % (rbad, rn)
    assert cn == 60000000 and cbad == 0, "remainder criterion wrong in %d of %d cases" % (cbad, cn)
