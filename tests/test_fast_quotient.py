"""CPU proof of the guarded fast element quotient of the GPU quantizer.

The element step of the method is h = rint(RN(x / (d/2))) (the signed
half-step count; ties to even). The kernels first try q0 = RN(x * rcp), with
rcp = v_rcp_f32(d/2), within one ulp of 2/d, and take h = rint(q0) for a
whole block when every |q0 - rint(q0)| of it is below 0.5 - 2^-17;
otherwise the block takes the exact quotient. This test runs both in binary32 on the CPU
(IEEE division, no contraction) and checks, wherever the guard accepts q0:

* |h_exact| <= 14: rint(q0) == h_exact, bit for bit (the sign of zero
  included);
* otherwise both counts are at least 12 in magnitude with the same sign (the
  E2M1 convert saturates every such count to the same code);

exhaustively over every numerator significand in the 8 binades with
quotients in [2^-3, 32) (and the negated values), for the 8 E4M3 divisor
significands, and on a sample of numerators for random divisor significands
(general global scales), each with the reciprocal RN(1/b) and both of its
neighbours (every value a one-ulp reciprocal can take). It also
checks that exact ties (quotients on a half-integer) are always sent to the
exact path, that tiny, zero and large numerators behave, and reports how
often the guard rejects a value.
"""
import os
import subprocess

import pytest

SRC = r"""
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>
static float u2f(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
static uint32_t f2u(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }
static const float kGuard = 0.5f - 0x1p-17f;
/* 1 when the guard accepts and the fast count is wrong; *rej counts rejects */
static int check(float x, float hd, float rcp, long* rej) {
    const float q0 = x * rcp;
    const float h = rintf(q0);
    const float far = fabsf(q0 - h);
    const float he = rintf(x / hd);
    if (!(far < kGuard)) { ++*rej; return 0; }
    if (fabsf(he) <= 14.0f) return f2u(h) != f2u(he);
    return !(fabsf(h) >= 12.0f && fabsf(he) >= 12.0f && signbit(h) == signbit(he));
}
int main(int argc, char** argv) {
    long bad = 0, n = 0, rej = 0;
    /* E4M3 significands, three reciprocals each, numerators with quotients
       in [2^-3, 32) and their negatives */
    for (int m = 0; m < 8; ++m) {
        const float hd = 1.0f + m / 8.0f;
        const float r0 = 1.0f / hd;
        const float rcps[3] = {r0, nextafterf(r0, 0.0f), nextafterf(r0, INFINITY)};
        for (int k = 0; k < 3; ++k) {
            const float rcp = rcps[k];
            #pragma omp parallel for reduction(+:bad,n,rej) schedule(static)
            for (uint32_t mx = 0; mx < (1u << 23); ++mx)
                for (int e = -3; e <= 4; ++e) {
                    const float x = ldexpf(u2f((127u << 23) | mx), e);
                    bad += check(x, hd, rcp, &rej) + check(-x, hd, rcp, &rej);
                    n += 2;
                }
        }
    }
    /* exact ties: x = (j + 1/2) hd for half-integers up to 12, all E4M3
       significands, reciprocal RN(1/hd) and neighbours: always rejected */
    long tie_ok = 0, ties = 0;
    for (int m = 0; m < 8; ++m)
        for (int j = 0; j < 24; ++j) {
            const float hd = 1.0f + m / 8.0f, x = (j + 0.5f) * hd;
            if ((double)x != ((double)j + 0.5) * (double)hd) continue;
            const float r0 = 1.0f / hd;
            const float rcps[3] = {r0, nextafterf(r0, 0.0f), nextafterf(r0, INFINITY)};
            for (int k = 0; k < 3; ++k) {
                long r = 0;
                bad += check(x, hd, rcps[k], &r);
                tie_ok += r; ++ties;
            }
        }
    /* tiny, zero and huge numerators (E4M3 significands, exact reciprocal) */
    for (int m = 0; m < 8; ++m) {
        const float hd = 1.0f + m / 8.0f, rcp = 1.0f / hd;
        const float xs[8] = {0.0f, -0.0f, 0x1p-149f, -0x1p-149f, 0x1p-127f, 0x1.8p-20f,
                             0x1p100f, -0x1.7p120f};
        for (int i = 0; i < 8; ++i) { long r = 0; bad += check(xs[i], hd, rcp, &r); ++n; }
    }
    /* random divisor significands, RN(1/b) and both neighbours, every 5th
       numerator significand */
    srand(4242);
    const int ndiv = atoi(argv[1]);
    for (int t = 0; t < ndiv; ++t) {
        const uint32_t md = ((uint32_t)rand() ^ ((uint32_t)rand() << 15)) & 0x7fffffu;
        const float hd = u2f((127u << 23) | md), r0 = 1.0f / hd;
        const float rcps[3] = {r0, nextafterf(r0, 0.0f), nextafterf(r0, INFINITY)};
        for (int k = 0; k < 3; ++k) {
            const float rcp = rcps[k];
            #pragma omp parallel for reduction(+:bad,n,rej) schedule(static)
            for (uint32_t mx = 0; mx < (1u << 23); mx += 5)
                for (int e = -3; e <= 4; ++e) {
                    const float x = ldexpf(u2f((127u << 23) | mx), e);
                    bad += check(x, hd, rcp, &rej) + check(-x, hd, rcp, &rej);
                    n += 2;
                }
        }
    }
    printf("%ld %ld %ld %ld %ld\n", n, bad, rej, ties, tie_ok);
    return 0;
}
"""


@pytest.mark.slow
def test_guarded_fast_quotient_gives_the_exact_counts(tmp_path):
    c = tmp_path / "fastq.c"
    c.write_text(SRC)
    exe = tmp_path / "fastq"
    subprocess.run(["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
                    "-std=c11", str(c), "-o", str(exe), "-lm"], check=True)
    out = subprocess.run([str(exe), "32"], capture_output=True, text=True, check=True,
                         env={**os.environ, "OMP_NUM_THREADS": str(min(8, os.cpu_count() or 1))})
    n, bad, rej, ties, tie_ok = map(int, out.stdout.split())
    exhaustive = 8 * 3 * (1 << 23) * 8 * 2
    sampled = 32 * 3 * (((1 << 23) + 4) // 5) * 8 * 2
    assert n == exhaustive + 8 * 8 + sampled
    assert bad == 0, "fast count accepted but wrong in %d of %d cases" % (bad, n)
    # every exact tie is sent to the exact path
    assert ties > 100 and tie_ok == ties
    # the guard rejects few values: about 2^-16 of uniformly spread quotients
    # (plus the exact ties on the half-integer grid of the E4M3 divisors)
    assert 0 < rej < n * 1e-3
