"""Exhaustive check, on the GPU, of the quotient sequence the quantizer uses
for divisions by a general global scale's block divisors (nvfp4_device.hpp
div_rn with a correctly rounded reciprocal): every pair of binary32
significands (2^46 pairs; libnvfp4_divcheck.so, include/nvfp4_divcheck.h).
The quotient of two normal numbers through that sequence depends only on
their significands while the intermediates stay in the normal range, which
the quantizer's global-scale range [2^-64, 2^64] guarantees, so this covers
every quotient the general-scale path computes. The acceptance criterion
(the exact remainder against half the gap between binary32 neighbours) is
checked against IEEE division on the CPU in test_division_proof.py, and a
run on the uncorrected first quotient shows that it rejects wrong
quotients here too."""
import ctypes as C
import time

import pytest
import torch

from moe_swiglu_epilogue_amd import build as B

pytestmark = pytest.mark.gpu

SIG = 1 << 23
CHUNK = 1 << 16


def say(*a):
    print("[gpu]", *a, flush=True)


@pytest.fixture(scope="module")
def lib():
    assert torch.cuda.is_available(), "this test needs the GPU"
    L = C.CDLL(B.DIVCHECK_LIB)
    L.nvfp4_divcheck.argtypes = [C.c_uint32, C.c_uint32, C.c_int, C.c_void_p, C.c_void_p,
                                 C.c_void_p]
    L.nvfp4_divcheck.restype = C.c_int
    return L


def _run(L, first, count, naive, fails, witness):
    st = torch.cuda.current_stream().cuda_stream
    assert L.nvfp4_divcheck(first, count, naive, fails.data_ptr(), witness.data_ptr(), st) == 0


def _decode(w):
    w &= (1 << 64) - 1
    return (w >> 23, w & (SIG - 1))


def test_check_rejects_uncorrected_quotients(lib):
    """The first quotient RN(a RN(1/b)) alone is wrong for some pairs: the
    check must find them (and so is able to fail)."""
    fails = torch.zeros(1, dtype=torch.int64, device="cuda")
    witness = torch.full((1,), -1, dtype=torch.int64, device="cuda")
    _run(lib, SIG - 4096, 4096, 1, fails, witness)
    n = int(fails.item())
    say("uncorrected first quotient: %d of %d pairs wrong" % (n, 4096 * SIG))
    assert n > 0 and int(witness.item()) != -1


def test_div_rn_every_significand_pair(lib):
    fails = torch.zeros(1, dtype=torch.int64, device="cuda")
    witness = torch.full((1,), -1, dtype=torch.int64, device="cuda")
    t0 = time.time()
    for k, first in enumerate(range(0, SIG, CHUNK)):
        _run(lib, first, CHUNK, 0, fails, witness)
        if k % 16 == 15:
            torch.cuda.synchronize()
            say("divisor significands %d / %d done, %.1f s, failures %d"
                % (first + CHUNK, SIG, time.time() - t0, int(fails.item())))
    torch.cuda.synchronize()
    n = int(fails.item())
    w = int(witness.item())
    assert n == 0, "div_rn not correctly rounded for %d pairs; first (m_b, m_a) = %s" % (
        n, _decode(w))
    assert w == -1
