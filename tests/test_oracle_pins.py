"""Pins of the CPU oracle to things other than itself.

* the worked facts the pages print (tests/golden/page_facts.txt);
* PyTorch's float8_e4m3fn cast and decode (a library routine), exhaustively
  over every binary32 in [0, 448] and all 256 codes;
* the OCP E2M1 format definition (bias-1 exponent, 1 mantissa bit);
* PyTorch's float64 SiLU for the SwiGLU step, plus closed forms;
* an exact-rational restatement (tests/exact_twin.py) on small inputs,
  including every injected edge block of the standalone workload;
* invariants that follow from the definitions.

The ``pin_*`` functions are also run by test_oracle_mutants.py against
deliberately broken copies of the oracle, to show they catch such mistakes.
"""
import math
import os

import numpy as np
import pytest
import torch

import exact_twin as twin
import oracle
from moe_swiglu_epilogue_amd import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "page_facts.txt")


def _num(s):
    s = s.strip()
    if s == "nan":
        return float("nan")
    return int(s, 16) if s.startswith("0x") else float(s)


def _facts():
    out = []
    with open(GOLDEN) as f:
        for line in f:
            line = line.split("#", 1)[0] if line.startswith("#") else line
            if not line.strip():
                continue
            body, _, cite = line.partition("|")
            kind, a, b = body.split()
            out.append((kind, _num(a), _num(b), cite.strip()))
    return out


def _block_with(value, amax=6.0):
    x = np.zeros(16, np.float32)
    x[0] = amax
    x[1] = value
    return x


# ---- pin functions (each raises AssertionError on a mismatch) ---------------
def pin_page_facts():
    for kind, a, b, cite in _facts():
        if kind == "fp8_encode":
            got = oracle.fp8_encode_scalar(a)
            assert got == b, (kind, a, hex(got), cite)
        elif kind == "fp8_decode":
            got = oracle.fp8_decode(int(a))
            if math.isnan(b):
                assert math.isnan(got), (kind, a, got, cite)
            else:
                # the pages print 6 significant digits
                assert abs(got - b) <= 5e-7 * max(1.0, abs(b)), (kind, a, got, cite)
        elif kind == "e2m1_nibble":
            packed, sf, _, _ = oracle.quantize_block(_block_with(a))
            assert sf == 0x38, "amax 6 must give scale 1.0"
            assert packed[0] >> 4 == b, (kind, a, packed[0] >> 4, cite)
        elif kind == "e2m1_nibble_half_up":
            hs = int(math.floor(2 * a + 0.5))
            assert oracle.e2m1_index(hs) == b, (kind, a, cite)
            packed, _, _, _ = oracle.quantize_block(_block_with(a))
            assert packed[0] >> 4 != b, "oracle must not round half up"
        elif kind == "e2m1_index":
            assert oracle.e2m1_index(int(a)) == b, (kind, a, cite)
        else:
            raise AssertionError("unknown fact kind " + kind)


def pin_fp8_decode_vs_torch():
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float32)
    for c in range(256):
        got = oracle.fp8_decode(c)
        r = float(ref[c])
        if math.isnan(r):
            assert math.isnan(got), hex(c)
        else:
            assert got == r and math.copysign(1, got) == math.copysign(1, r), (hex(c), got, r)


def pin_fp8_encode_vs_torch(step: int = 1, chunk: int = 1 << 26):
    """Every binary32 bit pattern in [0, 448] (step 1), or a strided subset."""
    top = int(np.array(448.0, np.float32).view(np.uint32))
    for start in range(0, top + 1, chunk * step):
        stop = min(top + 1, start + chunk * step)
        a = np.arange(start, stop, step, dtype=np.uint32).view(np.float32)
        got = oracle.fp8_encode(a)
        ref = torch.from_numpy(a).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        bad = np.nonzero(got != ref)[0]
        assert bad.size == 0, ("fp8 encode differs from torch", a[bad[:5]],
                               got[bad[:5]], ref[bad[:5]])


def pin_fp8_saturation():
    vals = np.array([448.0, 448.00003, 460.0, 464.0, 470.0, 480.0, 500.0, 1e4,
                     3.0e38, np.inf], np.float32)
    assert np.all(oracle.fp8_encode(vals) == 0x7E)


def pin_fp8_roundtrip():
    for c in range(0x7F):
        assert oracle.fp8_encode_scalar(oracle.fp8_decode(c)) == c, hex(c)


def pin_e2m1_format():
    """The 16 E2M1 codes from the OCP bit-field definition."""
    for nib in range(16):
        s, e, m = nib >> 3, (nib >> 1) & 3, nib & 1
        mag = 0.5 * m if e == 0 else 2.0 ** (e - 1) * (1 + 0.5 * m)
        want = -mag if s else mag
        got = oracle.e2m1_decode(nib)
        assert got == want and math.copysign(1, got) == math.copysign(1, want), nib


def pin_e2m1_table():
    """step_to_idx equals ties-to-even nearest rounding of hs/2 onto the E2M1
    grid (brute force over the grid)."""
    from fractions import Fraction as F
    for hs in range(13):
        assert oracle.e2m1_index(hs) == twin.e2m1_nearest_index(F(hs, 2)), hs
    assert oracle.e2m1_index(13) == -1 and oracle.e2m1_index(-1) == -1


def _swiglu_inputs(n=200000, seed=11):
    rng = np.random.default_rng(seed)
    g = np.concatenate([rng.standard_normal(n) * 3,
                        rng.uniform(-120, 120, n // 4),
                        np.array([0.0, -0.0, 1e-3, -1e-3, 20, -20, 88, -88, 100, -100,
                                  700, -700, 800, -800])])
    u = np.concatenate([rng.standard_normal(g.size - 14) * 2,
                        np.array([1.0, -1.0, 2.0, -3.0, 1.0, 1.0, -1.0, 1.0, 1.0,
                                  2.0, 1.0, 1.0, -1.0, 1.0])])
    gb = W.bf16_bits_to_f32(W.to_bf16_bits(g))
    ub = W.bf16_bits_to_f32(W.to_bf16_bits(u))
    return gb, ub


def pin_swiglu_vs_torch():
    g, u = _swiglu_inputs()
    gate_up = W.to_bf16_bits(W.interleave(g.reshape(1, -1)[:, :g.size // 8 * 8],
                                          u.reshape(1, -1)[:, :g.size // 8 * 8]))
    y = oracle.swiglu(gate_up).reshape(-1)
    n = y.size
    gt = torch.from_numpy(g[:n].astype(np.float64))
    ut = torch.from_numpy(u[:n].astype(np.float64))
    ref = (torch.nn.functional.silu(gt) * ut).to(torch.float32).numpy()
    # both are float64 evaluations rounded once to float32; allow 1 ulp
    yi = y.view(np.int32).astype(np.int64)
    ri = ref.view(np.int32).astype(np.int64)
    same_sign = np.signbit(y) == np.signbit(ref)
    ulps = np.abs(yi - ri)
    tiny = (np.abs(ref) < 1e-37) & (np.abs(y) < 1e-37)
    assert np.all(same_sign | tiny)
    assert np.all((ulps <= 1) | tiny), np.max(ulps)
    assert np.mean(ulps == 0) > 0.99


def pin_swiglu_closed_forms():
    # silu(0) * u = 0 with the sign of gate * up
    for g, u in ((0.0, 1.0), (0.0, -1.0), (-0.0, 1.0), (-0.0, -1.0), (2.0, 0.0), (2.0, -0.0)):
        y = oracle.swiglu_scalar(g, u)
        assert y == 0.0 and math.copysign(1, y) == math.copysign(1, g) * math.copysign(1, u)
    # for large gate, silu(g) = g to within 1 ulp of binary32, so y = RN(g*u)
    for g in (40.0, 64.0, 100.0, 1000.0):
        for u in (1.0, -2.5, 3.0):
            assert oracle.swiglu_scalar(g, u) == np.float32(g * u)
    # silu(g) - silu(-g) = g
    for g in (0.5, 1.0, 2.0, 3.75, 7.0):
        d = oracle.swiglu_scalar(g, 1.0) - oracle.swiglu_scalar(-g, 1.0)
        assert abs(d - g) <= 4 * np.spacing(np.float32(g))
    # silu(g) at a point checked by hand: g = ln 3 gives sigmoid 3/4
    g = float(np.float32(math.log(3.0)))
    assert abs(oracle.swiglu_scalar(g, 1.0) - 0.75 * g) <= 1e-6 * g


def _twin_blocks():
    rng = np.random.default_rng(21)
    blocks = [(vals, 1.0) for _, vals in W.standalone_blocks(rng)]
    for _ in range(150):
        scale = 10.0 ** rng.uniform(-4, 4)
        blocks.append((rng.standard_normal(16) * scale, 1.0))
    for _ in range(150):
        gs = float(np.float32(10.0 ** rng.uniform(-3, 1)))
        scale = 10.0 ** rng.uniform(-3, 3)
        blocks.append((rng.standard_normal(16) * scale, gs))
    # blocks whose s values sit exactly on half-steps at a non-power-of-two scale
    for d in (1.25, 1.75, 0.875, 3.0 / 512.0, 448.0):
        blocks.append((np.array(twin_ties()) * d, 1.0))
    return [(W.bf16_bits_to_f32(W.to_bf16_bits(v)), gs) for v, gs in blocks]


def twin_ties():
    return [6.0, 0.25, 0.75, 1.25, 1.75, 2.25, 2.5, 2.75, 3.25, 3.5, 3.75, 4.75,
            5.0, 5.25, 5.75, -0.25]


def pin_quantize_vs_twin():
    for x, gs in _twin_blocks():
        p, sf, bsf, v = oracle.quantize_block(x, gs)
        tp, tsf, tbsf, tv = twin.quantize_block(list(x), gs)
        assert sf == tsf, (x, gs, sf, tsf)
        assert list(p) == tp, (x, gs, list(p), tp)
        assert bsf == float(tbsf)
        assert [float(a) for a in v] == [float(b) for b in tv]


def pin_dequant_closed_form():
    """All 127 finite scales x random nibbles x three global scales, and a
    different global scale on every row, against RN32(RN32(e2m1 * scale) * gs)
    computed from the format definitions."""
    rng = np.random.default_rng(31)
    scales = np.arange(0, 0x7F, dtype=np.uint8).reshape(-1, 1)
    rows = scales.shape[0]
    per_row = (10.0 ** rng.uniform(-3, 1, rows)).astype(np.float32)   # a scale per row
    for gs_rows in (np.full(rows, 1.0, np.float32),
                    np.full(rows, np.float32(rng.uniform(1e-3, 1.0)), np.float32),
                    np.full(rows, 3.3e-3, np.float32), per_row):
        p = rng.integers(0, 256, (rows, 8)).astype(np.uint8)
        p[0] = np.arange(0, 128, 16) | np.arange(1, 129, 16)   # all 16 nibbles once
        out = oracle.dequantize(p, scales, gs_rows)
        for r in range(rows):
            for c in range(16):
                byte = int(p[r, c // 2])
                nib = byte & 15 if c % 2 == 0 else byte >> 4
                want = twin.dequant_value(nib, int(scales[r, 0]), float(gs_rows[r]))
                assert out[r, c] == float(want), (r, c, nib, scales[r, 0], gs_rows[r])


def pin_group_amax():
    """Per-expert max |y| against numpy's own reduction over each expert's
    rows, with empty experts (amax 0) and each expert's extreme value planted
    on its first or last row and column, negative."""
    rng = np.random.default_rng(41)
    rows, cols = 300, 48
    y = (rng.standard_normal((rows, cols)) * 10.0 ** rng.uniform(-3, 3, (rows, 1))).astype(np.float32)
    offsets = np.array([0, 0, 1, 57, 57, 120, 299, 300, 300], np.int32)
    for e in range(offsets.size - 1):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi > lo:
            r, c = (hi - 1, cols - 1) if e % 2 else (lo, 0)
            y[r, c] = np.float32(-1.0e4 * (e + 1))
    got = oracle.group_amax(y, offsets)
    for e in range(offsets.size - 1):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        want = np.float32(np.max(np.abs(y[lo:hi]))) if hi > lo else np.float32(0.0)
        assert got[e] == want, (e, got[e], want)


def pin_expert_global_scale():
    """gs = RN32(amax / (6 * 448)): exact powers of two, 1.0 for an all-zero
    expert, the nearest binary32 to the exact rational quotient (also far
    outside any practical range, down into the subnormals), and the defining
    property that the expert's largest block gets scale byte 0x7e (the FP8
    maximum 448)."""
    from fractions import Fraction as F
    ks = np.arange(-20, 21)
    amax = (2688.0 * 2.0 ** ks).astype(np.float32)
    assert np.array_equal(oracle.expert_global_scale(amax), (2.0 ** ks).astype(np.float32))
    assert oracle.expert_global_scale(np.zeros(3, np.float32)).tolist() == [1.0, 1.0, 1.0]
    rng = np.random.default_rng(43)
    a = (10.0 ** rng.uniform(-6, 6, 400)).astype(np.float32)
    edge = np.array([2688.0 * 2.0 ** -100, 2688.0 * 2.0 ** -120, 1e-30, 1e-40, 2.0 ** -149,
                     2688.0 * 2.0 ** 101, 3.0e38], np.float32)
    a = np.concatenate([a, edge])
    gs = oracle.expert_global_scale(a)
    for ai, gi in zip(a, gs):
        q = F(float(ai)) / 2688
        err = abs(F(float(gi)) - q)
        for nb in (np.nextafter(gi, np.float32(np.inf)), np.nextafter(gi, np.float32(0))):
            assert err <= abs(F(float(nb)) - q), (ai, gi)
    assert gs[-7] == np.float32(2.0 ** -100) and gs[-6] == np.float32(2.0 ** -120)
    assert gs[-2] == np.float32(2.0 ** 101) and gs[-3] == 0.0     # 2^-149 / 2688 rounds to 0
    for ai, gi in zip(a[:100], gs[:100]):
        x = np.zeros(16, np.float32)
        x[5] = -ai
        _, sf, _, _ = oracle.quantize_block(x, float(gi))
        assert sf == 0x7E, (ai, gi, hex(sf))


def pin_bf16_vs_torch(step: int = 997, chunk: int = 1 << 24):
    """FP32 -> BF16 rounding against PyTorch's conversion (a library routine)
    over every step-th binary32 bit pattern (step 1: all of them)."""
    for start in range(0, 1 << 32, chunk * step):
        stop = min(1 << 32, start + chunk * step)
        a = np.arange(start, stop, step, dtype=np.uint64).astype(np.uint32).view(np.float32)
        got = oracle.f32_to_bf16(a)
        ref = torch.from_numpy(a).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        nan = np.isnan(a)
        assert np.all((got[nan] & 0x7FFF) > 0x7F80)
        bad = np.nonzero((got != ref) & ~nan)[0]
        assert bad.size == 0, ("bf16 differs from torch", a[bad[:5]], got[bad[:5]], ref[bad[:5]])


def pin_bf16_ties():
    """Closed form at exact ties (low 16 bits 0x8000): round to the even
    neighbour; just above or below a tie, to the nearer one. Covers normal,
    subnormal and the overflow to infinity."""
    rng = np.random.default_rng(51)
    hi = np.concatenate([rng.integers(0, 0x7F80, 20000), np.arange(0, 0x100),
                         np.arange(0x7F00, 0x7F80)]).astype(np.uint32)
    for sign in (0, 0x8000):
        h = hi | sign
        tie = ((h << 16) | 0x8000).view(np.float32)
        want = (h + (h & 1)).astype(np.uint16)
        assert np.array_equal(oracle.f32_to_bf16(tie), want)
        above = ((h << 16) | 0x8001).view(np.float32)
        assert np.array_equal(oracle.f32_to_bf16(above), (h + 1).astype(np.uint16))
        below = ((h << 16) | 0x7FFF).view(np.float32)
        assert np.array_equal(oracle.f32_to_bf16(below), h.astype(np.uint16))


def pin_swiglu_bf16_vs_torch():
    """The compact pass equals the (pinned) FP32 SwiGLU rounded by PyTorch."""
    x = W.random_fused(37, 1040, 61, 3.0)
    ref = torch.from_numpy(oracle.swiglu(x)).to(torch.bfloat16).view(torch.int16).numpy()
    assert np.array_equal(oracle.swiglu_bf16(x), ref.view(np.uint16))


def pin_swiglu_f32():
    """The FP32-input driver (fused-GEMM epilogue reference): bit-exact with
    the pinned BF16 driver on BF16-representable inputs, and within 1 ulp of
    PyTorch's float64 SiLU on arbitrary FP32 accumulators."""
    x = W.random_fused(11, 1040, 71, 2.0)
    assert np.array_equal(oracle.swiglu_f32(W.bf16_bits_to_f32(x)).view(np.uint32),
                          oracle.swiglu(x).view(np.uint32))
    rng = np.random.default_rng(72)
    acc = (rng.standard_normal((13, 2 * 1040)) * 4).astype(np.float32)
    y = oracle.swiglu_f32(acc)
    g = np.concatenate([acc[:, 16 * b: 16 * b + 8] for b in range(1040 // 8)], axis=1)
    u = np.concatenate([acc[:, 16 * b + 8: 16 * b + 16] for b in range(1040 // 8)], axis=1)
    ref = (torch.nn.functional.silu(torch.from_numpy(g.astype(np.float64))) *
           torch.from_numpy(u.astype(np.float64))).to(torch.float32).numpy()
    ulps = np.abs(y.view(np.int32).astype(np.int64) - ref.view(np.int32).astype(np.int64))
    assert np.all(ulps <= 1), ulps.max()


def pin_moe_l1_gemm():
    """The grouped float64 GEMM against a brute-force loop (every product and
    sum written out) on a tiny ragged case with empty experts, and its row
    selection against the full result."""
    rng = np.random.default_rng(73)
    tokens, hidden, n, experts = 11, 8, 6, 4
    x = W.to_bf16_bits(rng.standard_normal((tokens, hidden)))
    w = W.to_bf16_bits(rng.standard_normal((experts, n, hidden)))
    off = np.array([0, 0, 4, 4, 11], np.int32)
    got = oracle.moe_l1_gemm(x, w, off)
    xf, wf = W.bf16_bits_to_f32(x).astype(float), W.bf16_bits_to_f32(w).astype(float)
    for t in range(tokens):
        e = max(i for i in range(experts) if off[i] <= t and off[i + 1] > t)
        for j in range(n):
            want = 0.0
            for k in range(hidden):
                want += xf[t, k] * wf[e, j, k]
            assert abs(got[t, j] - want) <= 1e-12 * (1 + abs(want)), (t, j)
    sel = np.array([10, 3, 4, 0])
    assert np.array_equal(oracle.moe_l1_gemm(x, w, off, rows=sel), got[sel])
    one = oracle.moe_l1_gemm(x, w[1], None)
    assert np.allclose(one, xf @ wf[1].T, rtol=0, atol=1e-12)


def _twin_rows(x, gs_rows, packed, scales, what, rows=None, blocks=None):
    """Every block of the selected rows of FP32 x against the exact-rational
    twin with that row's global scale."""
    nb = x.shape[1] // 16
    for r in (range(x.shape[0]) if rows is None else rows):
        for b in (range(nb) if blocks is None else blocks):
            tp, tsf, _, _ = twin.quantize_block(list(x[r, 16 * b:16 * b + 16]), float(gs_rows[r]))
            assert scales[r, b] == tsf, (what, r, b, float(gs_rows[r]), scales[r, b], tsf)
            assert list(packed[r, 8 * b:8 * b + 8]) == tp, (what, r, b, float(gs_rows[r]))


def _row_scales(rows, seed):
    """One global scale per row: general binary32 values over 10^[-3, 1]
    (so the quantized bytes depend on them), with a few powers of two and 1.0."""
    rng = np.random.default_rng(seed)
    g = (10.0 ** rng.uniform(-3, 1, rows)).astype(np.float32)
    g[::5] = np.float32(2.0) ** rng.integers(-6, 3, g[::5].size).astype(np.float32)
    g[1] = np.float32(1.0)
    return g


def pin_quantize_rows_gs():
    """The row drivers with one global scale per row: quantize_bf16 and
    quantize_f32 against the exact-rational twin, block by block, on a ragged
    shape whose rows each carry a different scale. A driver that ignores
    gs_rows, uses one row's scale for every row or reads the wrong row's
    scale fails here."""
    rng = np.random.default_rng(81)
    rows, cols = 9, 80
    x = W.to_bf16_bits(rng.standard_normal((rows, cols)) * 10.0 ** rng.uniform(-2, 2, (rows, 1)))
    gs = _row_scales(rows, 82)
    p, s = oracle.quantize_bf16(x, gs)
    _twin_rows(W.bf16_bits_to_f32(x), gs, p, s, "quantize_bf16")
    xf = (rng.standard_normal((rows, cols)) * 10.0 ** rng.uniform(-3, 3, (rows, 1))).astype(np.float32)
    p, s = oracle.quantize_f32(xf, gs)
    _twin_rows(xf, gs, p, s, "quantize_f32")
    # reversing the rows reverses the output rows (the scale travels with its row)
    p2, s2 = oracle.quantize_f32(xf[::-1].copy(), gs[::-1].copy())
    assert np.array_equal(p2, p[::-1]) and np.array_equal(s2, s[::-1])


def pin_fused_driver():
    """The fused reference driver, the source of the expected bytes of every
    fused parity case, pinned through independent routes:
    * its FP32 SwiGLU output against PyTorch's float64 SiLU of the gate and up
      values that were interleaved into the input ([gate x8, up x8] subtiles,
      built here from separate gate and up tensors), within 1 ulp;
    * its bytes, block by block, against the exact-rational twin applied to
      PyTorch's values, with a different global scale on every row (ragged:
      the row length is not a multiple of 64 blocks)."""
    rng = np.random.default_rng(83)
    rows, inter = 7, 112
    g = W.to_bf16_bits(rng.standard_normal((rows, inter)) * 2.0)
    u = W.to_bf16_bits(rng.standard_normal((rows, inter)) * 10.0 ** rng.uniform(-2, 2, (rows, 1)))
    x = W.interleave(g, u)
    gs = _row_scales(rows, 84)
    p, s, y = oracle.swiglu_quantize(x, gs)
    gt = torch.from_numpy(W.bf16_bits_to_f32(g).astype(np.float64))
    ut = torch.from_numpy(W.bf16_bits_to_f32(u).astype(np.float64))
    ref = (torch.nn.functional.silu(gt) * ut).to(torch.float32).numpy()
    ulps = np.abs(y.view(np.int32).astype(np.int64) - ref.view(np.int32).astype(np.int64))
    assert np.all(ulps <= 1) and np.all(np.signbit(y) == np.signbit(ref)), "fused driver swiglu"
    assert np.mean(ulps == 0) > 0.99
    nb = inter // 16
    same = (y.view(np.uint32) == ref.view(np.uint32)).reshape(rows, nb, 16).all(axis=2)
    assert same.mean() > 0.9
    for r in range(rows):
        _twin_rows(ref, gs, p, s, "fused driver", rows=[r],
                   blocks=[b for b in range(nb) if same[r, b]])
    # without gs every row uses 1.0
    p1, s1, _ = oracle.swiglu_quantize(x)
    _twin_rows(ref, np.ones(rows, np.float32), p1, s1, "fused driver gs=1",
               rows=[0, rows - 1], blocks=[b for b in range(nb) if same[0, b] and same[rows - 1, b]])


def pin_rows_global_scale():
    """Per-expert scales expanded to rows by the offsets rule (row r belongs
    to expert e when offsets[e] <= r < offsets[e+1]), with empty experts,
    checked row by row."""
    off = np.array([0, 0, 3, 3, 4, 9, 9], np.int32)
    gs = np.array([0.5, 0.25, 3.0, 0.125, 7.0, 9.0], np.float32)
    got = oracle.rows_global_scale(gs, off, 9)
    for r in range(9):
        e = [i for i in range(gs.size) if off[i] <= r < off[i + 1]]
        assert len(e) == 1 and got[r] == gs[e[0]], (r, got[r])


def pin_paged_kv():
    """The paged KV-cache write and read against what the slot rule fixes:
    identity slots reduce to quantize_bf16 of the rows; permuting rows and
    slots together gives the same cache; rows whose slot is outside
    [0, num_slots) (-1, num_slots, far beyond, a large negative) leave a
    poisoned cache row untouched, as do slots no row names; the read returns
    dequantize of each named row and zeros for skipped slots; a global scale
    goes through as a per-row scale of quantize_bf16."""
    rng = np.random.default_rng(91)
    rows, cols, num_slots = 9, 64, 16
    x = W.to_bf16_bits(rng.standard_normal((rows, cols)) * 3.0)
    p_ref, s_ref = oracle.quantize_bf16(x)
    pc = np.full((rows, cols // 2), 0xA5, np.uint8)
    sc = np.full((rows, cols // 16), 0x5A, np.uint8)
    oracle.quantize_paged(x, np.arange(rows), pc, sc)
    assert np.array_equal(pc, p_ref) and np.array_equal(sc, s_ref)
    slots = np.array([5, -1, 0, 15, 16, 3, 1000, -7, 9], np.int64)
    pc = np.full((num_slots, cols // 2), 0xA5, np.uint8)
    sc = np.full((num_slots, cols // 16), 0x5A, np.uint8)
    oracle.quantize_paged(x, slots, pc, sc)
    named = {5: 0, 0: 2, 15: 3, 3: 5, 9: 8}
    for slot in range(num_slots):
        if slot in named:
            assert np.array_equal(pc[slot], p_ref[named[slot]]), slot
            assert np.array_equal(sc[slot], s_ref[named[slot]]), slot
        else:
            assert (pc[slot] == 0xA5).all() and (sc[slot] == 0x5A).all(), slot
    perm = rng.permutation(rows)
    pc2 = np.full_like(pc, 0xA5)
    sc2 = np.full_like(sc, 0x5A)
    oracle.quantize_paged(x[perm], slots[perm], pc2, sc2)
    assert np.array_equal(pc2, pc) and np.array_equal(sc2, sc)
    out = oracle.dequantize_paged(pc, sc, slots)
    deq = oracle.dequantize(p_ref, s_ref)
    for r, slot in enumerate(slots):
        if 0 <= slot < num_slots:
            assert np.array_equal(out[r], deq[r]), r
        else:
            assert (out[r] == 0).all() and not np.signbit(out[r]).any(), r
    g = np.float32(0.37)
    pg, sg = oracle.quantize_bf16(x, np.full(rows, g, np.float32))
    pc3 = np.zeros((rows, cols // 2), np.uint8)
    sc3 = np.zeros((rows, cols // 16), np.uint8)
    oracle.quantize_paged(x, np.arange(rows)[::-1].copy(), pc3, sc3, gs=float(g))
    assert np.array_equal(pc3, pg[::-1]) and np.array_equal(sc3, sg[::-1])
    assert np.array_equal(oracle.dequantize_paged(pc3, sc3, np.arange(rows)[::-1].copy(), gs=float(g)),
                          oracle.dequantize(pg, sg, np.full(rows, g, np.float32)))


ALL_PINS = [pin_page_facts, pin_fp8_decode_vs_torch, pin_fp8_saturation,
            pin_fp8_roundtrip, pin_e2m1_format, pin_e2m1_table, pin_swiglu_vs_torch,
            pin_swiglu_closed_forms, pin_quantize_vs_twin, pin_dequant_closed_form,
            pin_group_amax, pin_expert_global_scale, pin_bf16_vs_torch, pin_bf16_ties,
            pin_swiglu_bf16_vs_torch, pin_swiglu_f32, pin_moe_l1_gemm, pin_paged_kv,
            pin_quantize_rows_gs, pin_fused_driver, pin_rows_global_scale]


# ---- tests --------------------------------------------------------------------
@pytest.mark.parametrize("pin", ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin()


@pytest.mark.slow
def test_fp8_encode_exhaustive_vs_torch():
    pin_fp8_encode_vs_torch(step=1)


def test_standalone_workload_vs_twin():
    """Every block of the 128 x 256 standalone workload (random and injected)
    against the exact-rational twin."""
    w = W.standalone()
    packed, scales = oracle.quantize_bf16(w.x)
    x = W.bf16_bits_to_f32(w.x)
    rng = np.random.default_rng(5)
    nb = x.shape[1] // 16
    injected = list(w.meta["injected"].keys())
    sample = injected + [(int(r), int(b)) for r, b in
                         zip(rng.integers(0, x.shape[0], 300), rng.integers(0, nb, 300))]
    for r, b in sample:
        tp, tsf, _, _ = twin.quantize_block(list(x[r, 16 * b:16 * b + 16]), 1.0)
        assert scales[r, b] == tsf, (r, b)
        assert list(packed[r, 8 * b:8 * b + 8]) == tp, (r, b)


def test_standalone_injected_scales():
    """The injected blocks land where the pages and the format put them."""
    w = W.standalone()
    _, scales = oracle.quantize_bf16(w.x)
    x = W.bf16_bits_to_f32(w.x)
    for (r, b), kind in w.meta["injected"].items():
        blk = x[r, 16 * b:16 * b + 16]
        amax = float(np.max(np.abs(blk)))
        sf = int(scales[r, b])
        if kind in ("zero", "negzero", "tiny"):
            assert sf == 0x00, (kind, amax)
        elif kind == "large":
            want = {1440.0: 0x77, 1488.0: 0x78}.get(amax, 0x7E)
            assert sf == want, (amax, hex(sf))
        elif kind == "subnormal_scale":
            assert 0x01 <= sf <= 0x08, (amax, hex(sf))
        elif kind == "fp8_ties":
            want = {6.375: 0x38, 7.125: 0x3A, 11.625: 0x40}[amax]
            assert sf == want, (amax, hex(sf))


def test_invariants_random():
    rng = np.random.default_rng(41)
    rows, cols = 256, 512
    x = (rng.standard_normal((rows, cols)) *
         10.0 ** rng.uniform(-4, 4, (rows, 1))).astype(np.float32)
    gs = (10.0 ** rng.uniform(-2, 1, rows)).astype(np.float32)
    packed, scales, bsf, v = oracle.quantize_f32(x, gs, diag=True)
    assert scales.max() <= 0x7E
    deq = oracle.dequantize(packed, scales, gs)
    nb = cols // 16
    for r in range(rows):
        for b in range(nb):
            blk = x[r, 16 * b:16 * b + 16]
            sf = int(scales[r, b])
            dec = oracle.fp8_decode(sf)
            denom = np.float32(dec) * gs[r]
            if sf == 0 or bsf[r, b] >= 448.0 or bsf[r, b] < 2.0 ** -6:
                continue
            # unsaturated normal-scale block: the amax element gets magnitude 7
            j = int(np.argmax(np.abs(blk)))
            byte = int(packed[r, 8 * b + j // 2])
            nib = byte & 15 if j % 2 == 0 else byte >> 4
            assert nib & 7 == 7, (r, b)
            # reconstruction error is at most 1.25 denominators (|s| <= 6)
            err = np.abs(deq[r, 16 * b:16 * b + 16].astype(np.float64) - blk)
            assert np.all(err <= 1.25 * float(denom) * (1 + 2.0 ** -20)), (r, b)
    # v is 2 min(|s|, 6): in [0, 12]
    assert v.min() >= 0 and v.max() <= 12


def test_zero_blocks_and_signs():
    z = np.zeros(16, np.float32)
    p, sf, _, _ = oracle.quantize_block(z)
    assert sf == 0 and np.all(p == 0)
    p, sf, _, _ = oracle.quantize_block(-z)
    assert sf == 0 and np.all(p == 0x88)
    # a negative value that rounds to magnitude 0 keeps its sign bit
    x = _block_with(-0.1)
    p, _, _, _ = oracle.quantize_block(x)
    assert p[0] >> 4 == 0x8


@pytest.mark.slow
def test_bf16_exhaustive_vs_torch():
    pin_bf16_vs_torch(step=1)
