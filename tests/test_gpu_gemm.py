"""Parity of the MoE L1 grouped GEMM (matrix cores) and its fused SwiGLU +
NVFP4 epilogue with the oracle: a float64 GEMM of the same BF16 operands,
rounded to FP32 accumulators, then the oracle's SwiGLU and quantizer.

* Exact-arithmetic operands (multiples of 1/8 and 1/16): every FP32 sum is
  exact in any order, so the GPU accumulators equal the oracle's bit for bit.
  The BF16 GEMM output is then bit-exact, and the fused path follows the fused
  acceptance rules of tests/parity.py (SwiGLU within 2e-6, codes exact
  outside rounding boundaries, zero-tolerance re-quantize).
* Random operands: the accumulators differ from the exact sums by rounding.
  Each is checked against the bound hidden * 2^-24 * sum_k |x_k w_k| (FP32
  summation in any order), the SwiGLU values against that bound propagated
  through silu(g) u, and the quantized bytes by re-quantizing the kernel's
  own FP32 SwiGLU values (zero tolerance).
* The production launch (no FP32 debug output) writes the same bytes.
"""
import numpy as np
import pytest
import torch

import oracle
import parity as P
from moe_swiglu_epilogue_amd import workloads as W

pytestmark = pytest.mark.gpu


def say(*a):
    print("[gpu]", *a, flush=True)


@pytest.fixture(scope="module")
def M():
    import moe_swiglu_epilogue_amd as M
    assert torch.cuda.is_available()
    M.binding.raw()
    return M


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def dev_bf16(bits):
    return dev(np.asarray(bits).view(np.int16)).view(torch.bfloat16)


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def run(M, g, gs=None, offsets=True):
    x, w = dev_bf16(g.x), dev_bf16(g.w1)
    off = dev(g.offsets) if offsets else None
    gst = None if gs is None else dev(np.asarray(gs, np.float32))
    out = M.moe_l1_gemm_bf16(x, w if offsets else w[0], off)
    p, s, y = M.moe_l1_gemm_swiglu_nvfp4(x, w if offsets else w[0], off, gst, swiglu_out=True)
    p2, s2 = M.moe_l1_gemm_swiglu_nvfp4(x, w if offsets else w[0], off, gst)
    res = dict(bf16=host(out.view(torch.int16)).view(np.uint16), p=host(p), s=host(s), y=host(y),
               p2=host(p2), s2=host(s2))
    P.assert_bytes_equal("production packed", res["p2"], res["p"])
    P.assert_bytes_equal("production scales", res["s2"], res["s"])
    return res


def gs_rows_of(g, gs, rows=None):
    if gs is None:
        return None
    r = oracle.rows_global_scale(np.asarray(gs, np.float32), g.offsets, g.x.shape[0])
    return r if rows is None else r[rows]


# hidden / 64 K slices: 1, 2, 3, 4, 5, 8, 16 and 64. The K loop loads slices
# one and two ahead with waits counted for the steady state; one slice loads
# nothing in the loop, two load only the first slice's successor, three or
# more run the steady state and its last two slices. The last two cases have
# more than 256 tiles, so some workgroups take a second tile, whose first
# slice is loaded during the first tile's epilogue (with one and two slices).
@pytest.mark.parametrize("tokens,hidden,inter,experts,seed", [
    (300, 256, 128, 5, 1), (1000, 512, 384, 9, 2), (257, 64, 128, 1, 3), (513, 1024, 256, 3, 4),
    (256, 4096, 128, 2, 5), (130, 128, 128, 2, 6), (260, 192, 256, 2, 7), (511, 320, 128, 4, 8),
    (40000, 64, 256, 3, 9), (40000, 128, 256, 5, 10)])
def test_gemm_exact_operands(M, tokens, hidden, inter, experts, seed):
    g = W.moe_gemm(seed, tokens, hidden, inter, experts, exact=True)
    acc = oracle.moe_l1_gemm(g.x, g.w1, g.offsets)
    acc32 = acc.astype(np.float32)
    assert np.array_equal(acc32.astype(np.float64), acc), "operands must sum exactly"
    gs = np.float32(np.random.default_rng(seed).uniform(0.01, 2.0, experts))
    say("moe_l1_gemm exact", tokens, hidden, inter, "experts", experts, g.offsets[:6])
    r = run(M, g, gs)
    P.assert_bytes_equal("bf16 GEMM", r["bf16"], oracle.f32_to_bf16(acc32))
    ry = oracle.swiglu_f32(acc32)
    gsr = gs_rows_of(g, gs)
    rp, rs, rbsf, rv = oracle.quantize_f32(ry, gsr, diag=True)
    rep = P.fused_report(r["p"], r["s"], r["y"], rp, rs, ry, rbsf, rv, gsr)
    say("fused GEMM exact", rep)
    if rep.swiglu_bad:
        yg, yr = r["y"].astype(np.float64), ry.astype(np.float64)
        bad = np.argwhere(~((np.abs(yg - yr) <= np.maximum(2e-6 * np.abs(yr), P.SWIGLU_ABS))
                            & (np.signbit(yg) == np.signbit(yr))))
        for t, j in bad[:8]:
            col = 16 * (j // 8) + j % 8
            say("swiglu outlier: g %r u %r gpu %r ref %r rel %.3g" % (
                float(acc32[t, col]), float(acc32[t, col + 8]), float(yg[t, j]), float(yr[t, j]),
                abs(yg[t, j] - yr[t, j]) / max(abs(yr[t, j]), 1e-45)))
    P.assert_fused_ok(rep, "fused GEMM exact operands")


def test_gemm_single_expert_no_offsets(M):
    g = W.moe_gemm(5, 200, 128, 128, 1, exact=True)
    acc32 = oracle.moe_l1_gemm(g.x, g.w1[0], None).astype(np.float32)
    r = run(M, g, None, offsets=False)
    P.assert_bytes_equal("bf16 GEMM, one expert", r["bf16"], oracle.f32_to_bf16(acc32))
    ry = oracle.swiglu_f32(acc32)
    rp, rs, rbsf, rv = oracle.quantize_f32(ry, None, diag=True)
    P.assert_fused_ok(P.fused_report(r["p"], r["s"], r["y"], rp, rs, ry, rbsf, rv), "one expert")


def test_gemm_pitched_operands(M):
    """x, w1 and the BF16 output as views into wider buffers (ld_x, ld_w and
    ld_out above the used columns). The padding of x and w1 holds BF16 NaN,
    so a read past `hidden` would poison the accumulators; the output's
    padding is poisoned and must stay untouched."""
    tokens, hidden, inter, E = 700, 256, 128, 3
    n = 2 * inter
    g = W.moe_gemm(41, tokens, hidden, inter, E, exact=True)
    nan = np.uint16(0x7FC0)
    xb = np.full((tokens, hidden + 72), nan, np.uint16)
    xb[:, :hidden] = g.x
    wb = np.full((E, n, hidden + 136), nan, np.uint16)
    wb[:, :, :hidden] = g.w1
    x = dev_bf16(xb)[:, :hidden]
    w = dev_bf16(wb)[:, :, :hidden]
    off = dev(g.offsets)
    out_big = torch.full((tokens, n + 40), -7.0, dtype=torch.bfloat16, device="cuda")
    M.moe_l1_gemm_bf16(x, w, off, out=out_big[:, :n])
    p, s, y = M.moe_l1_gemm_swiglu_nvfp4(x, w, off, None, swiglu_out=True)
    ob = host(out_big.view(torch.int16)).view(np.uint16)
    say("gemm pitched: ld_x %d ld_w %d ld_out %d" % (x.stride(0), w.stride(1), out_big.stride(0)))
    assert (ob[:, n:] == np.uint16(0xC0E0)).all(), "output padding was written"
    acc32 = oracle.moe_l1_gemm(g.x, g.w1, g.offsets).astype(np.float32)
    P.assert_bytes_equal("bf16 GEMM, pitched", ob[:, :n], oracle.f32_to_bf16(acc32))
    ry = oracle.swiglu_f32(acc32)
    rp, rs, rbsf, rv = oracle.quantize_f32(ry, None, diag=True)
    P.assert_fused_ok(P.fused_report(host(p), host(s), host(y), rp, rs, ry, rbsf, rv),
                      "fused GEMM, pitched operands")


@pytest.mark.parametrize("tokens,offsets", [
    (600, [0, 500, 100, 900, 300]),     # decreasing steps and an end past the rows
    (300, [0, 300, 0, 300, 0]),         # every other expert claims all rows again
    (300, [-50, 100, 200]),             # negative start; rows 200.. belong to no expert
])
def test_gemm_offsets_out_of_rule_stay_in_bounds(M, tokens, offsets):
    """expert_offsets that break the rules (device data, not checked) give
    unspecified bytes for the rows they cover but no access outside the
    buffers. The kernel clamps the offsets to [0, tokens] and takes their
    running maximum, so that the row ranges are disjoint; this pins that
    handling: covered rows equal the oracle's GEMM under those ranges, and
    the poisoned rows behind every output stay untouched."""
    E = len(offsets) - 1
    g = W.moe_gemm(31, tokens, 128, 128, E, exact=True)
    eff = np.maximum.accumulate(np.clip(np.asarray(offsets, np.int64), 0, tokens))
    covered = np.arange(eff[0], eff[-1])
    x, w = dev_bf16(g.x), dev_bf16(g.w1)
    off = dev(np.asarray(offsets, np.int32))
    n, inter, guard = 256, 128, 64
    out = torch.full((tokens + guard, n), -7.0, dtype=torch.bfloat16, device="cuda")
    pk = torch.full((tokens + guard, inter // 2), 0x5A, dtype=torch.uint8, device="cuda")
    sc = torch.full((tokens + guard, inter // 16), 0x5A, dtype=torch.uint8, device="cuda")
    yv = torch.full((tokens + guard, inter), -7.0, dtype=torch.float32, device="cuda")
    M.moe_l1_gemm_bf16(x, w, off, out=out[:tokens])
    M.moe_l1_gemm_swiglu_nvfp4(x, w, off, None, packed=pk[:tokens], scales=sc[:tokens],
                               swiglu_out=yv[:tokens])
    res = {k: host(t) for k, t in dict(out=out.view(torch.int16), pk=pk, sc=sc, y=yv).items()}
    say("gemm offsets out of rule", offsets, "-> ranges", eff.tolist())
    assert (res["out"][tokens:] == np.int16(np.float32(-7.0).view(np.int32) >> 16)).all()
    assert (res["pk"][tokens:] == 0x5A).all() and (res["sc"][tokens:] == 0x5A).all()
    assert (res["y"][tokens:] == np.float32(-7.0)).all()
    acc32 = oracle.moe_l1_gemm(g.x, g.w1, eff, rows=covered).astype(np.float32)
    P.assert_bytes_equal("bf16 GEMM, covered rows", res["out"][covered].view(np.uint16),
                         oracle.f32_to_bf16(acc32))
    ry = oracle.swiglu_f32(acc32)
    rp, rs, rbsf, rv = oracle.quantize_f32(ry, None, diag=True)
    rep = P.fused_report(res["pk"][covered], res["sc"][covered], res["y"][covered], rp, rs, ry,
                         rbsf, rv)
    P.assert_fused_ok(rep, "fused GEMM, covered rows")


def check_random(g, r, rows, gs=None):
    """Bound checks of a random-operand run on the given token rows."""
    acc = oracle.moe_l1_gemm(g.x, g.w1, g.offsets, rows=rows)
    mag = oracle.moe_l1_gemm(g.x & np.uint16(0x7FFF), g.w1 & np.uint16(0x7FFF), g.offsets, rows=rows)
    hidden = g.x.shape[1]
    bound = hidden * 2.0 ** -24 * mag + P.SWIGLU_ABS
    # BF16 output: within half a BF16 ulp of the exact sum, plus the bound
    got = (r["bf16"][rows].astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    half_ulp = np.abs(acc) * 2.0 ** -8 + 2.0 ** -134
    assert np.all(np.abs(got - acc) <= half_ulp + bound), "bf16 GEMM outside the bound"
    # SwiGLU: |dy| <= |u| |silu'(g)| dg + |silu(g)| du, silu'(g) = s (1 + g (1 - s))
    n = acc.shape[1]
    gi = np.concatenate([np.arange(16 * b, 16 * b + 8) for b in range(n // 16)])
    gg, uu = acc[:, gi], acc[:, gi + 8]
    bg, bu = bound[:, gi], bound[:, gi + 8]
    sg = 1.0 / (1.0 + np.exp(-np.clip(gg, -700, 700)))
    y_ref = gg * sg * uu
    tol = (np.abs(uu) * np.abs(sg * (1 + gg * (1 - sg))) * bg + np.abs(gg * sg) * bu
           + np.maximum(2e-6 * np.abs(y_ref), P.SWIGLU_ABS))
    err = np.abs(r["y"][rows].astype(np.float64) - y_ref)
    assert np.all(err <= tol), ("swiglu outside the bound", float((err / tol).max()))
    # bytes: the oracle quantizer on the kernel's own FP32 SwiGLU values
    qp, qs = oracle.quantize_f32(r["y"][rows], gs_rows_of(g, gs, rows))
    P.assert_bytes_equal("requantize packed", r["p"][rows], qp)
    P.assert_bytes_equal("requantize scales", r["s"][rows], qs)
    # code agreement with the oracle's own SwiGLU of the exact sums (reported)
    rp, rs = oracle.quantize_f32(oracle.swiglu_f32(acc.astype(np.float32)), gs_rows_of(g, gs, rows))
    return (float(np.mean(P.nibbles(rp) != P.nibbles(r["p"][rows]))),
            float(np.mean(rs != r["s"][rows])), float((err / tol).max()))


@pytest.mark.parametrize("tokens,hidden,inter,experts,seed", [
    (700, 1024, 256, 6, 11), (2048, 2048, 512, 16, 12), (600, 448, 256, 3, 13)])
def test_gemm_random_operands(M, tokens, hidden, inter, experts, seed):
    g = W.moe_gemm(seed, tokens, hidden, inter, experts)
    say("moe_l1_gemm random", tokens, hidden, inter, "experts", experts)
    r = run(M, g)
    codes, scl, worst = check_random(g, r, np.arange(tokens))
    say("random: code mismatch %.2e, scale mismatch %.2e vs the exact-sum oracle; worst err/tol %.3f"
        % (codes, scl, worst))


def test_gemm_many_small_experts(M):
    """256 experts with Zipf(1.1) row counts over 16384 rows: most experts are
    one partial 256-row tile, some are empty."""
    g = W.moe_gemm(21, 16384, 512, 256, 256, exact=True)
    counts = np.diff(g.offsets)
    say("moe_l1_gemm 256 experts exact: rows per expert min %d max %d, empty %d"
        % (counts.min(), counts.max(), (counts == 0).sum()))
    acc32 = oracle.moe_l1_gemm(g.x, g.w1, g.offsets).astype(np.float32)
    gs = np.float32(np.random.default_rng(21).uniform(0.05, 1.0, 256))
    r = run(M, g, gs)
    P.assert_bytes_equal("bf16 GEMM, 256 experts", r["bf16"], oracle.f32_to_bf16(acc32))
    ry = oracle.swiglu_f32(acc32)
    gsr = gs_rows_of(g, gs)
    rp, rs, rbsf, rv = oracle.quantize_f32(ry, gsr, diag=True)
    rep = P.fused_report(r["p"], r["s"], r["y"], rp, rs, ry, rbsf, rv, gsr)
    say("256 experts exact", rep)
    P.assert_fused_ok(rep, "fused GEMM, 256 experts")
    gr = W.moe_gemm(22, 16384, 512, 256, 256)
    rr = run(M, gr)
    codes, scl, worst = check_random(gr, rr, np.arange(16384))
    say("256 experts random: code mismatch %.2e, scale mismatch %.2e; worst err/tol %.3f"
        % (codes, scl, worst))


def test_gemm_prefill_shape_sampled(M):
    """32768 token rows, hidden 7168, I = 3072, 8 experts (Zipf): sampled rows
    (random, every expert's first and last row, the first rows of row tiles)."""
    g = W.moe_gemm()
    tokens = g.x.shape[0]
    say("moe_l1_gemm prefill-shaped", g.x.shape, g.w1.shape)
    r = run(M, g)
    rng = np.random.default_rng(66)
    extra = np.concatenate([g.offsets[:-1], g.offsets[1:] - 1, g.offsets[:-1] + 128])
    rows = np.unique(np.concatenate([rng.choice(tokens, 192, replace=False),
                                     extra[(extra >= 0) & (extra < tokens)]]))
    codes, scl, worst = check_random(g, r, rows)
    say("prefill-shaped sampled rows %d: code mismatch %.2e, scale mismatch %.2e; worst err/tol %.3f"
        % (rows.size, codes, scl, worst))


def test_gemm_epilogue_over_every_bf16_gate(M):
    """The fused epilogue's FP32 SwiGLU (exp2 and reciprocal, not the table of
    the standalone kernel) over every finite BF16 gate value times up values
    1, -1, 0.5 and -0.75. One-hot activations make the GEMM deliver chosen
    accumulators exactly: x[t][k] = (k == t), so acc[t][n] = w1[n][t]."""
    inter, rows = 4096, 64
    gates = np.concatenate([np.arange(0, 0x7F80), np.arange(0x8000, 0xFF80)]).astype(np.uint16)
    ups = np.array([0x3F80, 0xBF80, 0x3F00, 0xBF40], np.uint16)
    g = np.tile(gates, ups.size)
    u = np.repeat(ups, gates.size)
    n = rows * inter
    g = np.concatenate([g, np.zeros(n - g.size, np.uint16)]).reshape(rows, inter)
    u = np.concatenate([u, np.full(n - u.size, 0x3F80, np.uint16)]).reshape(rows, inter)
    acc_bits = W.interleave(g, u)                                   # [rows][2I]
    x = np.where(np.eye(rows, dtype=bool), np.uint16(0x3F80), np.uint16(0))
    w1 = np.ascontiguousarray(acc_bits.T)[None]                     # [1][2I][rows]
    off = np.array([0, rows], np.int32)
    wl = W.GemmWorkload(x, w1, off, inter)
    acc = oracle.moe_l1_gemm(x, w1, off)
    acc32 = acc.astype(np.float32)
    # each accumulator is its chosen value, except that a -0 gate sums with
    # +0 products to +0 (IEEE), on the GPU as in the oracle
    got = (acc32.view(np.uint32) >> 16).astype(np.uint16)
    assert np.array_equal(got[acc_bits != 0x8000], acc_bits[acc_bits != 0x8000])
    assert (got[acc_bits == 0x8000] == 0).all()
    say("moe_l1_gemm every BF16 gate through the epilogue:", x.shape, w1.shape)
    r = run(M, wl)
    P.assert_bytes_equal("bf16 GEMM", r["bf16"], oracle.f32_to_bf16(acc32))
    ry = oracle.swiglu_f32(acc32)
    rp, rs, rbsf, rv = oracle.quantize_f32(ry, None, diag=True)
    rep = P.fused_report(r["p"], r["s"], r["y"], rp, rs, ry, rbsf, rv)
    say("every-gate epilogue:", rep)
    if rep.swiglu_bad:
        yg, yr = r["y"].astype(np.float64), ry.astype(np.float64)
        bad = np.argwhere(~((np.abs(yg - yr) <= np.maximum(2e-6 * np.abs(yr), P.SWIGLU_ABS))
                            & (np.signbit(yg) == np.signbit(yr))))
        for t, j in bad[:: max(1, len(bad) // 24)][:24]:
            col = 16 * (j // 8) + j % 8
            say("outlier: g %r (0x%04x) u %r gpu %r ref %r" % (
                float(acc32[t, col]), int(acc_bits[t, col]), float(acc32[t, col + 8]),
                float(yg[t, j]), float(yr[t, j])))
        gbad = np.array([acc32[t, 16 * (j // 8) + j % 8] for t, j in bad])
        say("outlier gates: min %r max %r" % (float(gbad.min()), float(gbad.max())))
    assert rep.swiglu_bad == 0, rep
    assert rep.requant_mismatch == 0, rep
    assert rep.scale_mismatch == rep.scale_exempt, rep
    assert rep.code_mismatch == rep.code_exempt, rep
