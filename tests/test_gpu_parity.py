"""Parity of the HIP path (through the C ABI) with the CPU oracle, on the GPU.

Standalone quantize and dequantize are bit-exact; the fused SwiGLU + NVFP4
path follows the acceptance rules in tests/parity.py, and on the seeded
workloads its bytes are also checked to equal the oracle's exactly.
Workloads: the 128x256 standalone tensor with its injected edge blocks, the
512x4096 and 8192x4096 fused tensors (every element checked), the 65536x6144
prefill tensor and the 131072x4096 ragged 256-expert tensor at full size
(sampled rows checked element by element against the acceptance rules with
the FP32 SwiGLU values, every row's bytes against the oracle's), plus edge
cases.
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
    assert torch.cuda.is_available(), "these tests need the GPU"
    M.binding.raw()     # loads libmoe_nvfp4.so or raises
    return M


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def dev_bf16(bits):
    return dev(bits.view(np.int16)).view(torch.bfloat16)


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def gs_tensor(gs):
    return None if gs is None else dev(np.asarray(gs, np.float32).reshape(-1))


# ---- standalone quantize: bit-exact -----------------------------------------------
def test_standalone_workload_bit_exact(M):
    w = W.standalone()
    say("nvfp4_quantize standalone 128x256 seed 1")
    p, s = M.nvfp4_quantize(dev_bf16(w.x))
    rp, rs = oracle.quantize_bf16(w.x)
    P.assert_bytes_equal("scales", host(s), rs)
    P.assert_bytes_equal("packed", host(p), rp)


def test_standalone_e2m1_convert_all_half_steps(M):
    """Every half-step value and sign through the hardware E2M1 convert,
    including -0 and the ties 2.5, 3.5, 5 (d = 1, scale byte 0x38)."""
    vals = np.array([k / 2 for k in range(13)] + [0.0, 6.0, 6.0], np.float64)
    rows = np.stack([vals, -vals, np.where(np.arange(16) % 2 == 0, vals, -vals)])
    x = W.to_bf16_bits(rows)
    say("nvfp4_quantize half-step blocks")
    p, s = M.nvfp4_quantize(dev_bf16(x))
    rp, rs = oracle.quantize_bf16(x)
    assert np.all(host(s) == 0x38)
    P.assert_bytes_equal("packed", host(p), rp)


@pytest.mark.parametrize("rows,cols,ld,seed", [
    (1, 16, 16, 1), (3, 48, 48, 2), (7, 1600, 1600, 3), (64, 4096, 4104, 4),
    (257, 1040, 1048, 5), (1000, 256, 256, 6),
    # 16-byte stores, tiles walked in pairs: an odd tile count (the last
    # tile closes its pair alone) with pairs that straddle a row break
    # (144 blocks = 64 + 64 + 16 per row), and 80-block rows with a pitch
    (5, 2304, 2304, 7), (9, 1280, 1296, 11), (1, 3072, 3072, 12)])
def test_standalone_shapes_bit_exact(M, rows, cols, ld, seed):
    rng = np.random.default_rng(seed)
    full = W.random_plain(rows, ld, seed, scale=10.0 ** rng.uniform(-3, 3))
    gs = np.float32(rng.uniform(0.01, 2.0))
    say("nvfp4_quantize", rows, cols, "ld", ld, "gs", gs)
    xt = dev_bf16(full)[:, :cols]
    p, s = M.nvfp4_quantize(xt, gs_tensor(gs))
    rp, rs = oracle.quantize_bf16(full[:, :cols], np.full(rows, gs, np.float32))
    P.assert_bytes_equal("scales", host(s), rs)
    P.assert_bytes_equal("packed", host(p), rp)


def test_standalone_experts_bit_exact(M):
    rows, cols, E = 3000, 512, 37
    x = W.random_plain(rows, cols, 8, scale=3.0)
    off = W.random_offsets(rows, E, seed=9, empty=6)
    gs = (10.0 ** np.random.default_rng(10).uniform(-3, 0, E)).astype(np.float32)
    say("nvfp4_quantize experts", rows, cols, E)
    p, s = M.nvfp4_quantize(dev_bf16(x), gs_tensor(gs), dev(off))
    rp, rs = oracle.quantize_bf16(x, oracle.rows_global_scale(gs, off, rows))
    P.assert_bytes_equal("scales", host(s), rs)
    P.assert_bytes_equal("packed", host(p), rp)


def test_standalone_experts_long_walk_bit_exact(M):
    """65536 x 4096 with 64 experts: 262144 tiles, so every wave of the
    persistent grid walks more than 64 tiles (in pairs) and refills its
    per-lane expert lookahead more than once."""
    rows, cols, E = 65536, 4096, 64
    x = W.random_plain(rows, cols, 13, scale=2.0)
    off = W.random_offsets(rows, E, seed=14, empty=5)
    gs = (10.0 ** np.random.default_rng(15).uniform(-3, 1, E)).astype(np.float32)
    say("nvfp4_quantize experts", rows, cols, E)
    p, s = M.nvfp4_quantize(dev_bf16(x), gs_tensor(gs), dev(off))
    rp, rs = oracle.quantize_bf16(x, oracle.rows_global_scale(gs, off, rows))
    P.assert_bytes_equal("scales", host(s), rs)
    P.assert_bytes_equal("packed", host(p), rp)


# ---- fused path ----------------------------------------------------------------------
def run_fused(M, x, gs=None, off=None, rows_gs=None, debug=True):
    xt = dev_bf16(x)
    out = M.swiglu_nvfp4_quantize(xt, gs_tensor(gs), None if off is None else dev(off),
                                  swiglu_out=debug)
    return [host(t) for t in out]


# The seeded workloads below also assert exact bytes: with sigma and the
# product in binary64 the kernel's y is the oracle's except within about
# 2^-52 of a binary32 rounding midpoint, and on these inputs none of those
# few values sits at a quantization boundary (the acceptance rule above stays
# the contract).
def assert_exact(rep, what):
    assert rep.scale_mismatch == 0 and rep.code_mismatch == 0, "%s not byte-exact: %s" % (what, rep)


def fused_check(M, x, what, gs=None, off=None, exact=False):
    rows = x.shape[0]
    gs_rows = None
    if gs is not None:
        gs_rows = (oracle.rows_global_scale(gs, off, rows) if off is not None
                   else np.full(rows, gs, np.float32))
    say("swiglu_nvfp4_quantize", what, x.shape)
    p, s, y = run_fused(M, x, gs, off)
    rp, rs, ry, rbsf, rv = oracle.swiglu_quantize(x, gs_rows, diag=True)
    rep = P.fused_report(p, s, y, rp, rs, ry, rbsf, rv, gs_rows)
    say(what, rep)
    P.assert_fused_ok(rep, what)
    if exact:
        assert_exact(rep, what)
    # the production launch (no FP32 debug output) writes the same bytes
    p2, s2 = run_fused(M, x, gs, off, debug=False)
    P.assert_bytes_equal(what + " production packed", p2, p)
    P.assert_bytes_equal(what + " production scales", s2, s)
    return rep


def test_fused_small_workload(M):
    fused_check(M, W.fused_small().x, "fused_small 512x4096", exact=True)


def test_fused_decode_workload(M):
    fused_check(M, W.decode().x, "decode 8192x4096", exact=True)


@pytest.mark.parametrize("rows,inter,seed,scale", [
    (1, 16, 1, 1.0), (5, 48, 2, 4.0), (33, 1040, 3, 0.01), (130, 3072, 4, 30.0),
    (64, 8192, 5, 1.0)])
def test_fused_shapes(M, rows, inter, seed, scale):
    fused_check(M, W.random_fused(rows, inter, seed, scale), "random %dx%d" % (rows, inter))


def test_fused_global_scale_and_experts(M):
    rows, inter, E = 2000, 512, 19
    x = W.random_fused(rows, inter, 12, 2.0)
    fused_check(M, x, "scalar gs", gs=np.float32(0.0371))
    off = W.random_offsets(rows, E, seed=13, empty=4)
    gs = (10.0 ** np.random.default_rng(14).uniform(-3, 0.5, E)).astype(np.float32)
    fused_check(M, x, "experts", gs=gs, off=off)


def test_fused_swiglu_extremes(M):
    """Gate across [-100, 100] (exp over/underflow, large |g|) and zeros of
    both signs."""
    rows, inter = 64, 1024
    rng = np.random.default_rng(15)
    g = rng.uniform(-100, 100, (rows, inter))
    u = rng.standard_normal((rows, inter)) * 10.0 ** rng.uniform(-2, 2, (rows, 1))
    g[0, :16] = 0.0
    g[1, :16] = -0.0
    u[2, :16] = -0.0
    x = W.to_bf16_bits(W.interleave(g, u))
    fused_check(M, x, "swiglu extremes")


def test_fused_pitched_input(M):
    rows, inter, ld = 300, 1024, 2 * 1024 + 64
    full = W.random_fused(rows, ld // 2, 16, 1.0)
    say("swiglu_nvfp4_quantize pitched", rows, inter, ld)
    xt = dev_bf16(full)[:, :2 * inter]
    p, s = [host(t) for t in M.swiglu_nvfp4_quantize(xt)]
    rp, rs, ry, rbsf, rv = oracle.swiglu_quantize(full[:, :2 * inter], diag=True)
    rep = P.fused_report(p, s, None, rp, rs, ry, rbsf, rv)
    say("pitched", rep)
    P.assert_fused_ok(rep, "pitched")


# ---- full-size workloads: sampled rows ------------------------------------------------
def _sample_rows(rows, n, seed, extra=()):
    rng = np.random.default_rng(seed)
    pick = set(rng.choice(rows, size=min(n, rows), replace=False).tolist())
    pick |= {0, rows - 1} | set(int(r) for r in extra if 0 <= r < rows)
    return np.array(sorted(pick))


def test_fused_prefill_full_size_sampled(M):
    w = W.prefill()
    rows, inter = w.rows, w.out_cols
    say("swiglu_nvfp4_quantize prefill", w.x.shape)
    xt = dev_bf16(w.x)
    p, s = M.swiglu_nvfp4_quantize(xt)
    p, s = host(p), host(s)
    del xt
    sel = _sample_rows(rows, 1024, 44)
    rp, rs, ry, rbsf, rv = oracle.swiglu_quantize(w.x[sel], diag=True)
    # same rows through the debug launch for the FP32 values and the re-quantize rule
    yp, ys, yy = run_fused(M, w.x[sel])
    P.assert_bytes_equal("debug vs production packed", yp, p[sel])
    P.assert_bytes_equal("debug vs production scales", ys, s[sel])
    rep = P.fused_report(p[sel], s[sel], yy, rp, rs, ry, rbsf, rv)
    say("prefill sampled", rep)
    P.assert_fused_ok(rep, "prefill sampled rows")
    # every row: the bytes equal the oracle's
    say("oracle over every prefill row")
    rp, rs, _ = oracle.swiglu_quantize(w.x)
    P.assert_bytes_equal("prefill scales, every row", s, rs)
    P.assert_bytes_equal("prefill packed, every row", p, rp)
    del rp, rs
    # properties over every row: scale bytes never NaN, zero scale <=> zero codes
    assert s.max() <= 0x7E
    z = s == 0
    codes = P.nibbles(p).reshape(rows, inter // 16, 16) & 7
    assert np.all(codes[z] == 0)


def test_fused_ragged_experts_and_dequant(M):
    w = W.ragged()
    rows, inter = w.rows, w.out_cols
    off = w.offsets
    say("oracle swiglu for per-expert global scales", w.x.shape)
    y_ref = oracle.swiglu(w.x)
    gs = oracle.expert_global_scale(oracle.group_amax(y_ref, off))
    gs_rows = oracle.rows_global_scale(gs, off, rows)
    say("swiglu_nvfp4_quantize ragged", w.x.shape, "experts", off.size - 1)
    xt = dev_bf16(w.x)
    gst, offt = gs_tensor(gs), dev(off)
    pt, st = M.swiglu_nvfp4_quantize(xt, gst, offt)
    # the on-device global-scale pre-pass at full size
    say("swiglu_nvfp4_global_scale ragged")
    ggs, gam = M.swiglu_nvfp4_global_scale(xt, offt, amax=True)
    ggs, gam = host(ggs), host(gam)
    amax_ref = oracle.group_amax(y_ref, off)
    assert np.all(np.abs(gam - amax_ref) <= P.SWIGLU_RTOL * amax_ref), "expert amax"
    P.assert_bytes_equal("gs from the GPU amax", ggs.view(np.uint32),
                         oracle.expert_global_scale(gam).view(np.uint32))
    # and on this input the GPU's SwiGLU maxima are the oracle's, bit for bit
    P.assert_bytes_equal("expert amax", gam.view(np.uint32), amax_ref.view(np.uint32))
    P.assert_bytes_equal("expert gs", ggs.view(np.uint32), gs.view(np.uint32))
    del xt
    say("nvfp4_dequantize ragged")
    dq = M.nvfp4_dequantize(pt, st, gst, offt)
    p, s, dq = host(pt), host(st), host(dq)
    counts = np.diff(off)
    bounds = np.concatenate([off[:-1], off[1:] - 1])
    sel = _sample_rows(rows, 2048, 55, extra=bounds)
    rp, rs, ry, rbsf, rv = oracle.swiglu_quantize(w.x[sel], gs_rows[sel], diag=True)
    rep = P.fused_report(p[sel], s[sel], None, rp, rs, ry, rbsf, rv)
    say("ragged sampled", rep, "empty experts", int((counts == 0).sum()))
    P.assert_fused_ok(rep, "ragged sampled rows")
    del y_ref
    say("oracle over every ragged row")
    rpa, rsa, _ = oracle.swiglu_quantize(w.x, gs_rows)
    P.assert_bytes_equal("ragged scales, every row", s, rsa)
    P.assert_bytes_equal("ragged packed, every row", p, rpa)
    del rpa, rsa
    # dequant round trip, every row: bit-exact against the oracle's dequant of
    # the GPU bytes (equal to the oracle's own bytes, checked above)
    say("oracle dequant over every ragged row")
    rdq = oracle.dequantize(p, s, gs_rows)
    P.assert_bytes_equal("dequant, every row", dq.view(np.uint32), rdq.view(np.uint32))


# ---- more experts than the LDS expert table holds -------------------------------------
@pytest.mark.parametrize("experts,empty,seed", [(1025, 100, 31), (1500, 300, 32), (4000, 1500, 33)])
def test_many_experts_scalar_lookup(M, experts, empty, seed):
    """Above 1024 experts the quantize kernels find each tile's expert by a
    per-tile scalar binary search instead of the workgroup's LDS table, and
    the dequantize always does: standalone quantize, fused quantize and
    dequantize against the oracle's per-row scales, with empty experts
    (including the first and the last) and a ragged row length (1040 values:
    one full and one partial tile per row). The global-scale calls, whose
    per-workgroup maxima live in LDS, reject that many experts."""
    rows, cols = 6000, 1040
    rng = np.random.default_rng(seed)
    off = W.random_offsets(rows, experts, seed, empty=empty)
    assert np.count_nonzero(np.diff(off) == 0) >= empty // 2
    gs = (10.0 ** rng.uniform(-3, 1, experts)).astype(np.float32)
    gs[::7] = np.float32(2.0) ** rng.integers(-8, 3, gs[::7].size).astype(np.float32)
    gs_rows = oracle.rows_global_scale(gs, off, rows)
    gst, offt = gs_tensor(gs), dev(off)
    x = W.random_plain(rows, cols, seed, scale=3.0)
    say("nvfp4_quantize", rows, cols, "experts", experts)
    p, s = M.nvfp4_quantize(dev_bf16(x), gst, offt)
    rp, rs = oracle.quantize_bf16(x, gs_rows)
    P.assert_bytes_equal("scales", host(s), rs)
    P.assert_bytes_equal("packed", host(p), rp)
    say("nvfp4_dequantize", rows, cols, "experts", experts)
    dq = host(M.nvfp4_dequantize(p, s, gst, offt))
    P.assert_bytes_equal("dequant", dq.view(np.uint32), oracle.dequantize(rp, rs, gs_rows).view(np.uint32))
    xf = W.random_fused(rows, cols, seed + 100, 2.0)
    fused_check(M, xf, "fused, %d experts" % experts, gs=gs, off=off)
    with pytest.raises(M.Nvfp4Error):
        M.nvfp4_global_scale(dev_bf16(x), offt)


# ---- extreme values: saturated scales, overflowing quotients, infinite SwiGLU --------
def _huge_blocks(rows, cols, rng):
    """BF16 values spread over the whole finite range, both signs, with
    blocks of one huge value among small ones, zeros of both signs and the
    largest finite BF16."""
    x = rng.standard_normal((rows, cols)) * 10.0 ** rng.uniform(-5, 38.5, (rows, 1))
    x = np.clip(x, -3.38e38, 3.38e38)
    x[0, :16] = 0.0
    x[0, 16:32] = -0.0
    x[1, :16] = rng.standard_normal(16)
    x[1, 5] = 3.38e38
    x[2, 16:32] = -3.38e38
    x[3, :16] = rng.standard_normal(16) * 1e-30
    x[3, 7] = -2.0e38
    return W.to_bf16_bits(x)


@pytest.mark.parametrize("gs", [2.0 ** -60, 3.0e-17, 1.0, 2.0 ** 60],
                         ids=["gs_2^-60", "gs_3e-17", "gs_1", "gs_2^60"])
def test_standalone_saturated_and_overflowing_quotients(M, gs):
    """Tiny global scales (down to the range's end, power of two and general)
    with values up to the largest finite BF16: the block scales saturate at
    448 and many quotients x / (d/2) lie beyond the binary32 range, which the
    kernel clamps before dividing. Bit-exact against the oracle, which divides
    in IEEE arithmetic (an infinite quotient gives the largest code)."""
    rows, cols = 64, 512
    x = _huge_blocks(rows, cols, np.random.default_rng(71))
    g = np.float32(gs)
    say("nvfp4_quantize extremes, gs", float(g))
    p, s = M.nvfp4_quantize(dev_bf16(x), gs_tensor(g))
    rp, rs = oracle.quantize_bf16(x, np.full(rows, g, np.float32))
    P.assert_bytes_equal("scales", host(s), rs)
    P.assert_bytes_equal("packed", host(p), rp)
    assert (rs == 0x7E).any()


@pytest.mark.parametrize("gs", [1.0, 2.0 ** -60, 3.0e-17], ids=["gs_1", "gs_2^-60", "gs_3e-17"])
def test_fused_infinite_and_tiny_swiglu(M, gs):
    """Gates and ups whose products leave the FP32 range (SwiGLU values that
    are infinite, and finite ones behind an overflowed g u), gates far below
    -87 (sigmoid below the binary32 range) and tiny products, with ordinary
    and tiny global scales: the fused acceptance rules (no SwiGLU floor but
    one subnormal step) and the re-quantize rule."""
    rng = np.random.default_rng(72)
    rows, inter = 64, 512
    gvals = np.array([200.0, -200.0, 1.5, -1.5, -90.0, -100.0, -300.0, 40.0, 0.5, -0.0])
    uvals = np.array([3.38e38, -3.38e38, 2.5e38, 1e30, -3e35, 1e-38, -2.0 ** -133, 1.0])
    g = rng.choice(gvals, (rows, inter)) * rng.uniform(0.5, 1.0, (rows, inter))
    u = rng.choice(uvals, (rows, inter)) * rng.uniform(0.5, 1.0, (rows, inter))
    g[:8] = rng.standard_normal((8, inter))            # ordinary rows too
    x = W.to_bf16_bits(W.interleave(g, u))
    y = oracle.swiglu(x)
    assert np.isinf(y).any() and (np.abs(y[np.isfinite(y)]) > 1e37).any()
    fused_check(M, x, "infinite and tiny swiglu, gs %r" % gs, gs=np.float32(gs))


# ---- global-scale pre-pass ----------------------------------------------------------------
def _group_max(y, off):
    return np.array([np.max(np.abs(y[a:b])) if b > a else 0.0 for a, b in zip(off[:-1], off[1:])],
                    np.float32)


@pytest.mark.parametrize("rows,cols,experts,empty,seed", [
    (1, 16, 0, 0, 1), (300, 1040, 7, 2, 2), (1024, 2048, 64, 9, 3), (77, 4096, 0, 0, 4)])
def test_global_scale_plain_exact(M, rows, cols, experts, empty, seed):
    x = W.random_plain(rows, cols, seed, scale=10.0)
    off = W.random_offsets(rows, experts, seed, empty=empty) if experts else None
    # plant each expert's extreme on its first or last row, negative
    groups = off if off is not None else np.array([0, rows], np.int32)
    for e, (a, b) in enumerate(zip(groups[:-1], groups[1:])):
        if b > a:
            x[b - 1 if e % 2 else a, (7 * e) % cols] = W.to_bf16_bits(np.array([-3.0e4 - e]))[0]
    xf = W.bf16_bits_to_f32(x)
    say("nvfp4_global_scale", rows, cols, "experts", experts, "empty", empty)
    xt = dev_bf16(x)
    offt = None if off is None else dev(off)
    gs, am = M.nvfp4_global_scale(xt, offt, amax=True)
    gs2 = M.nvfp4_global_scale(xt, offt)            # gs doubles as the accumulator
    gs, am, gs2 = host(gs), host(am), host(gs2)
    ref_am = oracle.group_amax(xf, groups)
    P.assert_bytes_equal("amax", am.view(np.uint32), ref_am.view(np.uint32))
    ref_gs = oracle.expert_global_scale(ref_am)
    P.assert_bytes_equal("gs", gs.view(np.uint32), ref_gs.view(np.uint32))
    P.assert_bytes_equal("gs without amax", gs2.view(np.uint32), ref_gs.view(np.uint32))


@pytest.mark.parametrize("rows,inter,experts,empty,seed", [
    (64, 1040, 0, 0, 5), (700, 2048, 32, 5, 6), (513, 3072, 256, 40, 7)])
def test_global_scale_fused(M, rows, inter, experts, empty, seed):
    x = W.random_fused(rows, inter, seed, 2.0)
    off = W.random_offsets(rows, experts, seed, empty=empty) if experts else None
    groups = off if off is not None else np.array([0, rows], np.int32)
    say("swiglu_nvfp4_global_scale", rows, inter, "experts", experts, "empty", empty)
    xt = dev_bf16(x)
    offt = None if off is None else dev(off)
    gs, am = M.swiglu_nvfp4_global_scale(xt, offt, amax=True)
    _, _, y = M.swiglu_nvfp4_quantize(xt, swiglu_out=True)
    gs, am, y = host(gs), host(am), host(y)
    # exactly the largest |y| of the quantizer's own FP32 SwiGLU values
    P.assert_bytes_equal("amax vs the kernel's y", am.view(np.uint32),
                         _group_max(y, groups).view(np.uint32))
    ref_am = oracle.group_amax(oracle.swiglu(x), groups)
    assert np.all(np.abs(am - ref_am) <= P.SWIGLU_RTOL * ref_am), "amax vs oracle"
    P.assert_bytes_equal("gs", gs.view(np.uint32),
                         oracle.expert_global_scale(am).view(np.uint32))
    # the quantize that consumes these scales meets the fused acceptance rules
    fused_check(M, x, "fused with device global scales", gs=gs if off is not None else gs[0],
                off=off)


def test_global_scale_empty_and_zero(M):
    for fn, cols in ((M.nvfp4_global_scale, 32), (M.swiglu_nvfp4_global_scale, 64)):
        gs, am = fn(torch.zeros((0, cols), dtype=torch.bfloat16, device="cuda"), amax=True)
        assert host(gs).tolist() == [1.0] and host(am).tolist() == [0.0]
        off = dev(np.zeros(5, np.int32))
        gs, am = fn(torch.zeros((0, cols), dtype=torch.bfloat16, device="cuda"), off, amax=True)
        assert host(gs).tolist() == [1.0] * 4 and host(am).tolist() == [0.0] * 4
        z = torch.zeros((40, cols), dtype=torch.bfloat16, device="cuda")
        off = dev(np.array([0, 10, 10, 40], np.int32))
        z[10:40] = 1.0
        gs, am = fn(z, off, amax=True)
        gs, am = host(gs), host(am)
        assert gs[0] == 1.0 and am[0] == 0.0 and gs[1] == 1.0 and am[1] == 0.0
        assert am[2] > 0 and gs[2] == np.float32(am[2]) / np.float32(2688.0)


def test_global_scale_clamped_range(M):
    """Product behaviour outside the quantizers' global-scale range: experts
    with tiny (~1e-30) and huge (~1e36) values get the oracle's
    RN32(amax / 2688) clamped to [2^-64, 2^64] (the range the kernels'
    quotients are exact for), and the quantize with those scales is
    bit-exact against the oracle fed the same scales."""
    rng = np.random.default_rng(61)
    rows, cols = 48, 256
    x = rng.standard_normal((rows, cols))
    x[:16] *= 1e-30
    x[16:32] *= 1e36
    xb = W.to_bf16_bits(x)
    off = np.array([0, 16, 32, 48], np.int32)
    say("global scale clamp: experts of magnitude 1e-30, 1e36, 1")
    gs, am = M.nvfp4_global_scale(dev_bf16(xb), dev(off), amax=True)
    gs, am = host(gs), host(am)
    ref_am = oracle.group_amax(W.bf16_bits_to_f32(xb), off)
    ref_gs = oracle.expert_global_scale(ref_am)
    assert np.array_equal(am.view(np.uint32), ref_am.view(np.uint32))
    assert ref_gs[0] < 2.0 ** -64 and ref_gs[1] > 2.0 ** 64 and 2.0 ** -64 < ref_gs[2] < 2.0 ** 64
    want = np.clip(ref_gs, np.float32(2.0 ** -64), np.float32(2.0 ** 64)).astype(np.float32)
    assert np.array_equal(gs.view(np.uint32), want.view(np.uint32)), (gs, ref_gs)
    p, s = M.nvfp4_quantize(dev_bf16(xb), dev(gs), dev(off))
    rp, rs = oracle.quantize_bf16(xb, oracle.rows_global_scale(gs, off, rows))
    P.assert_bytes_equal("scales", host(s), rs)
    P.assert_bytes_equal("packed", host(p), rp)


# ---- compact SwiGLU pass (two-pass variant) -------------------------------------------
def bf16_check(M, x, what, ld_out=None, quantize_cols=None):
    rows, inter = x.shape[0], x.shape[1] // 2
    xt = dev_bf16(x)
    if ld_out is None:
        buf = None
        out = torch.empty((rows, inter), dtype=torch.bfloat16, device="cuda")
    else:
        buf = torch.full((rows, ld_out), float("nan"), dtype=torch.bfloat16, device="cuda")
        out = buf[:, :inter]
    say("swiglu_bf16", what, x.shape, "ld_out", ld_out)
    M.swiglu_bf16(xt, out=out)
    got = host(out.contiguous().view(torch.int16)).view(np.uint16)
    rep = P.bf16_report(got, oracle.swiglu_bf16(x), oracle.swiglu(x))
    say(what, rep)
    assert rep.ok(), "%s: %s" % (what, rep)
    if buf is not None:     # the pitch padding is untouched
        pad = host(buf[:, inter:].contiguous().view(torch.int16)).view(np.uint16)
        assert np.all(pad == 0x7FC0), "padding written"
    # second pass: the standalone quantize of the GPU's own BF16 values, bit-exact
    # (over the first quantize_cols columns: infinite values are outside the
    # quantizer's contract)
    qc = inter if quantize_cols is None else quantize_cols
    p, s = M.nvfp4_quantize(out[:, :qc])
    rp, rs = oracle.quantize_bf16(np.ascontiguousarray(got[:, :qc]))
    P.assert_bytes_equal(what + " two-pass scales", host(s), rs)
    P.assert_bytes_equal(what + " two-pass packed", host(p), rp)
    return got


def test_swiglu_bf16_exact_products(M):
    """Gates >= 256 make sigma exactly 1 in FP32, so y = gate * up is the exact
    product of two BF16 values (16 significant bits): the BF16 rounding of
    every pair of significands is checked bit for bit, with 3132 exact ties,
    mantissa carries, both signs and the overflow to inf."""
    i = np.arange(128)
    gate = (256.0 * (1 + i / 128.0)).reshape(-1, 1)
    ups = []
    for e in (0, -3, 9, -120, 100, 119):
        for sign in (1.0, -1.0):
            ups.append(sign * (1 + i / 128.0) * 2.0 ** e)
    up = np.concatenate(ups).reshape(1, -1)
    g = np.broadcast_to(gate, (128, up.shape[1]))
    u = np.broadcast_to(up, (128, up.shape[1]))
    x = W.to_bf16_bits(W.interleave(g, u))
    y = oracle.swiglu(x)
    with np.errstate(over="ignore"):
        exact = (g.astype(np.float64) * u.astype(np.float64)).astype(np.float32)
    assert np.array_equal(y, exact)
    assert ((y.view(np.uint32) & 0xFFFF) == 0x8000).sum() > 3000 and np.isinf(y).any()
    finite = up.shape[1] - 256             # the last exponent's columns overflow
    assert np.isfinite(y[:, :finite]).all() and np.isinf(y[:, finite:]).any()
    got = bf16_check(M, x, "exact products", quantize_cols=finite)
    P.assert_bytes_equal("exact products", got, oracle.swiglu_bf16(x))


def test_swiglu_bf16_workloads(M):
    bf16_check(M, W.fused_small().x, "fused_small 512x4096")
    bf16_check(M, W.decode().x, "decode 8192x4096")


@pytest.mark.parametrize("rows,inter,seed,scale,ld_out", [
    (1, 16, 1, 1.0, None), (5, 48, 2, 30.0, 56), (33, 1040, 3, 1.0, None),
    (130, 3072, 4, 0.01, 3136), (64, 8192, 5, 4.0, None)])
def test_swiglu_bf16_shapes(M, rows, inter, seed, scale, ld_out):
    bf16_check(M, W.random_fused(rows, inter, seed, scale), "random %dx%d" % (rows, inter), ld_out)


# ---- dequantize -----------------------------------------------------------------------
@pytest.mark.parametrize("rows,cols,seed", [(1, 16, 1), (9, 1040, 2), (513, 4096, 3)])
def test_dequant_bit_exact(M, rows, cols, seed):
    rng = np.random.default_rng(seed)
    p = rng.integers(0, 256, (rows, cols // 2)).astype(np.uint8)
    s = rng.integers(0, 0x7F, (rows, cols // 16)).astype(np.uint8)
    gs = np.float32(rng.uniform(1e-3, 4.0))
    say("nvfp4_dequantize", rows, cols, "gs", gs)
    out = host(M.nvfp4_dequantize(dev(p), dev(s), gs_tensor(gs)))
    ref = oracle.dequantize(p, s, np.full(rows, gs, np.float32))
    P.assert_bytes_equal("dequant", out.view(np.uint32), ref.view(np.uint32))


# ---- every byte written, deterministic ----------------------------------------------
def test_poisoned_outputs_fully_written(M):
    x = W.random_fused(77, 1040, 21, 1.0)
    xt = dev_bf16(x)
    results = []
    for poison in (0xA5, 0x5A):
        p = torch.full((77, 520), poison, dtype=torch.uint8, device="cuda")
        s = torch.full((77, 65), poison, dtype=torch.uint8, device="cuda")
        y = torch.full((77, 1040), float("nan"), dtype=torch.float32, device="cuda")
        say("swiglu_nvfp4_quantize poison", hex(poison))
        M.swiglu_nvfp4_quantize(xt, packed=p, scales=s, swiglu_out=y)
        results.append((host(p), host(s), host(y)))
    for a, b in zip(results[0], results[1]):
        assert np.array_equal(a.view(np.uint8), b.view(np.uint8))
    assert not np.isnan(results[0][2]).any()
    xq = W.random_plain(77, 1040, 22)
    outs = []
    for poison in (0xA5, 0x5A):
        p = torch.full((77, 520), poison, dtype=torch.uint8, device="cuda")
        s = torch.full((77, 65), poison, dtype=torch.uint8, device="cuda")
        M.nvfp4_quantize(dev_bf16(xq), packed=p, scales=s)
        outs.append((host(p), host(s)))
    assert np.array_equal(outs[0][0], outs[1][0]) and np.array_equal(outs[0][1], outs[1][1])
    o = [host(M.nvfp4_dequantize(dev(outs[0][0]), dev(outs[0][1]),
                                 out=torch.full((77, 1040), v, device="cuda")))
         for v in (float("nan"), 7.0)]
    assert np.array_equal(o[0].view(np.uint32), o[1].view(np.uint32))


def test_empty_inputs_are_noops(M):
    x = torch.zeros((0, 64), dtype=torch.bfloat16, device="cuda")
    p, s = M.swiglu_nvfp4_quantize(x)
    assert p.shape == (0, 16) and s.shape == (0, 2)
    p, s = M.nvfp4_quantize(torch.zeros((0, 32), dtype=torch.bfloat16, device="cuda"))
    assert p.shape == (0, 16)
    out = M.nvfp4_dequantize(torch.zeros((0, 8), dtype=torch.uint8, device="cuda"),
                             torch.zeros((0, 1), dtype=torch.uint8, device="cuda"))
    assert out.shape == (0, 16)
    torch.cuda.synchronize()


def test_bad_arguments_raise(M):
    x = torch.zeros((4, 40), dtype=torch.bfloat16, device="cuda")   # I = 20, not /16
    with pytest.raises(M.Nvfp4Error):
        M.swiglu_nvfp4_quantize(x)
    with pytest.raises(M.Nvfp4Error):
        M.nvfp4_quantize(torch.zeros((4, 24), dtype=torch.bfloat16, device="cuda"))


def test_outputs_as_torch_fp8_and_fp4_views(M):
    """The outputs are valid torch views: scales as float8_e4m3fn (torch's own
    decode of our scale bytes, on the GPU) and packed as float4_e2m1fn_x2;
    codes decoded from the nibbles (even element in the low nibble) times
    torch's scale values equal the library's dequantize exactly (gs = 1: the
    products are exact in FP32)."""
    x = W.random_fused(64, 1024, seed=21, scale=3.0)
    say("swiglu_nvfp4_quantize for dtype views", x.shape)
    p, s = M.swiglu_nvfp4_quantize(dev_bf16(x))
    rows, cols = p.shape[0], p.shape[1] * 2
    sv = s.view(torch.float8_e4m3fn)
    pv = p.view(torch.float4_e2m1fn_x2)
    assert sv.shape == s.shape and pv.shape == p.shape
    dq = M.nvfp4_dequantize(p, s)
    nib = torch.stack([p & 15, p >> 4], dim=-1).reshape(rows, cols).long()
    e2m1 = torch.tensor([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], device="cuda")
    sign = 1.0 - 2.0 * (nib >> 3).float()
    vals = e2m1[nib & 7] * sign * sv.float().repeat_interleave(16, dim=1)
    torch.cuda.synchronize()
    assert torch.equal(vals, dq)
    assert int((s == 0x7F).sum()) == 0 and int((s == 0xFF).sum()) == 0   # never NaN
