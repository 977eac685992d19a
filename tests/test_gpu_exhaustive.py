"""Brute force of the standalone quantizer on the GPU against the oracle, bit
for bit, over the BF16 value space:

* every positive finite BF16 value as a block's amax (so every block-scale
  computation and FP8 encode the quantizer can reach from a BF16 input),
  each block holding 15 neighbouring values below the amax with
  alternating signs;
* one amax per BF16 exponent with every smaller BF16 magnitude as elements
  (random signs): about 2 million element quotients across 127 scales.

Both runs use a power-of-two global scale (the v_rcp_f32 path of the element
quotient) and a general one (the IEEE-division path).

The fused path gets the same treatment for its SwiGLU: every finite BF16 gate
value (both signs, zero and subnormals included: every entry of the kernel's
sigmoid table and both clamped ends) times up values of every size: 1, -1,
0.5 and -0.75; 1e30 and -3e35 (so that gates far below -87, whose sigmoid is
below the binary32 normal range, give SwiGLU values well inside it); the
largest BF16 (g u then overflows FP32 for |g| >= 1, though y may not); and
the smallest subnormal BF16 (products below the normal range). Each y is
checked against the oracle with the fused acceptance rules."""
from decimal import Decimal, localcontext

import numpy as np
import pytest
import torch

import oracle
import parity as P
from moe_swiglu_epilogue_amd import workloads as W

pytestmark = pytest.mark.gpu


def say(*a):
    print("[gpu]", *a, flush=True)


def amax_sweep_blocks():
    a = np.arange(0x0001, 0x7F80, dtype=np.int64)             # positive finite BF16
    j = np.arange(1, 16, dtype=np.int64)
    vals = np.maximum(a[:, None] - 37 * j[None, :], 0)          # smaller patterns
    sign = np.where(j % 2 == 1, 0x8000, 0)[None, :]
    blocks = np.concatenate([a[:, None], vals | sign], axis=1)
    return blocks.astype(np.uint16)


def element_sweep_blocks(seed=5):
    rng = np.random.default_rng(seed)
    out = []
    for amax in range(0x0100, 0x7F80, 0x100):                # one per exponent
        v = np.arange(0, amax, dtype=np.int64)
        v = v[:v.size - v.size % 15].reshape(-1, 15)
        v |= np.where(rng.random(v.shape) < 0.5, 0x8000, 0)
        out.append(np.concatenate([np.full((v.shape[0], 1), amax), v], axis=1))
    return np.concatenate(out).astype(np.uint16)


@pytest.mark.parametrize("gs", [1.0, 0.7], ids=["gs_pow2", "gs_general"])
def test_standalone_quantize_over_bf16_space(gs):
    import moe_swiglu_epilogue_amd as M
    blocks = np.concatenate([amax_sweep_blocks(), element_sweep_blocks()])
    nb = blocks.shape[0] - blocks.shape[0] % 16
    x = blocks[:nb].reshape(-1, 256)                            # 16 blocks per row
    say("standalone quantize over the BF16 space: %d blocks, gs %r" % (nb, gs))
    xt = torch.from_numpy(x.view(np.int16)).cuda().view(torch.bfloat16)
    g = np.float32(gs)
    p, s = M.nvfp4_quantize(xt, torch.tensor([g], device="cuda"))
    torch.cuda.synchronize()
    rp, rs = oracle.quantize_bf16(x, np.full(x.shape[0], g, np.float32))
    P.assert_bytes_equal("scales", s.cpu().numpy(), rs)
    P.assert_bytes_equal("packed", p.cpu().numpy(), rp)
    say("bit-exact: %d elements, %d distinct scale bytes" % (x.size, np.unique(rs).size))


def gate_sweep_input(inter=2048):
    gates = np.concatenate([np.arange(0, 0x7F80), np.arange(0x8000, 0xFF80)]).astype(np.uint16)
    # 1, -1, 0.5, -0.75, 1e30, -3e35, the largest finite BF16, -2^-133
    ups = np.concatenate([np.array([0x3F80, 0xBF80, 0x3F00, 0xBF40], np.uint16),
                          W.to_bf16_bits(np.array([1e30, -3e35])),
                          np.array([0x7F7F, 0x8001], np.uint16)])
    g = np.tile(gates, ups.size)
    u = np.repeat(ups, gates.size)
    n = -(-g.size // inter) * inter
    g = np.concatenate([g, np.zeros(n - g.size, np.uint16)]).reshape(-1, inter)
    u = np.concatenate([u, np.full(n - u.size, 0x3F80, np.uint16)]).reshape(-1, inter)
    return W.interleave(g, u)


def test_fused_swiglu_over_every_bf16_gate():
    import moe_swiglu_epilogue_amd as M
    x = gate_sweep_input()
    say("fused quantize over every finite BF16 gate:", x.shape)
    xt = torch.from_numpy(x.view(np.int16)).cuda().view(torch.bfloat16)
    p, s, y = M.swiglu_nvfp4_quantize(xt, swiglu_out=True)
    torch.cuda.synchronize()
    p, s, y = p.cpu().numpy(), s.cpu().numpy(), y.cpu().numpy()
    rp, rs, ry, rbsf, rv = oracle.swiglu_quantize(x, diag=True)
    rep = P.fused_report(p, s, y, rp, rs, ry, rbsf, rv)
    say("every-gate sweep:", rep)
    # every y within the SwiGLU tolerance; the GPU's bytes are exactly the
    # quantize of its own y; every byte that differs from the oracle's lies
    # at a rounding boundary (a directed sweep, so the exempt count is
    # reported, not capped by the random-workload fraction)
    assert rep.swiglu_bad == 0, rep
    assert rep.requant_mismatch == 0, rep
    assert rep.scale_mismatch == rep.scale_exempt, rep
    assert rep.code_mismatch == rep.code_exempt, rep
    # with the sigmoid in binary64, every gate's bytes are the oracle's
    assert rep.scale_mismatch == 0 and rep.code_mismatch == 0, rep
    # and every y with |g u| >= 2^-126 is the oracle's, bit for bit, unless
    # the exact g u sigma(g) lies within 2^-50 (relative) of the midpoint
    # between the two values (the kernel's binary64 sigma and product, and
    # the oracle's float64 evaluation, are each within a few 2^-53 of it),
    # which 60-digit arithmetic decides here for each such value; below
    # 2^-126 the kernel's binary32 g u is itself rounded, so y may be one
    # subnormal step away, which the SwiGLU rule allows
    gf = W.bf16_bits_to_f32(x)
    gu = np.stack([gf[:, 16 * k + j].astype(np.float64) * gf[:, 16 * k + 8 + j]
                   for k in range(x.shape[1] // 16) for j in range(8)], axis=1)
    differ = y.view(np.uint32) != ry.view(np.uint32)
    big = np.abs(gu) >= 2.0 ** -126
    odd = np.argwhere(differ & big)
    say("every-gate sweep: %d of %d SwiGLU values differ from the oracle's, %d of them "
        "with |g u| >= 2^-126" % (differ.sum(), y.size, len(odd)))
    assert len(odd) <= 32
    for r, c in odd:
        col = 16 * (c // 8) + c % 8
        with localcontext() as ctx:
            ctx.prec = 60
            g, u = Decimal(float(gf[r, col])), Decimal(float(gf[r, col + 8]))
            exact = g * u / (1 + (-g).exp())
            mid = (Decimal(float(y[r, c])) + Decimal(float(ry[r, c]))) / 2
            rel = abs(exact - mid) / abs(exact)
        say("  g %r u %r: kernel %r oracle %r, exact value %.3g from their midpoint"
            % (float(g), float(u), float(y[r, c]), float(ry[r, c]), float(rel)))
        assert rel <= Decimal(2) ** -50


def test_compact_swiglu_over_every_bf16_gate():
    """The compact BF16 SwiGLU pass (same sigmoid table, then round to BF16)
    over the same sweep: every output equals the oracle's BF16 rounding of
    its SwiGLU, except within the SwiGLU tolerance of a BF16 midpoint."""
    import moe_swiglu_epilogue_amd as M
    x = gate_sweep_input()
    say("compact swiglu over every finite BF16 gate:", x.shape)
    xt = torch.from_numpy(x.view(np.int16)).cuda().view(torch.bfloat16)
    out = M.swiglu_bf16(xt)
    torch.cuda.synchronize()
    got = out.view(torch.int16).cpu().numpy().view(np.uint16)
    rep = P.bf16_report(got, oracle.swiglu_bf16(x), oracle.swiglu(x))
    say("every-gate compact:", rep)
    assert rep.mismatch == rep.exempt, rep
