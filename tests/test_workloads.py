"""Seeded input generators: determinism, shapes and the stated structure."""
import numpy as np

from moe_swiglu_epilogue_amd import workloads as W


def test_bf16_rounding_is_rne():
    # 1 + 2^-8 is a tie between 1 and 1 + 2^-7: goes to the even mantissa (1)
    x = np.array([1.0, 1 + 2**-8, 1 + 3 * 2**-8, -2.5, 0.0, -0.0], np.float64)
    b = W.to_bf16_bits(x)
    back = W.bf16_bits_to_f32(b)
    assert back.tolist() == [1.0, 1.0, 1 + 2**-6, -2.5, 0.0, -0.0]
    assert np.signbit(back[5])


def test_interleave_layout():
    g = np.arange(32, dtype=np.float32).reshape(2, 16)
    u = -g
    x = W.interleave(g, u)
    assert x.shape == (2, 32)
    assert np.array_equal(x[0, 0:8], g[0, 0:8])
    assert np.array_equal(x[0, 8:16], u[0, 0:8])
    assert np.array_equal(x[0, 16:24], g[0, 8:16])
    assert np.array_equal(x[1, 24:32], u[1, 8:16])


def test_standalone_deterministic():
    a, b = W.standalone(), W.standalone()
    assert a.x.shape == (128, 256) and a.x.dtype == np.uint16
    assert W.sha256(a.x) == W.sha256(b.x)
    assert len(a.meta["injected"]) == len(W.standalone_blocks(np.random.default_rng(0)))
    assert W.sha256(W.standalone(seed=7).x) != W.sha256(a.x)


def test_fused_small_and_decode_shapes():
    w = W.fused_small()
    assert w.x.shape == (512, 4096) and w.fused and w.out_cols == 2048
    d = W.decode()
    assert d.x.shape == (8192, 4096)
    x = W.bf16_bits_to_f32(d.x)
    # 2 % of output blocks have all 32 feeding inputs at +0.0
    blocks = x.reshape(8192, 128, 32)
    zero = np.all(blocks == 0, axis=2)
    assert 0.015 < zero.mean() < 0.025
    # 1 % outliers x100 give a heavy tail
    assert np.max(np.abs(x)) > 1000


def test_prefill_chunks_are_independent():
    c0 = W.prefill_chunk(0, total_rows=8192, inter=64)
    c1 = W.prefill_chunk(1, total_rows=8192, inter=64)
    w = W.prefill(rows=8192, inter=64)
    assert np.array_equal(w.x[:4096], c0) and np.array_equal(w.x[4096:], c1)
    # per-row lognormal factor: row scales vary widely
    x = W.bf16_bits_to_f32(w.x)
    rms = np.sqrt(np.mean(x.astype(np.float64) ** 2, axis=1))
    assert rms.max() / rms.min() > 20


def test_ragged_offsets():
    off = W.ragged_offsets()
    assert off.dtype == np.int32 and off.size == 257
    assert off[0] == 0 and off[-1] == 131072
    counts = np.diff(off)
    assert np.all(counts >= 0)
    # Zipf(1.1): the largest expert holds far more rows than the median one
    assert counts.max() > 10 * np.median(counts)
    assert np.array_equal(off, W.ragged_offsets())


def test_random_offsets_with_empty_experts():
    off = W.random_offsets(1000, 16, seed=3, empty=3)
    c = np.diff(off)
    assert off[0] == 0 and off[-1] == 1000 and np.all(c >= 0)
    assert c[0] == 0 and (c == 0).sum() >= 2
