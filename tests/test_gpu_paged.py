"""Paged KV-cache write and read on the GPU (nvfp4_quantize_paged and
nvfp4_dequantize_paged through the C ABI), bit-exact against the oracle.

The whole cache is compared byte for byte after each write, so rows that no
slot names must keep their poison bytes, and skipped tokens (slot -1, slots
at or past num_slots, large negative slots) must write nothing. Head sizes are
the attention head dimensions of the pages (64, 128, 256, 512), plus one row
length whose block count is not a multiple of 16 (the narrow store path).
"""
import numpy as np
import pytest
import torch

import oracle
from moe_swiglu_epilogue_amd import workloads as W

pytestmark = pytest.mark.gpu


def say(*a):
    print("[gpu]", *a, flush=True)


@pytest.fixture(scope="module")
def M():
    import moe_swiglu_epilogue_amd as M
    assert torch.cuda.is_available(), "these tests need the GPU"
    M.binding.raw()
    return M


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def poisoned(num_slots, cols):
    pc = np.full((num_slots, cols // 2), 0xA5, np.uint8)
    sc = np.full((num_slots, cols // 16), 0x5A, np.uint8)
    return pc, sc


def bits(a):
    return np.ascontiguousarray(a, np.float32).view(np.uint32)


@pytest.mark.parametrize("tokens,heads,head_dim,num_slots,seed,gs,pitch", [
    (300, 8, 128, 1024, 1, None, 0),
    (257, 1, 64, 300, 2, 0.37, 0),
    (64, 4, 256, 64, 3, None, 16),
    (1000, 2, 512, 5000, 4, 2.0, 0),
    (129, 3, 80, 400, 5, None, 8),      # 240 columns: 15 blocks per row (narrow stores)
])
def test_paged_write_and_read_bit_exact(M, tokens, heads, head_dim, num_slots, seed, gs, pitch):
    w = W.kv_cache(seed, tokens, heads, head_dim, num_slots if num_slots > tokens else tokens,
                   pad_fraction=0.05)
    cols = heads * head_dim
    if num_slots <= tokens:                 # every slot used exactly once (a permutation)
        slots = np.random.default_rng(seed).permutation(num_slots).astype(np.int64)
    else:
        slots = w.slots.copy()
    slots[3::17] = num_slots + np.arange(len(slots[3::17]))      # past the cache: skipped
    slots[5::29] = -(2 ** 40)                                    # far negative: skipped
    say("nvfp4_quantize_paged", tokens, "x", cols, "slots", num_slots, "gs", gs, "pitch", pitch,
        "skipped", int(((slots < 0) | (slots >= num_slots)).sum()))
    xb = np.zeros((tokens, cols + pitch), np.uint16)
    xb[:, :cols] = w.x
    x = dev(xb.view(np.int16)).view(torch.bfloat16)[:, :cols]
    pc_ref, sc_ref = poisoned(num_slots, cols)
    pc, sc = dev(pc_ref), dev(sc_ref)
    g = None if gs is None else dev(np.array([gs], np.float32))
    M.nvfp4_quantize_paged(x, dev(slots), pc, sc, g)
    oracle.quantize_paged(w.x, slots, pc_ref, sc_ref, gs)
    assert np.array_equal(host(pc), pc_ref)
    assert np.array_equal(host(sc), sc_ref)
    read = np.concatenate([slots, np.array([-1, num_slots, 0, num_slots - 1], np.int64)])
    out = M.nvfp4_dequantize_paged(pc, sc, dev(read), g)
    ref = oracle.dequantize_paged(pc_ref, sc_ref, read, gs)
    assert np.array_equal(bits(host(out)), bits(ref))


def test_paged_successive_writes(M):
    """Two writes into one cache (as successive decode steps append tokens):
    the second leaves the first's rows alone."""
    a = W.kv_cache(11, 200, 8, 128, 1000, pad_fraction=0.0)
    b = W.kv_cache(12, 100, 8, 128, 1000, pad_fraction=0.0)
    free = np.setdiff1d(np.arange(1000), a.slots)
    b_slots = np.random.default_rng(12).choice(free, 100, replace=False).astype(np.int64)
    pc_ref, sc_ref = poisoned(1000, 1024)
    pc, sc = dev(pc_ref), dev(sc_ref)
    for wl, sl in ((a, a.slots), (b, b_slots)):
        say("nvfp4_quantize_paged step", wl.x.shape)
        M.nvfp4_quantize_paged(dev(wl.x.view(np.int16)).view(torch.bfloat16), dev(sl), pc, sc)
        oracle.quantize_paged(wl.x, sl, pc_ref, sc_ref)
    assert np.array_equal(host(pc), pc_ref) and np.array_equal(host(sc), sc_ref)


def test_paged_full_size(M):
    """The benchmark's KV workload: 65536 tokens x 8 heads x 128 into a
    131072-slot cache, 1% padding; every cache byte checked, then the read
    of all 65536 slots."""
    w = W.kv_cache()
    cols = w.heads * w.head_dim
    say("nvfp4_quantize_paged full size", w.x.shape, "slots", w.num_slots)
    pc_ref, sc_ref = poisoned(w.num_slots, cols)
    pc, sc = dev(pc_ref), dev(sc_ref)
    slots = dev(w.slots)
    M.nvfp4_quantize_paged(dev(w.x.view(np.int16)).view(torch.bfloat16), slots, pc, sc)
    oracle.quantize_paged(w.x, w.slots, pc_ref, sc_ref)
    assert np.array_equal(host(pc), pc_ref) and np.array_equal(host(sc), sc_ref)
    out = M.nvfp4_dequantize_paged(pc, sc, slots)
    ref = oracle.dequantize_paged(pc_ref, sc_ref, w.slots)
    assert np.array_equal(bits(host(out)), bits(ref))
