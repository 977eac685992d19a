"""Writes tests/golden/bench_output_sha256.json: the SHA-256 of the oracle's
output bytes for every workload that bench.py times, except the grouped GEMM
(its random operands are summed in a different order on the matrix cores, so
its bytes are not expected to match). bench.py hashes the outputs of its last
timed launch of each workload and reports whether they equal these.

Every value here comes from oracle/ on the seeded inputs of
moe_swiglu_epilogue_amd/workloads.py, with the bench's shapes and arguments:

* prefill (65536 x 6144, gs 1): the fused quantize; the standalone quantize of
  its first 3072 columns; the dequantize of the fused outputs; the per-tensor
  global scale; the compact SwiGLU pass and the quantize of its output;
* ragged (131072 x 4096, 256 experts): per-expert global scales from the
  expert amax, the fused quantize with them, and the dequantize;
* decode (8192 x 4096), the small standalone (128 x 256) and small fused
  (512 x 4096) workloads: the quantize outputs;
* the paged KV cache (65536 tokens x 1024 into 131072 zeroed slots): the cache
  after the write, and the read.

Run from the repository root: python tests/golden/make_bench_hashes.py
"""
import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
from moe_swiglu_epilogue_amd import workloads as W  # noqa: E402

OUT = os.path.join(os.path.dirname(os.path.abspath(__file__)), "bench_output_sha256.json")


def per_tensor_gs(y):
    return oracle.expert_global_scale(oracle.group_amax(y, np.array([0, y.shape[0]], np.int32)))


def compute(say=lambda *a: None) -> dict:
    """The digests, keyed as bench.py checks them."""
    h = {}

    say("prefill")
    x = W.prefill().x
    rows, two_i = x.shape
    inter = two_i // 2
    p, s, y = oracle.swiglu_quantize(x)
    h["prefill.packed"], h["prefill.scales"] = W.sha256(p), W.sha256(s)
    pq, sq = oracle.quantize_bf16(np.ascontiguousarray(x[:, :inter]))
    h["nvfp4_quantize.packed"], h["nvfp4_quantize.scales"] = W.sha256(pq), W.sha256(sq)
    del pq, sq
    h["nvfp4_dequantize.out"] = W.sha256(oracle.dequantize(p, s))
    h["global_scale.gs"] = W.sha256(per_tensor_gs(y))
    del p, s, y
    yb = oracle.swiglu_bf16(x)
    h["swiglu_bf16.out"] = W.sha256(yb)
    pt, st = oracle.quantize_bf16(yb)
    h["two_pass.packed"], h["two_pass.scales"] = W.sha256(pt), W.sha256(st)
    del x, yb, pt, st

    say("ragged")
    w = W.ragged()
    p, s, y = oracle.swiglu_quantize(w.x)
    gs = oracle.expert_global_scale(oracle.group_amax(y, w.offsets))
    g_rows = oracle.rows_global_scale(gs, w.offsets, w.rows)
    p, s, _ = oracle.swiglu_quantize(w.x, g_rows)
    h["ragged.gs"] = W.sha256(gs)
    h["ragged.packed"], h["ragged.scales"] = W.sha256(p), W.sha256(s)
    h["ragged.dequantize"] = W.sha256(oracle.dequantize(p, s, g_rows))
    del w, p, s, y

    say("decode, small")
    for name, w in (("decode", W.decode()), ("small_fused", W.fused_small())):
        p, s, _ = oracle.swiglu_quantize(w.x)
        h[name + ".packed"], h[name + ".scales"] = W.sha256(p), W.sha256(s)
    p, s = oracle.quantize_bf16(W.standalone().x)
    h["small_standalone.packed"], h["small_standalone.scales"] = W.sha256(p), W.sha256(s)

    say("paged KV cache")
    kv = W.kv_cache()
    cols = kv.heads * kv.head_dim
    pc = np.zeros((kv.num_slots, cols // 2), np.uint8)
    sc = np.zeros((kv.num_slots, cols // 16), np.uint8)
    oracle.quantize_paged(kv.x, kv.slots, pc, sc)
    h["kv_write.packed_cache"], h["kv_write.scales_cache"] = W.sha256(pc), W.sha256(sc)
    h["kv_read.out"] = W.sha256(oracle.dequantize_paged(pc, sc, kv.slots))
    return h


def main():
    h = compute(lambda *a: print(*a, flush=True))
    with open(OUT, "w") as f:
        json.dump(h, f, indent=1, sort_keys=True)
        f.write("\n")
    print("wrote", OUT, len(h), "hashes")


if __name__ == "__main__":
    main()
