"""Benchmark: fused SwiGLU + NVFP4 quantize on the prefill-shaped MoE L1 output.

One step = one launch of ``swiglu_nvfp4_quantize`` over the whole prefill
workload: 65536 rows of interleaved BF16 [gate x8, up x8, ...] with
intermediate size 3072 (805,306,368 bytes read), writing 65536 x 1536 packed
E2M1 bytes and 65536 x 192 FP8 scale bytes. Inputs are seeded synthetic data
(gate/up ~ N(0,1) times a per-row lognormal(0,1) factor), resident in HBM
before timing starts.

Prints ONE JSON line with the throughput (HBM GB/s over the algorithmic bytes,
4.5625 B per output element), the roofline of the fused kernel, the CPU
oracle's throughput on the host cores, and secondary figures (standalone
quantize, dequantize, and in-repo read / copy kernels over the same input as
HBM ceilings).

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
"""
import argparse
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0               # MI355X HBM3E peak, 8 TB/s
ROWS, INTER = 65536, 3072
BYTES_PER_ELEM = 4.5625             # 4 B read (gate+up BF16) + 0.5 B codes + 1/16 B scale
ALG_BYTES = int(ROWS * INTER * BYTES_PER_ELEM)      # 918,552,576
PMC_SUMMARY = os.path.join(ROOT, "profiles", "fused_quantize_kernel_prefill_pmc.json")
CALIB_BLOCKS = 49152      # one 4 KB tile per wave over the 805 MB input


def load_calib():
    import ctypes as C
    from moe_swiglu_epilogue_amd import build
    if not os.path.exists(build.CALIB_LIB):
        raise RuntimeError("libnvfp4_calib.so is not built; run python -m moe_swiglu_epilogue_amd.build")
    lib = C.CDLL(build.CALIB_LIB)
    for fn in (lib.nvfp4_calib_copy, lib.nvfp4_calib_read):
        fn.argtypes = [C.c_void_p, C.c_void_p, C.c_int64, C.c_int32, C.c_void_p]
        fn.restype = C.c_int
    return lib


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for rel in ("moe_swiglu_epilogue_amd/csrc/moe_nvfp4.hip",
                "moe_swiglu_epilogue_amd/csrc/nvfp4_device.hpp"):
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic():
    """HBM bytes per launch from the committed rocprofv3 counter summary, when
    it was taken on the current kernel source; else None."""
    try:
        with open(PMC_SUMMARY) as f:
            s = json.load(f)
    except (OSError, ValueError):
        return None
    if s.get("kernel_source_sha256") != kernel_source_hash():
        return None
    return s.get("traffic_bytes_per_launch")


def checked(rc):
    if rc != 0:
        raise RuntimeError("calibration kernel returned %d" % rc)


def time_launches(fn, steps, warmup):
    """Warm up, then time `steps` back-to-back launches. Returns (wall seconds
    between two device synchronizations, device milliseconds per launch from
    one pair of HIP events recorded on the launch stream around the whole
    timed region)."""
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    start.record()
    for _ in range(steps):
        fn()
    end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return wall, start.elapsed_time(end) / steps


def cpu_baseline(x):
    """The CPU oracle on the same prefill input: all host threads over the
    whole workload (median of 3), plus one thread over 16384 rows."""
    import oracle
    n_elem = x.shape[0] * (x.shape[1] // 2)
    threads = oracle.num_threads()
    times = []
    for _ in range(3):
        t = time.perf_counter()
        oracle.swiglu_quantize(x)
        times.append(time.perf_counter() - t)
    med = statistics.median(times)
    oracle.set_num_threads(1)
    sub = x[:16384]
    t = time.perf_counter()
    oracle.swiglu_quantize(sub)
    one = time.perf_counter() - t
    oracle.set_num_threads(threads)
    one_elem = sub.shape[0] * (sub.shape[1] // 2)
    return {
        "value": round(n_elem * BYTES_PER_ELEM / med / 1e9, 3),
        "unit": "GB/s",
        "cores": threads,
        "kind": "oracle",
        "sample": "full prefill workload 65536x6144 BF16, median of 3 passes on %d threads "
                  "(%.2f s each); 1 thread over 16384 rows: %.3f GB/s"
                  % (threads, med, one_elem * BYTES_PER_ELEM / one / 1e9),
    }


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-secondary", action="store_true")
    ap.add_argument("--secondary-steps", type=int, default=20)
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: the fused SwiGLU+NVFP4 path has no cross-GPU "
              "step (rows shard with no exchange); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import moe_swiglu_epilogue_amd as M
    from moe_swiglu_epilogue_amd import workloads as W

    print("[bench] generating prefill workload %dx%d" % (ROWS, 2 * INTER), file=sys.stderr, flush=True)
    w = W.prefill(rows=ROWS, inter=INTER)
    dev = torch.device("cuda:0")
    x = torch.from_numpy(w.x.view(np.int16)).to(dev).view(torch.bfloat16)
    packed = torch.empty((ROWS, INTER // 2), dtype=torch.uint8, device=dev)
    scales = torch.empty((ROWS, INTER // 16), dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()

    def step():
        M.swiglu_nvfp4_quantize(x, packed=packed, scales=scales)

    print("[bench] timing %d steps after %d warmup" % (args.steps, args.warmup), file=sys.stderr, flush=True)
    wall, kern_ms = time_launches(step, args.steps, args.warmup)
    ms_per_step = wall * 1e3 / args.steps
    value = ALG_BYTES / (wall / args.steps) / 1e9
    achieved = ALG_BYTES / (kern_ms / 1e3) / 1e9

    secondary = None
    if not args.no_secondary:
        print("[bench] secondary: quantize, dequantize, copy ceiling", file=sys.stderr, flush=True)
        secondary = {}
        sec_steps = args.secondary_steps
        # standalone quantize of a compact BF16 tensor of the same output shape
        xq = x.view(torch.int16)[:, :INTER].contiguous().view(torch.bfloat16)
        pq = torch.empty_like(packed)
        sq = torch.empty_like(scales)
        _, mq = time_launches(lambda: M.nvfp4_quantize(xq, packed=pq, scales=sq), sec_steps, 3)
        secondary["nvfp4_quantize"] = {
            "shape": [ROWS, INTER], "bytes_per_launch": int(ROWS * INTER * 2.5625),
            "ms": round(mq, 4), "GB_s": round(ROWS * INTER * 2.5625 / mq / 1e6, 1)}
        del xq, pq, sq
        out = torch.empty((ROWS, INTER), dtype=torch.float32, device=dev)
        _, md = time_launches(lambda: M.nvfp4_dequantize(packed, scales, out=out), sec_steps, 3)
        secondary["nvfp4_dequantize"] = {
            "shape": [ROWS, INTER], "bytes_per_launch": int(ROWS * INTER * 4.5625),
            "ms": round(md, 4), "GB_s": round(ROWS * INTER * 4.5625 / md / 1e6, 1)}
        del out
        # in-repo calibration kernels over the same 805 MB input: HBM ceilings
        calib = load_calib()
        nbytes = x.numel() * 2
        scratch = torch.empty(CALIB_BLOCKS * 16, dtype=torch.uint8, device=dev)
        stream = torch.cuda.current_stream().cuda_stream
        _, mr = time_launches(lambda: checked(calib.nvfp4_calib_read(
            x.data_ptr(), scratch.data_ptr(), nbytes, CALIB_BLOCKS, stream)), sec_steps, 3)
        dst = torch.empty_like(x)
        _, mc = time_launches(lambda: checked(calib.nvfp4_calib_copy(
            x.data_ptr(), dst.data_ptr(), nbytes, CALIB_BLOCKS, stream)), sec_steps, 3)
        del dst, scratch
        read_gbs = nbytes / mr / 1e6
        copy_gbs = 2 * nbytes / mc / 1e6
        secondary["calib_read_ceiling"] = {"bytes_per_launch": nbytes, "ms": round(mr, 4),
                                           "GB_s": round(read_gbs, 1)}
        secondary["calib_copy_ceiling"] = {"bytes_per_launch": 2 * nbytes, "ms": round(mc, 4),
                                           "GB_s": round(copy_gbs, 1)}
        secondary["fused_frac_of_read_ceiling"] = round(achieved / read_gbs, 4)
        secondary["fused_frac_of_copy_ceiling"] = round(achieved / copy_gbs, 4)

    cpu = None
    if not args.no_cpu_baseline:
        print("[bench] cpu baseline (oracle on host cores)", file=sys.stderr, flush=True)
        cpu = cpu_baseline(w.x)

    line = {
        "metric": "fused SwiGLU+NVFP4 quantize HBM GB/s and % of MI355X peak, prefill shape",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic (seeded; gate/up N(0,1) x per-row lognormal(0,1))",
        "config": {"workload": "prefill-shaped MoE L1 epilogue", "rows": ROWS,
                   "intermediate": INTER, "input": [ROWS, 2 * INTER],
                   "layout": "interleaved [gate x8, up x8]", "global_scale": 1.0,
                   "alg_bytes_per_step": ALG_BYTES, "parallelism": "single GPU"},
        "pct_of_peak": round(100.0 * value / PEAK_HBM_GBS, 2),
        "elements_per_s": round(ROWS * INTER / (wall / args.steps), 1),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4),
                     "traffic": measured_traffic(),
                     "kernel": "quantize_tiles_kernel<FusedBlock, true>", "kernel_ms": round(kern_ms, 5)},
        "cpu_baseline": cpu,
        "secondary": secondary,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
