"""Benchmark: fused SwiGLU + NVFP4 quantize on the prefill-shaped MoE L1 output.

One step = one launch of ``swiglu_nvfp4_quantize`` over the whole prefill
workload: 65536 rows of interleaved BF16 [gate x8, up x8, ...] with
intermediate size 3072 (805,306,368 bytes read), writing 65536 x 1536 packed
E2M1 bytes and 65536 x 192 FP8 scale bytes. Inputs are seeded synthetic data
(gate/up ~ N(0,1) times a per-row lognormal(0,1) factor), resident in HBM
before timing starts.

Prints ONE JSON line with the throughput (HBM GB/s over the algorithmic bytes,
4.5625 B per output element), the roofline of the fused kernel, the CPU
oracle's throughput on the host cores, and secondary figures: the standalone
quantize, the dequantize and the global-scale pre-pass on the same tensor;
the two-pass ablation (compact BF16 SwiGLU, then the standalone quantize);
in-repo read / copy kernels over the same input as HBM ceilings, and a kernel
that moves the fused kernel's exact traffic mix (4 KB read, 576 B written
per wave tile) without its compute; the ragged
256-expert workload (pre-pass, quantize with per-expert scales, dequantize);
the decode-shaped workload over 8 rotating buffer sets, with the read and
traffic-mix ceilings at that size over the same rotation; the paged KV-cache
write and read (65536 tokens x 8 heads x 128, 131072 slots); the two small
cache-resident shapes (standalone 128 x 256, fused 512 x 4096) as launch
rates; the MoE L1 grouped GEMM with the fused epilogue against the unfused
flow and hipBLASLt.

Every timed region is preceded by --settle-ms of untimed back-to-back
launches (the clocks need ~30 ms of load to settle) and the warmup steps.
The last timed output of every workload but the GEMM is hashed and compared
with the digest of the oracle's output for the same input
(tests/golden/bench_output_sha256.json): `outputs_match_oracle`.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--settle-ms MS]
                  [--no-cpu-baseline] [--no-secondary] [--only ITEMS]
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
# SHA-256 of the oracle's outputs for the timed workloads, written by
# tests/golden/make_bench_hashes.py (which calls only oracle/)
EXPECTED_HASHES = os.path.join(ROOT, "tests", "golden", "bench_output_sha256.json")
# grid sizes (256-thread workgroups) tried for the calibration kernels; the
# best of them is the ceiling (measured: the read kernel peaks with a
# persistent grid of 6 workgroups per CU, the copy with one 4 KB tile per wave)
CALIB_READ_BLOCKS = (1024, 1536, 8192, 49152)
CALIB_COPY_BLOCKS = (512, 8192, 49152)
# unused dynamic LDS per 256-thread workgroup of the traffic-mix kernel (caps
# the waves per CU: all that fit, 16, 12)
CALIB_MIX_LDS = (0, 40960, 53248)
SECONDARY = ("nvfp4_quantize", "nvfp4_dequantize", "global_scale", "two_pass", "calib_read",
             "calib_copy", "calib_mix", "ragged", "decode", "small", "kv", "gemm")
PEAK_BF16_TFLOPS = 2500.0           # MI355X dense BF16 matrix peak


class OutputCheck:
    """Compares the SHA-256 of each workload's timed output with the digest of
    the oracle's output for the same input (stored in EXPECTED_HASHES). The
    benchmark runs no oracle code outside its CPU-baseline leg, so the other
    workloads are checked through these digests. A key without a stored digest
    is reported as unchecked."""

    def __init__(self):
        try:
            with open(EXPECTED_HASHES) as f:
                self.want = json.load(f)
        except (OSError, ValueError):
            self.want = {}
        self.results = {}

    @staticmethod
    def digest(t) -> str:
        import torch
        if t.dtype == torch.bfloat16:
            t = t.view(torch.int16)
        return hashlib.sha256(t.contiguous().cpu().numpy().tobytes()).hexdigest()

    def check(self, key, *tensors):
        """True when every tensor's bytes hash to the stored digest for key."""
        want = self.want.get(key)
        if want is None:
            self.results[key] = None
            return None
        ok = all(self.digest(t) == want for t in tensors)
        self.results[key] = ok
        return ok

    def report(self):
        done = {k: v for k, v in self.results.items() if v is not None}
        return {"checked": len(done), "matched": sum(1 for v in done.values() if v),
                "mismatched": sorted(k for k, v in done.items() if not v),
                "unchecked": sorted(k for k, v in self.results.items() if v is None),
                "expected_from": os.path.relpath(EXPECTED_HASHES, ROOT)}


def load_calib():
    import ctypes as C
    from moe_swiglu_epilogue_amd import build
    if not os.path.exists(build.CALIB_LIB):
        raise RuntimeError("libnvfp4_calib.so is not built; run python -m moe_swiglu_epilogue_amd.build")
    lib = C.CDLL(build.CALIB_LIB)
    for fn in (lib.nvfp4_calib_copy, lib.nvfp4_calib_read, lib.nvfp4_calib_mix):
        fn.argtypes = [C.c_void_p, C.c_void_p, C.c_int64, C.c_int32, C.c_void_p]
        fn.restype = C.c_int
    return lib


def kernel_source_hash() -> str:
    """SHA-256 of the quantize kernels' sources with comments and blank lines
    removed: any change to the code itself invalidates the stored counter
    summary, an edit of a comment does not."""
    import re
    h = hashlib.sha256()
    for rel in ("moe_swiglu_epilogue_amd/csrc/moe_nvfp4.hip",
                "moe_swiglu_epilogue_amd/csrc/nvfp4_device.hpp"):
        with open(os.path.join(ROOT, rel)) as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        lines = [re.sub(r"//.*$", "", l).rstrip() for l in text.splitlines()]
        h.update("\n".join(l for l in lines if l.strip()).encode())
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


class GpuStateSampler:
    """Samples the GPU's shader clock and board power from sysfs (read-only)
    every 5 ms in a background thread while a measurement runs,
    so that the result can be reported with the clock and power state it was
    taken at. Nothing is pinned or changed."""

    def __init__(self):
        import glob
        import threading
        dev = sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk"))
        self.base = os.path.dirname(dev[0]) if dev else None
        hw = sorted(glob.glob(os.path.join(self.base, "hwmon", "hwmon*"))) if self.base else []
        self.hwmon = hw[0] if hw else None
        self.samples = []
        self.timed = False
        self._stop = threading.Event()
        self._thread = threading.Thread(target=self._run, daemon=True)

    def _read(self, path):
        try:
            with open(path) as f:
                return f.read()
        except OSError:
            return None

    def _sample(self):
        out = {"timed": self.timed}
        t = self._read(os.path.join(self.base, "pp_dpm_sclk"))
        if t:
            cur = [l.split(":", 1)[1].strip(" *").lower().replace("mhz", "") for l in t.splitlines()
                   if l.endswith("*")]
            out["sclk_MHz"] = float(cur[0]) if cur and cur[0].replace(".", "").isdigit() else None
        if self.hwmon:
            pw = self._read(os.path.join(self.hwmon, "power1_input"))
            out["power_W"] = int(pw) / 1e6 if pw else None
        return out

    def _run(self):
        while not self._stop.wait(0.005):
            self.samples.append(self._sample())

    def __enter__(self):
        self.timed = False
        if self.base:
            self._thread.start()
        return self

    def mark_timed(self, on: bool):
        """Tag the following samples as taken inside (or outside) the timed
        region, and take one sample right at the boundary (the timed region
        of a short run can end before the 5 ms sampler fires): the sample at
        the start is tagged timed, the one at the end too."""
        if on:
            self.timed = True
        if self.base:
            self.samples.append(self._sample())
        if not on:
            self.timed = False

    def __exit__(self, *exc):
        self._stop.set()
        if self._thread.is_alive():
            self._thread.join()

    @staticmethod
    def _stats(v):
        v = sorted(v)
        return [round(v[0], 1), round(v[len(v) // 2], 1), round(v[-1], 1)] if v else None

    def report(self):
        if not self.base:
            return None
        rep = {}
        for label, want in (("timed", True), ("settle_and_warmup", False)):
            smp = [x for x in self.samples if x["timed"] == want]
            rep[label] = {
                "samples": len(smp),
                "sclk_MHz_min_median_max": self._stats([x["sclk_MHz"] for x in smp if x.get("sclk_MHz")]),
                "power_W_min_median_max": self._stats([x["power_W"] for x in smp if x.get("power_W")]),
            }
        mclk = self._read(os.path.join(self.base, "pp_dpm_mclk"))
        if mclk:
            rep["mclk"] = [l.split(":", 1)[1].strip(" *") for l in mclk.splitlines()
                           if l.endswith("*")]
        if self.hwmon:
            cap = self._read(os.path.join(self.hwmon, "power1_cap"))
            rep["power_cap_W"] = int(cap) / 1e6 if cap else None
            for lab in sorted(os.listdir(self.hwmon)):
                if lab.startswith("temp") and lab.endswith("_label"):
                    name = (self._read(os.path.join(self.hwmon, lab)) or "").strip()
                    val = self._read(os.path.join(self.hwmon, lab.replace("_label", "_input")))
                    if name and val:
                        rep.setdefault("temp_C_after", {})[name] = int(val) / 1e3
        return rep


def settle(fn, settle_ms):
    """Run fn back to back for settle_ms of wall time (untimed). Under
    sustained load the GPU's clocks need about 30 ms to reach their steady
    state, and they drop back after a fraction of a second idle; without
    this the first few milliseconds of any measurement run slower."""
    import torch
    t0 = time.perf_counter()
    while (time.perf_counter() - t0) * 1e3 < settle_ms:
        for _ in range(8):
            fn()
        torch.cuda.synchronize()


def time_launches(fn, steps, warmup, settle_ms=0.0, chunks=10, sampler=None):
    """Settle, warm up, then time `steps` back-to-back launches. Returns
    (wall seconds between two device synchronizations, device ms per launch
    from HIP events recorded on the launch stream around the whole region,
    per-launch ms of each of `chunks` equal runs of launches (events at the
    chunk boundaries))."""
    import torch
    settle(fn, settle_ms)
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    n_chunks = max(1, min(chunks, steps))
    bounds = [round(i * steps / n_chunks) for i in range(n_chunks + 1)]
    ev = [torch.cuda.Event(enable_timing=True) for _ in bounds]
    if sampler is not None:
        sampler.mark_timed(True)
    t0 = time.perf_counter()
    ev[0].record()
    for c in range(n_chunks):
        for _ in range(bounds[c + 1] - bounds[c]):
            fn()
        ev[c + 1].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    if sampler is not None:
        sampler.mark_timed(False)
    per = [ev[c].elapsed_time(ev[c + 1]) / (bounds[c + 1] - bounds[c]) for c in range(n_chunks)]
    return wall, ev[0].elapsed_time(ev[-1]) / steps, per


def pct(v, q):
    v = sorted(v)
    return v[min(len(v) - 1, max(0, int(round(q * (len(v) - 1)))))]


def measure(name, fn, nbytes, elems, steps, settle_ms, extra=None):
    """One secondary figure: kernel ms per launch and GB/s over `nbytes`."""
    _, ms, per = time_launches(fn, steps, 3, settle_ms)
    out = {"ms": round(ms, 4), "GB_s": round(nbytes / ms / 1e6, 1),
           "elements_per_s": round(elems / ms * 1e3, 1), "bytes_per_launch": int(nbytes),
           "ms_p10_p50_p90": [round(pct(per, q), 4) for q in (0.1, 0.5, 0.9)]}
    if extra:
        out.update(extra)
    print("[bench] %-34s %8.4f ms  %7.1f GB/s" % (name, ms, out["GB_s"]), file=sys.stderr, flush=True)
    return out


def graph_ms(fn, launches=50, replays=20):
    """Device ms per launch of `fn` captured `launches` times into one HIP
    graph and replayed `replays` times (events around the replays): what a
    launch costs without the host's enqueue work, for launch-bound shapes."""
    import torch
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for _ in range(3):
            fn()
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(launches):
            fn()
    g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(replays):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / (launches * replays)


def cpu_baseline(x, gpu_packed=None, gpu_scales=None, gpu_value=None):
    """The CPU oracle on the same prefill input: all host threads over the
    whole workload (median of 3), plus one thread over 16384 rows. The
    oracle's output of the last pass is compared byte for byte with the GPU's
    output of the last timed launch (the fused path's acceptance exempts
    codes whose scaled value lies within 1e-6 of a rounding boundary, so a
    handful of differing code bytes is expected; scale bytes differ only
    where an amax does)."""
    import numpy as np
    import oracle
    n_elem = x.shape[0] * (x.shape[1] // 2)
    threads = oracle.num_threads()
    times = []
    ref = None
    for _ in range(3):
        t = time.perf_counter()
        ref = oracle.swiglu_quantize(x)
        times.append(time.perf_counter() - t)
    med = statistics.median(times)
    oracle.set_num_threads(1)
    sub = x[:16384]
    t = time.perf_counter()
    oracle.swiglu_quantize(sub)
    one = time.perf_counter() - t
    oracle.set_num_threads(threads)
    one_elem = sub.shape[0] * (sub.shape[1] // 2)
    model = "unknown CPU"
    try:
        with open("/proc/cpuinfo") as f:
            model = next(l.split(":", 1)[1].strip() for l in f if l.startswith("model name"))
    except (OSError, StopIteration):
        pass
    out = {
        "value": round(n_elem * BYTES_PER_ELEM / med / 1e9, 3),
        "unit": "GB/s",
        "cores": threads,
        "kind": "oracle",
        "sample": "full prefill workload 65536x6144 BF16, median of 3 passes on %d threads "
                  "(%.2f s each); 1 thread over 16384 rows: %.3f GB/s; host CPU: %s"
                  % (threads, med, one_elem * BYTES_PER_ELEM / one / 1e9, model),
        "elements_per_s": round(n_elem / med, 1),
    }
    if gpu_value is not None:
        out["gpu_over_cpu"] = round(gpu_value / out["value"], 1)
    if gpu_packed is not None:
        gp = gpu_packed.cpu().numpy()
        gsc = gpu_scales.cpu().numpy()
        out["checked_against_gpu"] = {
            "packed_bytes": int(gp.size), "packed_bytes_differ": int(np.count_nonzero(gp != ref[0])),
            "scale_bytes": int(gsc.size), "scale_bytes_differ": int(np.count_nonzero(gsc != ref[1]))}
    return out


kern_ms_headline = []


def secondary_figures(M, W, x, packed, scales, args, dev, oc):
    """Other kernels and the other workload shapes (not the headline). Each
    workload's last timed output goes through oc (OutputCheck)."""
    import numpy as np
    import torch
    sec = {}
    st, ms = args.secondary_steps, args.settle_ms
    want = set(args.only.split(",")) if args.only else set(SECONDARY)
    # the other entry points on the prefill tensor
    if "nvfp4_quantize" in want:
        xq = x.view(torch.int16)[:, :INTER].contiguous().view(torch.bfloat16)
        pq, sq = torch.empty_like(packed), torch.empty_like(scales)
        sec["nvfp4_quantize"] = measure(
            "nvfp4_quantize prefill-shaped", lambda: M.nvfp4_quantize(xq, packed=pq, scales=sq),
            ROWS * INTER * 2.5625, ROWS * INTER, st, ms, {"shape": [ROWS, INTER]})
        oc.check("nvfp4_quantize.packed", pq)
        oc.check("nvfp4_quantize.scales", sq)
        del xq, pq, sq
    if "nvfp4_dequantize" in want:
        out = torch.empty((ROWS, INTER), dtype=torch.float32, device=dev)
        sec["nvfp4_dequantize"] = measure(
            "nvfp4_dequantize prefill-shaped",
            lambda: M.nvfp4_dequantize(packed, scales, out=out),
            ROWS * INTER * 4.5625, ROWS * INTER, st, ms, {"shape": [ROWS, INTER]})
        oc.check("nvfp4_dequantize.out", out)
        del out
    if "global_scale" in want:
        gsb = torch.empty(1, dtype=torch.float32, device=dev)
        sec["swiglu_nvfp4_global_scale"] = measure(
            "swiglu_nvfp4_global_scale prefill", lambda: M.swiglu_nvfp4_global_scale(x, gs=gsb),
            ROWS * INTER * 4.0, ROWS * INTER, st, ms,
            {"shape": [ROWS, 2 * INTER], "note": "per-tensor amax pre-pass; 3 launches"})
        oc.check("global_scale.gs", gsb)
    if "two_pass" in want:
        # the ablation that prices the fusion: SwiGLU to compact BF16 (4 B read,
        # 2 B written per element), then the standalone quantize of it
        # (2 + 0.5625 B): 8.5625 B per element for the same outputs
        yb = torch.empty((ROWS, INTER), dtype=torch.bfloat16, device=dev)
        pq, sq = torch.empty_like(packed), torch.empty_like(scales)
        sec["swiglu_bf16"] = measure(
            "swiglu_bf16 prefill", lambda: M.swiglu_bf16(x, out=yb), ROWS * INTER * 6.0,
            ROWS * INTER, st, ms, {"shape": [ROWS, 2 * INTER]})
        oc.check("swiglu_bf16.out", yb)

        def two_pass():
            M.swiglu_bf16(x, out=yb)
            M.nvfp4_quantize(yb, packed=pq, scales=sq)
        tp = measure("two-pass (swiglu_bf16 + nvfp4_quantize)", two_pass,
                     ROWS * INTER * 8.5625, ROWS * INTER, st, ms,
                     {"note": "GB_s over the two passes' own 8.5625 B per element"})
        tp["fused_speedup"] = round(tp["ms"] / kern_ms_headline[0], 3) if kern_ms_headline else None
        sec["two_pass"] = tp
        oc.check("two_pass.packed", pq)
        oc.check("two_pass.scales", sq)
        del yb, pq, sq
    # in-repo calibration kernels over the same 805 MB input: HBM ceilings
    nbytes = x.numel() * 2
    stream = torch.cuda.current_stream().cuda_stream
    if "calib_read" in want or "calib_copy" in want or "calib_mix" in want:
        calib = load_calib()
    if "calib_read" in want:
        scratch = torch.empty(max(CALIB_READ_BLOCKS) * 16, dtype=torch.uint8, device=dev)
        best = None
        for blocks in CALIB_READ_BLOCKS:
            r = measure("calib read ceiling, %d workgroups" % blocks,
                        lambda: checked(calib.nvfp4_calib_read(
                            x.data_ptr(), scratch.data_ptr(), nbytes, blocks, stream)),
                        nbytes, nbytes // 2, st, ms, {"workgroups": blocks})
            best = r if best is None or r["GB_s"] > best["GB_s"] else best
        sec["calib_read_ceiling"] = best
        del scratch
    if "calib_copy" in want:
        dst = torch.empty_like(x)
        best = None
        for blocks in CALIB_COPY_BLOCKS:
            r = measure("calib copy ceiling, %d workgroups" % blocks,
                        lambda: checked(calib.nvfp4_calib_copy(
                            x.data_ptr(), dst.data_ptr(), nbytes, blocks, stream)),
                        2 * nbytes, nbytes // 2, st, ms, {"workgroups": blocks})
            best = r if best is None or r["GB_s"] > best["GB_s"] else best
        sec["calib_copy_ceiling"] = best
        del dst
    if "calib_mix" in want:
        # the fused kernel's own mix: 576 bytes written per 4 KB read, no compute
        mix_out = torch.empty(nbytes // 4096 * 576, dtype=torch.uint8, device=dev)
        best = None
        for lds in CALIB_MIX_LDS:
            r = measure("calib traffic-mix ceiling, %d B LDS per workgroup" % lds,
                        lambda: checked(calib.nvfp4_calib_mix(
                            x.data_ptr(), mix_out.data_ptr(), nbytes, lds, stream)),
                        nbytes + mix_out.numel(), nbytes // 2, st, ms, {"lds_bytes": lds})
            best = r if best is None or r["GB_s"] > best["GB_s"] else best
        sec["calib_mix_ceiling"] = best
        del mix_out

    if "ragged" in want:
        # ragged grouped MoE: 256 experts (Zipf 1.1), 131072 x 4096, per-expert
        # global scales from the on-device pre-pass, then quantize and dequantize
        print("[bench] generating ragged 256-expert workload", file=sys.stderr, flush=True)
        w = W.ragged()
        rr, ri = w.rows, w.out_cols
        xr = torch.from_numpy(w.x.view(np.int16)).to(dev).view(torch.bfloat16)
        offr = torch.from_numpy(w.offsets).to(dev)
        ragged = {"shape": [rr, 2 * ri], "experts": 256, "input_sha256": W.sha256(w.x)}
        del w
        gsr = torch.empty(256, dtype=torch.float32, device=dev)
        pr = torch.empty((rr, ri // 2), dtype=torch.uint8, device=dev)
        sr = torch.empty((rr, ri // 16), dtype=torch.uint8, device=dev)
        ragged["global_scale"] = measure(
            "ragged swiglu_nvfp4_global_scale",
            lambda: M.swiglu_nvfp4_global_scale(xr, offr, gs=gsr), rr * ri * 4.0, rr * ri, st, ms)
        oc.check("ragged.gs", gsr)
        ragged["quantize"] = measure(
            "ragged swiglu_nvfp4_quantize",
            lambda: M.swiglu_nvfp4_quantize(xr, gsr, offr, packed=pr, scales=sr),
            rr * ri * BYTES_PER_ELEM, rr * ri, st, ms)
        oc.check("ragged.packed", pr)
        oc.check("ragged.scales", sr)
        del xr
        outr = torch.empty((rr, ri), dtype=torch.float32, device=dev)
        ragged["dequantize"] = measure(
            "ragged nvfp4_dequantize", lambda: M.nvfp4_dequantize(pr, sr, gsr, offr, out=outr),
            rr * ri * 4.5625, rr * ri, st, ms)
        oc.check("ragged.dequantize", outr)
        sec["ragged_256_experts"] = ragged
        del outr, pr, sr, gsr, offr

    if "decode" in want:
        # decode-shaped 8192 x 4096: the 67 MB input fits the 256 MB Infinity
        # Cache, so launches rotate over 8 distinct input/output sets (537 MB)
        print("[bench] generating decode-shaped workload", file=sys.stderr, flush=True)
        w = W.decode()
        dr, di = w.rows, w.out_cols
        base = torch.from_numpy(w.x.view(np.int16)).to(dev).view(torch.bfloat16)
        decode_sha = W.sha256(w.x)
        del w
        sets = [(base.clone(), torch.empty((dr, di // 2), dtype=torch.uint8, device=dev),
                 torch.empty((dr, di // 16), dtype=torch.uint8, device=dev)) for _ in range(8)]
        del base
        k = [0]

        def rotating():
            xi, pi, si = sets[k[0] % 8]
            k[0] += 1
            M.swiglu_nvfp4_quantize(xi, packed=pi, scales=si)
        dec = measure(
            "decode-shaped swiglu_nvfp4_quantize", rotating, dr * di * BYTES_PER_ELEM, dr * di,
            max(st, 80), ms, {"shape": [dr, 2 * di], "note": "8 rotating input/output sets",
                              "input_sha256": decode_sha})
        dec["graph_ms"] = round(graph_ms(rotating, launches=80, replays=10), 5)
        # the 8 sets hold copies of one input, so every set's output must match
        oc.check("decode.packed", *[o[1] for o in sets])
        oc.check("decode.scales", *[o[2] for o in sets])
        # the HBM ceilings at this size, over the same 8 rotating inputs: the
        # read kernel and the traffic-mix kernel (the fused kernel's 4 KB read
        # and 576 B written per wave tile, without compute)
        calib = load_calib()
        stream = torch.cuda.current_stream().cuda_stream
        nb = dr * 2 * di * 2
        scratch = torch.empty(8192 * 16, dtype=torch.uint8, device=dev)
        mix_out = [torch.empty(nb // 4096 * 576, dtype=torch.uint8, device=dev) for _ in range(8)]

        def read_rot(blocks):
            xi = sets[k[0] % 8][0]
            k[0] += 1
            checked(calib.nvfp4_calib_read(xi.data_ptr(), scratch.data_ptr(), nb, blocks, stream))

        def mix_rot():
            i = k[0] % 8
            k[0] += 1
            checked(calib.nvfp4_calib_mix(sets[i][0].data_ptr(), mix_out[i].data_ptr(), nb, 0,
                                          stream))
        best = None
        for blocks in (1024, 1536, 4096):
            r = measure("decode-size read ceiling, %d workgroups" % blocks,
                        lambda: read_rot(blocks), nb, nb // 2, max(st, 80), ms, {"workgroups": blocks})
            best = r if best is None or r["GB_s"] > best["GB_s"] else best
        mix = measure("decode-size traffic-mix ceiling", mix_rot, nb + nb // 4096 * 576, nb // 2,
                      max(st, 80), ms)
        dec["read_ceiling"] = best
        dec["mix_ceiling"] = mix
        dec["frac_of_mix_ceiling"] = round(dec["GB_s"] / mix["GB_s"], 4)
        dec["frac_of_read_ceiling"] = round(dec["GB_s"] / best["GB_s"], 4)
        sec["decode_shaped"] = dec
        del sets, scratch, mix_out
    if "small" in want:
        # the two small shapes: 128 x 256 standalone (84 KB moved) and
        # 512 x 4096 fused (4.8 MB). Both live in the Infinity Cache and a
        # launch is a few microseconds, so these are back-to-back launch
        # rates, not HBM figures.
        w = W.standalone()
        xs = torch.from_numpy(w.x.view(np.int16)).to(dev).view(torch.bfloat16)
        ps = torch.empty((w.rows, w.out_cols // 2), dtype=torch.uint8, device=dev)
        ss = torch.empty((w.rows, w.out_cols // 16), dtype=torch.uint8, device=dev)
        def small(name, fn, nbytes, elems, shape, sha):
            r = measure(name, fn, nbytes, elems, max(st, 200), ms,
                        {"shape": shape, "note": "cache-resident, launch-bound; ms is the eager "
                         "launch rate through the Python binding, graph_ms the device time per "
                         "launch inside a HIP graph of 50 launches", "input_sha256": sha})
            gm = graph_ms(fn)
            r["graph_ms"] = round(gm, 5)
            r["graph_elements_per_s"] = round(elems / gm * 1e3, 1)
            r["graph_GB_s"] = round(nbytes / gm / 1e6, 1)
            return r
        sec["small_standalone"] = small(
            "standalone 128x256 nvfp4_quantize", lambda: M.nvfp4_quantize(xs, packed=ps, scales=ss),
            w.rows * w.out_cols * 2.5625, w.rows * w.out_cols, [w.rows, w.out_cols],
            W.sha256(w.x))
        oc.check("small_standalone.packed", ps)
        oc.check("small_standalone.scales", ss)
        w = W.fused_small()
        xf = torch.from_numpy(w.x.view(np.int16)).to(dev).view(torch.bfloat16)
        pf = torch.empty((w.rows, w.out_cols // 2), dtype=torch.uint8, device=dev)
        sf = torch.empty((w.rows, w.out_cols // 16), dtype=torch.uint8, device=dev)
        sec["small_fused"] = small(
            "fused 512x4096 swiglu_nvfp4_quantize",
            lambda: M.swiglu_nvfp4_quantize(xf, packed=pf, scales=sf),
            w.rows * w.out_cols * BYTES_PER_ELEM, w.rows * w.out_cols, [w.rows, 2 * w.out_cols],
            W.sha256(w.x))
        oc.check("small_fused.packed", pf)
        oc.check("small_fused.scales", sf)
        del xs, ps, ss, xf, pf, sf
    if "kv" in want:
        # paged KV-cache write and read: 65536 tokens x 8 heads x 128 into a
        # 131072-slot NVFP4 cache (1% padding tokens, slot -1). Bytes: the
        # BF16 input of every token plus the codes and scales of the tokens
        # written; the read moves the cache bytes of the valid slots plus
        # the FP32 output of every row
        w = W.kv_cache()
        cols = w.heads * w.head_dim
        valid = int(((w.slots >= 0) & (w.slots < w.num_slots)).sum())
        xk = torch.from_numpy(w.x.view(np.int16)).to(dev).view(torch.bfloat16)
        sk = torch.from_numpy(w.slots).to(dev)
        pk = torch.zeros((w.num_slots, cols // 2), dtype=torch.uint8, device=dev)
        sck = torch.zeros((w.num_slots, cols // 16), dtype=torch.uint8, device=dev)
        n = w.x.shape[0]
        kv = {"shape": {"tokens": n, "heads": w.heads, "head_dim": w.head_dim,
                        "num_slots": w.num_slots, "valid_tokens": valid}}
        kv["write"] = measure("paged KV write nvfp4_quantize_paged",
                              lambda: M.nvfp4_quantize_paged(xk, sk, pk, sck),
                              n * cols * 2 + valid * cols * 0.5625, n * cols, st, ms)
        oc.check("kv_write.packed_cache", pk)
        oc.check("kv_write.scales_cache", sck)
        outk = torch.empty((n, cols), dtype=torch.float32, device=dev)
        kv["read"] = measure("paged KV read nvfp4_dequantize_paged",
                             lambda: M.nvfp4_dequantize_paged(pk, sck, sk, out=outk),
                             valid * cols * 0.5625 + n * cols * 4, n * cols, st, ms)
        oc.check("kv_read.out", outk)
        sec["kv_cache_paged"] = kv
        del xk, sk, pk, sck, outk
    if "gemm" in want:
        sec["moe_l1_gemm"] = gemm_figures(M, W, args)
    return sec


def gemm_figures(M, W, args):
    """The MoE L1 grouped GEMM with the fused SwiGLU + NVFP4 epilogue against
    the same GEMM core with a plain BF16 store (the cost of the fused
    epilogue: `epilogue_cost`), the unfused flow on that core (BF16 L1 output,
    then swiglu_nvfp4_quantize), and hipBLASLt's plain BF16 GEMM
    (torch.matmul per expert) for context: 32768 token rows, hidden 7168,
    I = 3072, 8 experts."""
    import numpy as np
    import torch
    print("[bench] generating MoE L1 GEMM workload", file=sys.stderr, flush=True)
    g = W.moe_gemm()
    T, H = g.x.shape
    N = g.w1.shape[1]
    inter = N // 2
    E = g.w1.shape[0]
    dev = torch.device("cuda:0")
    x = torch.from_numpy(g.x.view(np.int16)).to(dev).view(torch.bfloat16)
    w = torch.from_numpy(g.w1.view(np.int16)).to(dev).view(torch.bfloat16)
    off = torch.from_numpy(g.offsets).to(dev)
    offs = g.offsets.tolist()
    del g
    flop = 2.0 * T * H * N
    p = torch.empty((T, inter // 2), dtype=torch.uint8, device=dev)
    sc = torch.empty((T, inter // 16), dtype=torch.uint8, device=dev)
    yb = torch.empty((T, N), dtype=torch.bfloat16, device=dev)
    outs = [yb[offs[e]:offs[e + 1]] for e in range(E)]
    wt = [w[e].t() for e in range(E)]

    def fused():
        M.moe_l1_gemm_swiglu_nvfp4(x, w, off, packed=p, scales=sc)

    def bf16_output():
        M.moe_l1_gemm_bf16(x, w, off, out=yb)

    def unfused():
        M.moe_l1_gemm_bf16(x, w, off, out=yb)
        M.swiglu_nvfp4_quantize(yb, packed=p, scales=sc)

    def library():
        for e in range(E):
            torch.matmul(x[offs[e]:offs[e + 1]], wt[e], out=outs[e])

    res = {"shape": {"tokens": T, "hidden": H, "inter": inter, "experts": E},
           "flop_per_launch": flop}
    steps = max(5, args.secondary_steps // 4)
    for name, fn in (("fused", fused), ("bf16_output", bf16_output), ("unfused", unfused),
                     ("hipblaslt_bf16_gemm_only", library)):
        _, ms, per = time_launches(fn, steps, 2, args.settle_ms)
        res[name] = {"ms": round(ms, 4), "TFLOP_s": round(flop / ms / 1e9, 1),
                     "frac_of_bf16_peak": round(flop / ms / 1e9 / PEAK_BF16_TFLOPS, 4),
                     "ms_p10_p50_p90": [round(pct(per, q), 4) for q in (0.1, 0.5, 0.9)]}
        print("[bench] MoE L1 GEMM %-26s %8.4f ms  %7.1f TFLOP/s" % (name, ms, flop / ms / 1e9),
              file=sys.stderr, flush=True)
    res["fusion_speedup"] = round(res["unfused"]["ms"] / res["fused"]["ms"], 4)
    res["epilogue_cost"] = round(res["fused"]["ms"] / res["bf16_output"]["ms"] - 1.0, 4)
    return res


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--settle-ms", type=float, default=300.0,
                    help="untimed back-to-back launches before each warmup (clock settling)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-secondary", action="store_true")
    ap.add_argument("--secondary-steps", type=int, default=40)
    ap.add_argument("--only", default="",
                    help="comma list of secondary items to run (default all): " + ",".join(SECONDARY))
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

    print("[bench] timing %d steps after %d warmup (%.0f ms settle)"
          % (args.steps, args.warmup, args.settle_ms), file=sys.stderr, flush=True)
    with GpuStateSampler() as sampler:
        wall, kern_ms, per = time_launches(step, args.steps, args.warmup, args.settle_ms,
                                           sampler=sampler)
    gpu_state = sampler.report()
    kern_ms_headline.append(kern_ms)
    ms_per_step = wall * 1e3 / args.steps
    value = ALG_BYTES / (wall / args.steps) / 1e9
    achieved = ALG_BYTES / (kern_ms / 1e3) / 1e9
    print("[bench] fused prefill: %.4f ms/step wall, %.4f ms/launch events, %.1f GB/s"
          % (ms_per_step, kern_ms, value), file=sys.stderr, flush=True)
    # the timed launches' output, before any other measurement reuses the buffers
    output_sha = {"packed": W.sha256(packed.cpu().numpy()), "scales": W.sha256(scales.cpu().numpy())}
    oc = OutputCheck()
    oc.check("prefill.packed", packed)
    oc.check("prefill.scales", scales)

    secondary = None
    if not args.no_secondary:
        secondary = secondary_figures(M, W, x, packed, scales, args, dev, oc)
        if "calib_read_ceiling" in secondary:
            r = secondary["calib_read_ceiling"]["GB_s"]
            secondary["fused_frac_of_read_ceiling"] = round(achieved / r, 4)
        if "calib_copy_ceiling" in secondary:
            c = secondary["calib_copy_ceiling"]["GB_s"]
            secondary["fused_frac_of_copy_ceiling"] = round(achieved / c, 4)
        if "calib_mix_ceiling" in secondary:
            c = secondary["calib_mix_ceiling"]["GB_s"]
            secondary["fused_frac_of_mix_ceiling"] = round(achieved / c, 4)

    cpu = None
    if not args.no_cpu_baseline:
        print("[bench] cpu baseline (oracle on host cores)", file=sys.stderr, flush=True)
        cpu = cpu_baseline(w.x, packed, scales, value)

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
                   "alg_bytes_per_step": ALG_BYTES, "parallelism": "single GPU",
                   "settle_ms": args.settle_ms, "input_sha256": W.sha256(w.x)},
        "pct_of_peak": round(100.0 * value / PEAK_HBM_GBS, 2),
        "elements_per_s": round(ROWS * INTER / (wall / args.steps), 1),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4),
                     "traffic": measured_traffic(),
                     "kernel": "quantize_tiles_kernel<FusedBlock, true>",
                     "kernel_ms": round(kern_ms, 5),
                     "kernel_ms_p10_p50_p90": [round(pct(per, q), 5) for q in (0.1, 0.5, 0.9)]},
        "output_sha256": output_sha,
        "outputs_match_oracle": oc.report(),
        "cpu_baseline": cpu,
        "gpu_state": gpu_state,
        "secondary": secondary,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
