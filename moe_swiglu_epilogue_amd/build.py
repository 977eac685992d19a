"""Build libmoe_nvfp4.so (HIP kernels for gfx950 + the C ABI), the
bandwidth-calibration library libnvfp4_calib.so and the quotient-check
library libnvfp4_divcheck.so with hipcc.

The library is built in-tree, next to this file, so that it travels with the
source tree. Run ``python -m moe_swiglu_epilogue_amd.build``.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRC = os.path.join(HERE, "csrc", "moe_nvfp4.hip")
GEMM_SRC = os.path.join(HERE, "csrc", "moe_gemm.hip")
LIB = os.path.join(HERE, "libmoe_nvfp4.so")
CALIB_SRC = os.path.join(HERE, "csrc", "calib.hip")
CALIB_LIB = os.path.join(HERE, "libnvfp4_calib.so")
DIVCHECK_SRC = os.path.join(HERE, "csrc", "divcheck.hip")
DIVCHECK_LIB = os.path.join(HERE, "libnvfp4_divcheck.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    # IEEE binary32 semantics: no FMA contraction, correctly rounded '/'.
    "-ffp-contract=off", "-fhip-fp32-correctly-rounded-divide-sqrt",
    # no packed FP32 (v_pk_*_f32) instructions in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # atomics stay as written: the tile queue's one-lane LDS claim must not be
    # rewritten into a wave-wide form that waits for its result at once
    "-mllvm", "-amdgpu-atomic-optimizer-strategy=None",
    "-Wall",
]


def build(verbose: bool = False) -> str:
    """Build the three libraries; return the path of libmoe_nvfp4.so."""
    _build_one([CALIB_SRC], CALIB_LIB, verbose)
    _build_one([DIVCHECK_SRC], DIVCHECK_LIB, verbose)
    return _build_one([SRC, GEMM_SRC], LIB, verbose)


def _build_one(srcs, lib: str, verbose: bool) -> str:
    tmp = lib + ".tmp%d" % os.getpid()
    cmd = [HIPCC, *FLAGS, "-I", os.path.join(ROOT, "include"), *srcs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass does not know the packed-fp32 feature and says so; harmless
    err = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + err)
    if verbose and err.strip():
        print(err)
    os.replace(tmp, lib)
    return lib


def asm(out_path: str, src: str = SRC) -> None:
    """Write the gfx950 assembly of one source's kernels (for inspection)."""
    cmd = [HIPCC, *[f for f in FLAGS if f not in ("-shared", "-fPIC")], "-I",
           os.path.join(ROOT, "include"), "--cuda-device-only", "-S", src, "-o", out_path]
    subprocess.run(cmd, check=True, capture_output=True)


if __name__ == "__main__":
    print(build(verbose=True))
