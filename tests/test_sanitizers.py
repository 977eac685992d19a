"""CPU-only sanitizer runs.

* The oracle built with AddressSanitizer and UndefinedBehaviorSanitizer
  (gcc), driven by a small C program through every entry point on small,
  empty and edge-sized inputs: no sanitizer report.
* The library's host code built with AddressSanitizer and
  UndefinedBehaviorSanitizer (hipcc, host pass only; the device code is
  built as usual), driven through every C-ABI
  entry point with the argument errors its validation must catch. Every
  call is rejected before any HIP call (none reaches a launch), so no GPU
  is needed: no sanitizer report.
"""
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

ORACLE_DRIVER = r"""
#include <stdio.h>
#include <stdlib.h>
#include <string.h>
#include "nvfp4_oracle.h"
static uint32_t st = 12345u;
static float rnd(void) { st = st * 1664525u + 1013904223u; return ((st >> 8) / 16777216.0f - 0.5f) * 8.0f; }
static uint16_t bf(float f) { uint32_t u; memcpy(&u, &f, 4); return (uint16_t)(u >> 16); }
int main(void) {
    int shapes[][2] = {{0, 16}, {1, 16}, {3, 48}, {5, 256}, {2, 1040}};
    for (unsigned s = 0; s < sizeof shapes / sizeof shapes[0]; ++s) {
        int rows = shapes[s][0], cols = shapes[s][1], inter = cols;
        size_t n = (size_t)rows * cols;
        float *x = malloc((n + 1) * 4), *y = malloc((n + 1) * 4), *dq = malloc((n + 1) * 4);
        float *bsf = malloc((n / 16 + 1) * 4), *v = malloc((n + 1) * 4), *gs = malloc((rows + 1) * 4);
        uint16_t *xb = malloc((n + 1) * 2), *gu = malloc((2 * n + 1) * 2), *yb = malloc((n + 1) * 2);
        uint8_t *p = malloc(n / 2 + 1), *sc = malloc(n / 16 + 1);
        float *acc = malloc((2 * n + 1) * 4);
        for (size_t i = 0; i < n; ++i) { x[i] = rnd(); xb[i] = bf(x[i]); }
        for (size_t i = 0; i < 2 * n; ++i) { gu[i] = bf(rnd()); acc[i] = rnd(); }
        for (int r = 0; r < rows; ++r) gs[r] = 0.5f + r;
        if (oracle_quantize_f32_rows(x, rows, cols, cols, gs, p, sc, bsf, v)) return 2;
        if (oracle_quantize_bf16_rows(xb, rows, cols, cols, NULL, p, sc)) return 3;
        if (oracle_dequantize_rows(p, sc, rows, cols, gs, dq)) return 4;
        if (oracle_swiglu_rows(gu, rows, inter, 2 * inter, y)) return 5;
        if (oracle_swiglu_quantize_rows(gu, rows, inter, 2 * inter, gs, p, sc, y, bsf, v)) return 6;
        if (oracle_swiglu_bf16_rows(gu, rows, inter, 2 * inter, yb)) return 7;
        if (oracle_swiglu_f32_rows(acc, rows, inter, 2 * inter, y)) return 8;
        if (oracle_f32_to_bf16_array(x, (int64_t)n, yb)) return 9;
        int32_t off[4] = {0, rows / 2, rows / 2, rows};
        float am[3];
        if (oracle_group_amax(x, rows, cols, off, 3, am)) return 10;
        free(x); free(y); free(dq); free(bsf); free(v); free(gs); free(xb); free(gu); free(yb);
        free(p); free(sc); free(acc);
    }
    for (int c = 0; c < 256; ++c) (void)oracle_fp8_e4m3_encode(oracle_fp8_e4m3_decode((uint8_t)c));
    for (int h = -1; h <= 13; ++h) (void)oracle_e2m1_index(h);
    /* argument errors are reported, not crashed on */
    if (!oracle_quantize_f32_rows(NULL, 2, 16, 16, NULL, NULL, NULL, NULL, NULL)) return 11;
    if (!oracle_swiglu_rows(NULL, 2, 12, 24, NULL)) return 12;
    puts("oracle sanitizer run ok");
    return 0;
}
"""

HOST_DRIVER = r"""
#include <stdio.h>
#include <stdint.h>
#include "moe_nvfp4.h"
#define A ((void *)0x10000)
#define CHECK(e) do { if (!(e)) { printf("failed check at driver line %d\n", __LINE__); ++bad; } } while (0)
int main(void) {
    int bad = 0;
    CHECK(nvfp4_quantize(A, -1, 32, 32, NULL, NULL, 0, A, A, NULL) == NVFP4_ERROR_INVALID_VALUE);
    CHECK(nvfp4_quantize(A, 4, 24, 24, NULL, NULL, 0, A, A, NULL) == NVFP4_ERROR_UNSUPPORTED_SHAPE);
    CHECK(nvfp4_quantize((const uint16_t *)((char *)A + 2), 4, 32, 32, NULL, NULL, 0, A, A, NULL) == NVFP4_ERROR_MISALIGNED);
    CHECK(swiglu_nvfp4_quantize(A, 4, 32, 63, NULL, NULL, 0, A, A, NULL, NULL) == NVFP4_ERROR_INVALID_VALUE);
    CHECK(swiglu_nvfp4_quantize(A, 4, 32, 64, NULL, A, 0, A, A, NULL, NULL) == NVFP4_ERROR_INVALID_VALUE);
    CHECK(nvfp4_quantize(A, 4, 32, 16, NULL, NULL, 0, A, A, NULL) == NVFP4_ERROR_INVALID_VALUE);
    CHECK(nvfp4_quantize(A, 4, 32, 32, NULL, A, 0, A, A, NULL) == NVFP4_ERROR_INVALID_VALUE);
    CHECK(nvfp4_quantize(A, 4, 32, 32, NULL, NULL, 0, (uint8_t *)A + 4, A, NULL) == NVFP4_ERROR_MISALIGNED);
    CHECK(nvfp4_quantize(A, (int64_t)1 << 40, 32, 32, NULL, NULL, 0, A, A, NULL) == NVFP4_ERROR_UNSUPPORTED_SHAPE);
    CHECK(nvfp4_quantize(A, 4, INT64_MAX - 15, INT64_MAX, NULL, NULL, 0, A, A, NULL) != NVFP4_SUCCESS);
    CHECK(swiglu_nvfp4_quantize(A, 4, 32, 64, NULL, NULL, 0, A, A, (float *)A + 1, NULL) == NVFP4_ERROR_MISALIGNED);
    CHECK(nvfp4_dequantize(A, A, 4, 8, NULL, NULL, 0, A, NULL) == NVFP4_ERROR_UNSUPPORTED_SHAPE);
    CHECK(nvfp4_dequantize(A, NULL, 4, 32, NULL, NULL, 0, A, NULL) == NVFP4_ERROR_INVALID_VALUE);
    CHECK(nvfp4_global_scale(A, 4, 32, 32, A, 1025, NULL, A, NULL) == NVFP4_ERROR_UNSUPPORTED_SHAPE);
    CHECK(swiglu_nvfp4_global_scale(A, 4, 32, 64, NULL, 0, NULL, NULL, NULL) == NVFP4_ERROR_INVALID_VALUE);
    CHECK(swiglu_bf16(A, 4, 32, 64, (uint16_t *)((char *)A + 8), 32, NULL) == NVFP4_ERROR_MISALIGNED);
    CHECK(moe_l1_gemm_swiglu_nvfp4(A, A, 4, 96, 128, 96, 96, NULL, 0, NULL, A, A, NULL, NULL) == NVFP4_ERROR_UNSUPPORTED_SHAPE);
    CHECK(moe_l1_gemm_bf16(A, A, 4, 64, 256, 64, 64, A, 513, A, 256, NULL) == NVFP4_ERROR_UNSUPPORTED_SHAPE);
    CHECK(moe_l1_gemm_bf16(A, A, 4, 64, 256, 64, 32, A, 1, A, 256, NULL) == NVFP4_ERROR_INVALID_VALUE);
    CHECK(moe_l1_gemm_bf16(A, A, 4, 64, 200, 64, 64, A, 1, A, 256, NULL) == NVFP4_ERROR_UNSUPPORTED_SHAPE);
    CHECK(moe_l1_gemm_swiglu_nvfp4(A, A, 4, 64, 128, 64, 64, A, 1, NULL, (uint8_t *)A + 4, A, NULL, NULL) == NVFP4_ERROR_MISALIGNED);
    CHECK(moe_l1_gemm_swiglu_nvfp4(A, A, 4, 64, 128, 64, 64, A, 1, NULL, A, NULL, NULL, NULL) == NVFP4_ERROR_INVALID_VALUE);
    CHECK(moe_l1_gemm_bf16(A, A, 4, 64, 256, 64, INT64_MAX - 7, A, 1, A, 256, NULL) == NVFP4_ERROR_UNSUPPORTED_SHAPE);
    CHECK(moe_l1_gemm_bf16(A, A, 4, 64, 256, INT64_MAX - 7, 64, NULL, 0, A, 256, NULL) == NVFP4_ERROR_UNSUPPORTED_SHAPE);
    CHECK(moe_l1_gemm_bf16(A, A, 4, 64, 256, 64, 64, NULL, 0, A, INT64_MAX - 7, NULL) == NVFP4_ERROR_INVALID_VALUE);
    CHECK(moe_l1_gemm_swiglu_nvfp4(A, A, 4, 64, INT64_MAX / 2 + 1, 64, 64, NULL, 0, NULL, A, A, NULL, NULL) == NVFP4_ERROR_INVALID_VALUE);
    CHECK(swiglu_bf16(A, 4, 32, 64, A, INT64_MAX - 7, NULL) == NVFP4_ERROR_INVALID_VALUE);
    CHECK(swiglu_nvfp4_global_scale(A, 4, 32, INT64_MAX - 7, NULL, 0, NULL, A, NULL) == NVFP4_ERROR_INVALID_VALUE);
    CHECK(nvfp4_global_scale(A, 4, 32, INT64_MAX - 7, NULL, 0, NULL, A, NULL) == NVFP4_ERROR_INVALID_VALUE);
    for (int s = 0; s < 7; ++s) CHECK(nvfp4_status_string((nvfp4_status_t)s) != NULL);
    CHECK(nvfp4_quantize(NULL, 0, 32, 32, NULL, NULL, 0, NULL, NULL, NULL) == NVFP4_SUCCESS);
    printf("host sanitizer run: %d failures\n", bad);
    return bad != 0;
}
"""


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, (cmd[0], r.returncode, r.stdout[-2000:], r.stderr[-4000:])
    return r


@pytest.mark.slow
def test_oracle_under_asan_ubsan(tmp_path):
    src = os.path.join(ROOT, "oracle", "nvfp4_oracle.c")
    drv = tmp_path / "drv.c"
    drv.write_text(ORACLE_DRIVER)
    exe = tmp_path / "oracle_san"
    _run(["gcc", "-std=c11", "-O1", "-g", "-fopenmp", "-ffp-contract=off",
          "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
          "-I", os.path.join(ROOT, "oracle"), str(drv), src, "-o", str(exe), "-lm"])
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1", OMP_NUM_THREADS="2")
    r = _run([str(exe)], env=env)
    assert "oracle sanitizer run ok" in r.stdout
    assert "runtime error" not in r.stderr


@pytest.mark.slow
def test_host_library_under_asan_ubsan(tmp_path):
    from moe_swiglu_epilogue_amd import build as B
    rocm = os.path.dirname(os.path.dirname(B.HIPCC))
    san = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]
    lib = tmp_path / "libmoe_nvfp4_san.so"
    flags = [f for f in B.FLAGS if f != "-Wall"]
    host_san = [a for f in san for a in ("-Xarch_host", f)]
    _run([B.HIPCC, *flags, *host_san, "-I", os.path.join(ROOT, "include"),
          B.SRC, B.GEMM_SRC, "-o", str(lib)])
    syms = _run(["nm", "-D", str(lib)]).stdout
    assert "__asan_report" in syms and "__ubsan_handle" in syms, "host code not instrumented"
    drv = tmp_path / "drv.c"
    drv.write_text(HOST_DRIVER)
    exe = tmp_path / "host_san"
    # The driver is plain C, as a C caller of the library would be; it is
    # linked by the same clang whose sanitizer runtime the library expects.
    _run([os.path.join(rocm, "llvm", "bin", "clang"), "-std=c11", *san,
          "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(rocm, "include"),
          "-I", os.path.join(ROOT, "include"), str(drv), str(lib),
          "-L", os.path.join(rocm, "lib"), "-lamdhip64",
          "-Wl,-rpath," + str(tmp_path), "-Wl,-rpath," + os.path.join(rocm, "lib"), "-o", str(exe)])
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0")
    r = _run([str(exe)], env=env, timeout=120)
    assert "0 failures" in r.stdout
