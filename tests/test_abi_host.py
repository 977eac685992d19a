"""C ABI on the host, no GPU needed: the library loads, exports every symbol
that include/moe_nvfp4.h declares, and rejects bad arguments with the
documented status before touching HIP."""
import ctypes as C
import os
import re
import subprocess

import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe_nvfp4.h")
CALIB_HEADER = os.path.join(ROOT, "include", "nvfp4_calib.h")
DIVCHECK_HEADER = os.path.join(ROOT, "include", "nvfp4_divcheck.h")

OK, INVALID, SHAPE, MISALIGNED = 0, 1, 2, 3


@pytest.fixture(scope="module")
def lib():
    from moe_swiglu_epilogue_amd import binding, build
    if not os.path.exists(binding.LIB_PATH):
        build.build()
    return binding.raw()


def _declared(path=HEADER):
    text = open(path).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+char\s*\*|nvfp4_status_t|int)\s*(\w+)\s*\(",
                                 text, re.M)))


def _exported(lib_path):
    out = subprocess.run(["nm", "-D", "--defined-only", lib_path],
                         capture_output=True, text=True, check=True).stdout
    return set(l.split()[-1] for l in out.splitlines() if " T " in l)


def test_header_declares_the_entry_points():
    assert _declared() == sorted(["nvfp4_quantize", "swiglu_nvfp4_quantize",
                                  "nvfp4_dequantize", "nvfp4_global_scale",
                                  "swiglu_nvfp4_global_scale", "swiglu_bf16",
                                  "moe_l1_gemm_swiglu_nvfp4", "moe_l1_gemm_bf16",
                                  "nvfp4_quantize_paged", "nvfp4_dequantize_paged",
                                  "nvfp4_status_string"])


def test_library_exports_every_declared_symbol(lib):
    from moe_swiglu_epilogue_amd import binding
    exported = _exported(binding.LIB_PATH)
    for name in _declared():
        assert name in exported, name
        assert getattr(lib, name) is not None
    assert set(_declared()) == set(binding.EXPORTS)


def test_calib_library_exports_its_header(lib):
    import ctypes as C
    from moe_swiglu_epilogue_amd import build
    names = _declared(CALIB_HEADER)
    assert names == ["nvfp4_calib_copy", "nvfp4_calib_mix", "nvfp4_calib_read"]
    assert set(names) <= _exported(build.CALIB_LIB)
    cl = C.CDLL(build.CALIB_LIB)
    for fn in (cl.nvfp4_calib_copy, cl.nvfp4_calib_read):
        fn.argtypes = [C.c_void_p, C.c_void_p, C.c_int64, C.c_int32, C.c_void_p]
        assert fn(A16, A16, 24, 8, None) == 1        # not a multiple of 16
        assert fn(A16, A16 + 4, 32, 8, None) == 1    # misaligned
        assert fn(A16, A16, 32, 0, None) == 1        # no workgroups
        assert fn(A16, A16, 0, 8, None) == 0         # empty: no launch
    mix = cl.nvfp4_calib_mix
    mix.argtypes = [C.c_void_p, C.c_void_p, C.c_int64, C.c_int32, C.c_void_p]
    assert mix(A16, A16, 4096 + 16, 0, None) == 1     # not whole 4 KB tiles
    assert mix(A16, A16 + 4, 4096, 0, None) == 1      # misaligned
    assert mix(A16, A16, 4096, -1, None) == 1         # negative LDS
    assert mix(A16, A16, 4096, 65537, None) == 1      # more LDS than a workgroup can have
    assert mix(A16, A16, 0, 0, None) == 0             # empty: no launch


def test_divcheck_library_exports_its_header():
    import ctypes as C
    from moe_swiglu_epilogue_amd import build
    names = _declared(DIVCHECK_HEADER)
    assert names == ["nvfp4_divcheck"]
    assert set(names) <= _exported(build.DIVCHECK_LIB)
    fn = C.CDLL(build.DIVCHECK_LIB).nvfp4_divcheck
    fn.argtypes = [C.c_uint32, C.c_uint32, C.c_int, C.c_void_p, C.c_void_p, C.c_void_p]
    assert fn(0, 0, 0, A16, A16, None) == 1               # no divisors
    assert fn(1 << 23, 1, 0, A16, A16, None) == 1         # first beyond the significands
    assert fn((1 << 23) - 4, 5, 0, A16, A16, None) == 1   # range beyond them
    assert fn(0, 1, 0, None, A16, None) == 1              # no counter
    assert fn(0, 1, 0, A16, None, None) == 1              # no witness


def test_header_compiles_as_c(tmp_path):
    src = tmp_path / "t.c"
    src.write_text('#include "moe_nvfp4.h"\n#include "nvfp4_calib.h"\n#include "nvfp4_divcheck.h"\n'
                   'int main(void){return (int)NVFP4_SUCCESS;}\n')
    subprocess.run(["gcc", "-std=c11", "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"),
                    "-I", "/opt/rocm/include", "-c", str(src), "-o", str(tmp_path / "t.o")],
                   check=True)


def test_status_strings(lib):
    for s in range(5):
        assert lib.nvfp4_status_string(s)
    assert lib.nvfp4_status_string(99) == b"unknown status"


A16 = 0x10000      # a fake 16-byte-aligned "device" address, never dereferenced


def q(lib, x=A16, rows=4, cols=32, ld=32, gs=None, offs=None, ne=0, packed=A16, scales=A16):
    return lib.nvfp4_quantize(x, rows, cols, ld, gs, offs, ne, packed, scales, None)


def f(lib, x=A16, rows=4, inter=32, ld=64, gs=None, offs=None, ne=0, packed=A16,
      scales=A16, y=None):
    return lib.swiglu_nvfp4_quantize(x, rows, inter, ld, gs, offs, ne, packed, scales, y, None)


def d(lib, packed=A16, scales=A16, rows=4, cols=32, gs=None, offs=None, ne=0, out=A16):
    return lib.nvfp4_dequantize(packed, scales, rows, cols, gs, offs, ne, out, None)


def test_quantize_validation(lib):
    assert q(lib, rows=-1) == INVALID
    assert q(lib, cols=-16) == INVALID
    assert q(lib, cols=24, ld=24) == SHAPE
    assert q(lib, ld=16) == INVALID
    assert q(lib, x=None) == INVALID
    assert q(lib, packed=None) == INVALID
    assert q(lib, scales=None) == INVALID
    assert q(lib, x=A16 + 2) == MISALIGNED
    assert q(lib, ld=36) == MISALIGNED            # 72-byte pitch
    assert q(lib, packed=A16 + 4) == MISALIGNED
    assert q(lib, ne=3) == INVALID                # experts without offsets
    assert q(lib, offs=A16, ne=0) == INVALID      # offsets without experts
    assert q(lib, offs=A16, ne=-1) == INVALID
    assert q(lib, rows=2**31, cols=16, ld=16) == SHAPE
    # empty problems succeed without launching (NULL pointers are fine)
    assert q(lib, x=None, rows=0, packed=None, scales=None) == OK
    assert q(lib, x=None, cols=0, ld=0, packed=None, scales=None) == OK


def test_fused_validation(lib):
    assert f(lib, rows=-1) == INVALID
    assert f(lib, inter=8, ld=16) == SHAPE
    assert f(lib, ld=63) == INVALID
    assert f(lib, ld=68) == MISALIGNED
    assert f(lib, x=A16 + 8) == MISALIGNED
    assert f(lib, y=A16 + 8) == MISALIGNED
    assert f(lib, x=None) == INVALID
    assert f(lib, ne=2) == INVALID
    assert f(lib, inter=2**62, ld=2**62) == INVALID
    assert f(lib, rows=0, x=None, packed=None, scales=None) == OK


def test_dequant_validation(lib):
    assert d(lib, rows=-1) == INVALID
    assert d(lib, cols=8) == SHAPE
    assert d(lib, out=A16 + 4) == MISALIGNED
    assert d(lib, packed=A16 + 1) == MISALIGNED
    assert d(lib, out=None) == INVALID
    assert d(lib, offs=A16, ne=0) == INVALID
    assert d(lib, rows=0, packed=None, scales=None, out=None) == OK


def gsc(lib, fused=False, x=A16, rows=4, cols=32, ld=None, offs=None, ne=0, amax=None, gs=A16):
    if fused:
        return lib.swiglu_nvfp4_global_scale(x, rows, cols, 2 * cols if ld is None else ld,
                                             offs, ne, amax, gs, None)
    return lib.nvfp4_global_scale(x, rows, cols, cols if ld is None else ld, offs, ne, amax,
                                  gs, None)


@pytest.mark.parametrize("fused", [False, True])
def test_global_scale_validation(lib, fused):
    # every failing check returns before the first launch (rows == 0 is not a
    # no-op for these calls: they still write amax 0 and gs 1.0)
    assert gsc(lib, fused, rows=-1) == INVALID
    assert gsc(lib, fused, cols=24, ld=48 if fused else 24) == SHAPE
    assert gsc(lib, fused, ld=30 if not fused else 62) == INVALID
    assert gsc(lib, fused, gs=None) == INVALID
    assert gsc(lib, fused, x=None) == INVALID
    assert gsc(lib, fused, x=A16 + 2) == MISALIGNED
    assert gsc(lib, fused, gs=A16 + 2) == MISALIGNED
    assert gsc(lib, fused, amax=A16 + 1) == MISALIGNED
    assert gsc(lib, fused, ne=3) == INVALID
    assert gsc(lib, fused, offs=A16, ne=0) == INVALID
    assert gsc(lib, fused, offs=A16, ne=1025) == SHAPE
    assert gsc(lib, fused, rows=2**31, cols=16, ld=32 if fused else 16) == SHAPE


def sb(lib, x=A16, rows=4, inter=32, ld=64, out=A16, ld_out=32):
    return lib.swiglu_bf16(x, rows, inter, ld, out, ld_out, None)


def test_swiglu_bf16_validation(lib):
    assert sb(lib, rows=-1) == INVALID
    assert sb(lib, inter=8, ld=16, ld_out=8) == SHAPE
    assert sb(lib, ld=63) == INVALID
    assert sb(lib, ld_out=31) == INVALID
    assert sb(lib, x=None) == INVALID
    assert sb(lib, out=None) == INVALID
    assert sb(lib, x=A16 + 8) == MISALIGNED
    assert sb(lib, out=A16 + 8) == MISALIGNED
    assert sb(lib, ld_out=36) == MISALIGNED      # 72-byte output pitch
    assert sb(lib, ld=68) == MISALIGNED
    assert sb(lib, rows=2**31, inter=16, ld=32, ld_out=16) == SHAPE
    assert sb(lib, rows=0, x=None, out=None) == OK


def gf(lib, x=A16, w=A16, tokens=4, hidden=64, inter=128, ld_x=64, ld_w=64, offs=None, ne=0,
       gs=None, packed=A16, scales=A16, y=None):
    return lib.moe_l1_gemm_swiglu_nvfp4(x, w, tokens, hidden, inter, ld_x, ld_w, offs, ne, gs,
                                        packed, scales, y, None)


def gb(lib, x=A16, w=A16, tokens=4, hidden=64, n=256, ld_x=64, ld_w=64, offs=None, ne=0,
       out=A16, ld_out=256):
    return lib.moe_l1_gemm_bf16(x, w, tokens, hidden, n, ld_x, ld_w, offs, ne, out, ld_out, None)


def test_gemm_validation(lib):
    for f in (gf, gb):
        assert f(lib, tokens=-1) == INVALID
        assert f(lib, ld_x=32) == INVALID
        assert f(lib, ld_w=32) == INVALID
        assert f(lib, hidden=96, ld_x=96, ld_w=96) == SHAPE         # hidden % 64
        assert f(lib, ne=2) == INVALID
        assert f(lib, offs=A16, ne=0) == INVALID
        assert f(lib, offs=A16, ne=513) == SHAPE
        assert f(lib, x=A16 + 8) == MISALIGNED
        assert f(lib, w=A16 + 8) == MISALIGNED
        assert f(lib, ld_x=68) == MISALIGNED
        assert f(lib, x=None) == INVALID
        assert f(lib, hidden=0, ld_x=0, ld_w=0) == SHAPE
        assert f(lib, tokens=2**31) == SHAPE
        assert f(lib, ld_x=2**22) == SHAPE                         # 32-bit window offsets
        assert f(lib, ld_w=2**22) == SHAPE
        assert f(lib, ld_x=2**22 - 8, ld_w=2**22 - 8, x=None) == INVALID   # largest pitch passes
    assert gf(lib, inter=64) == SHAPE                              # 2 * inter % 256
    assert gf(lib, packed=None) == INVALID
    assert gf(lib, packed=A16 + 4) == MISALIGNED
    assert gf(lib, y=A16 + 8) == MISALIGNED
    assert gf(lib, tokens=0, x=None, w=None, packed=None, scales=None) == OK
    assert gb(lib, n=128, ld_out=128) == SHAPE
    assert gb(lib, ld_out=128) == INVALID
    assert gb(lib, out=A16 + 8) == MISALIGNED
    assert gb(lib, tokens=0, x=None, w=None, out=None) == OK


def qp(lib, x=A16, rows=4, cols=32, ld=32, gs=None, slots=A16, ns=8, packed=A16, scales=A16):
    return lib.nvfp4_quantize_paged(x, rows, cols, ld, gs, slots, ns, packed, scales, None)


def dp(lib, packed=A16, scales=A16, ns=8, slots=A16, rows=4, cols=32, gs=None, out=A16):
    return lib.nvfp4_dequantize_paged(packed, scales, ns, slots, rows, cols, gs, out, None)


def test_paged_validation(lib):
    assert qp(lib, rows=-1) == INVALID
    assert qp(lib, ns=-1) == INVALID
    assert qp(lib, ld=16) == INVALID
    assert qp(lib, cols=24, ld=24) == SHAPE
    assert qp(lib, ns=2**31) == SHAPE
    assert qp(lib, x=None) == INVALID
    assert qp(lib, slots=None) == INVALID
    assert qp(lib, packed=None) == INVALID
    assert qp(lib, scales=None) == INVALID
    assert qp(lib, x=A16 + 2) == MISALIGNED
    assert qp(lib, ld=36) == MISALIGNED
    assert qp(lib, packed=A16 + 4) == MISALIGNED
    assert qp(lib, slots=A16 + 4) == MISALIGNED
    assert qp(lib, rows=2**31, cols=16, ld=16) == SHAPE
    # nothing to write succeeds without launching (NULL pointers are fine)
    assert qp(lib, x=None, rows=0, slots=None, packed=None, scales=None) == OK
    assert qp(lib, x=None, slots=None, ns=0, packed=None, scales=None) == OK
    assert dp(lib, rows=-1) == INVALID
    assert dp(lib, ns=-1) == INVALID
    assert dp(lib, cols=24) == SHAPE
    assert dp(lib, ns=2**31) == SHAPE
    assert dp(lib, slots=None) == INVALID
    assert dp(lib, out=None) == INVALID
    assert dp(lib, packed=None) == INVALID
    assert dp(lib, out=A16 + 8) == MISALIGNED
    assert dp(lib, slots=A16 + 4) == MISALIGNED
    assert dp(lib, rows=0, slots=None, out=None, packed=None, scales=None) == OK
    # an empty cache may be NULL (every row reads as zeros)
    assert dp(lib, ns=0, packed=None, scales=None, rows=0) == OK


def test_pitch_extent_overflow_is_rejected(lib):
    """A row pitch whose byte extent rows * ld * 2 leaves int64 cannot
    describe a real buffer: every entry point says INVALID and computes
    nothing with it (the sanitizer build checks that no arithmetic
    overflows on the way)."""
    big = 2**63 - 8
    assert q(lib, ld=big) == INVALID
    assert f(lib, ld=big) == INVALID
    assert sb(lib, ld=big) == INVALID
    assert sb(lib, ld_out=big) == INVALID
    for fused in (False, True):
        assert gsc(lib, fused, ld=big) == INVALID
    for g in (gf, gb):
        # the grouped GEMM caps pitches below 2^22 first
        assert g(lib, ld_x=big) == SHAPE
        assert g(lib, ld_w=big) == SHAPE
        assert g(lib, offs=A16, ne=512, ld_w=2**63 // (2 * 512 * 256) + 8) == SHAPE
    assert gb(lib, ld_out=big) == INVALID
    # one row has no extent beyond its own columns
    assert q(lib, rows=1, ld=big, x=None) == INVALID   # still reaches the NULL check


def test_binding_rejects_host_tensors():
    import moe_swiglu_epilogue_amd as M
    x = torch.zeros(4, 32, dtype=torch.bfloat16)
    with pytest.raises(TypeError):
        M.nvfp4_quantize(x)
    with pytest.raises(TypeError):
        M.swiglu_nvfp4_quantize(torch.zeros(4, 64, dtype=torch.bfloat16))
    with pytest.raises(TypeError):
        M.nvfp4_dequantize(torch.zeros(4, 16, dtype=torch.uint8), torch.zeros(4, 2, dtype=torch.uint8))
    with pytest.raises(TypeError):
        M.nvfp4_global_scale(x)
    with pytest.raises(TypeError):
        M.swiglu_nvfp4_global_scale(torch.zeros(4, 64, dtype=torch.bfloat16))
    with pytest.raises(TypeError):
        M.swiglu_bf16(torch.zeros(4, 64, dtype=torch.bfloat16))
    cache_p, cache_s = torch.zeros(8, 16, dtype=torch.uint8), torch.zeros(8, 2, dtype=torch.uint8)
    with pytest.raises(TypeError):
        M.nvfp4_quantize_paged(x, torch.zeros(4, dtype=torch.int64), cache_p, cache_s)
    with pytest.raises(TypeError):
        M.nvfp4_dequantize_paged(cache_p, cache_s, torch.zeros(4, dtype=torch.int64))
