"""The pins must catch plausible mistakes in the oracle.

Each case plants one mistake in a private copy of the oracle's C source (the
kinds of bug the pages record - round-half-up, m/1024 subnormals, no mantissa
carry, a 240 clamp, bias 8 - plus a dropped sign, swapped nibbles, swapped
gate/up, a dropped global scale and a wrong exponent sign; and in the fused
reference driver and the row drivers: swapped gate/up, a wrong subtile
stride, a per-row global scale ignored or taken from the first row, a
shifted FP32 output), builds it with gcc into a temporary directory, swaps it
in, and requires that at least one pin fails. The committed oracle is never
modified.
"""
import os
import subprocess

import numpy as np

import pytest

import oracle
import test_oracle_pins as P
from oracle import build as B

MUTANTS = {
    "round_half_up": ("int hs = (int)rint((double)v);",
                      "int hs = (int)floor((double)v + 0.5);"),
    "subnormal_1024": ("(double)m / 512.0", "(double)m / 1024.0"),
    "no_mantissa_carry": ("if (mant == 8.0) {                    /* mantissa overflow: carry */\n        e += 1;\n        mant = 0.0;",
                          "if (mant == 8.0) {\n        mant = 7.0;"),
    "clamp_240": ("if (v > 448.0f)\n        v = 448.0f;", "if (v > 240.0f)\n        v = 240.0f;"),
    "bias_8": ("int biased = e + 7;", "int biased = e + 8;"),
    "decode_bias_8": ("ldexp(1.0 + (double)m / 8.0, e - 7)", "ldexp(1.0 + (double)m / 8.0, e - 8)"),
    "dropped_sign": ("(signbit(x[j]) ? 8 : 0)", "0"),
    "swapped_nibbles": ("code[2 * i] | (code[2 * i + 1] << 4)", "code[2 * i + 1] | (code[2 * i] << 4)"),
    "swapped_gate_up": ("float g = oracle_bf16_to_f32(row[base + j % 8]);\n            float u = oracle_bf16_to_f32(row[base + 8 + j % 8]);",
                        "float u = oracle_bf16_to_f32(row[base + j % 8]);\n            float g = oracle_bf16_to_f32(row[base + 8 + j % 8]);"),
    "no_global_scale_in_k": ("float k = 6.0f * gs;", "float k = 6.0f;"),
    "exp_sign": ("double y = g * u / (1.0 + exp(-g));", "double y = g * u / (1.0 + exp(g));"),
    "no_six_clamp": ("v = 2.0f * fminf(fabsf(s), 6.0f);", "v = fminf(2.0f * fabsf(s), 13.0f);"),
    "t7_toward_zero": ("{0, 1, 2, 3, 4, 4, 5, 6, 6, 6, 6, 7, 7}", "{0, 1, 2, 3, 4, 4, 5, 5, 6, 6, 6, 7, 7}"),
    "amax_skips_last_row": ("for (int64_t r = offsets[e]; r < offsets[e + 1]; ++r)",
                            "for (int64_t r = offsets[e]; r + 1 < offsets[e + 1]; ++r)"),
    "amax_signed": ("float a = fabsf(y[r * cols + c]);", "float a = y[r * cols + c];"),
    "bf16_half_up": ("q = ldexp(rint(ldexp(m, 8)), e - 8);", "q = ldexp(floor(ldexp(m, 8) + 0.5), e - 8);"),
    "bf16_truncate": ("q = ldexp(rint(ldexp(m, 8)), e - 8);", "q = ldexp(floor(ldexp(m, 8)), e - 8);"),
    "bf16_7_bits": ("q = ldexp(rint(ldexp(m, 8)), e - 8);", "q = ldexp(rint(ldexp(m, 7)), e - 7);"),
    "bf16_subnormal_8_bits": ("q = ldexp(rint(ldexp(a, 133)), -133);",
                              "{ int e2; double m2 = frexp(a, &e2); q = ldexp(rint(ldexp(m2, 8)), e2 - 8); }"),
    "swiglu_f32_swapped": ("y[r * inter + j] = oracle_swiglu(a[col], a[col + 8]);",
                           "y[r * inter + j] = oracle_swiglu(a[col + 8], a[col]);"),
    "swiglu_f32_stride": ("int64_t col = 16 * (j / 8) + j % 8;", "int64_t col = 8 * (j / 8) + j % 8;"),
    "swiglu_bf16_shifted": ("out[r * inter + j] = oracle_f32_to_bf16(y[j]);",
                            "out[r * inter + j] = oracle_f32_to_bf16(y[j ^ 1]);"),
    # the fused reference driver and the per-row global scales of the row drivers
    "fused_driver_swapped_gate_up": (
        "float g = oracle_bf16_to_f32(row[base + col % 8]);\n                float u = oracle_bf16_to_f32(row[base + 8 + col % 8]);",
        "float u = oracle_bf16_to_f32(row[base + col % 8]);\n                float g = oracle_bf16_to_f32(row[base + 8 + col % 8]);"),
    "fused_driver_stride": ("int64_t base = 16 * (col / 8);", "int64_t base = 8 * (col / 8);"),
    "fused_driver_ignores_gs": ("const uint16_t *row = in + r * ld_in;\n        float gs = gs_rows ? gs_rows[r] : 1.0f;",
                                "const uint16_t *row = in + r * ld_in;\n        float gs = 1.0f;"),
    "fused_driver_first_row_gs": ("const uint16_t *row = in + r * ld_in;\n        float gs = gs_rows ? gs_rows[r] : 1.0f;",
                                  "const uint16_t *row = in + r * ld_in;\n        float gs = gs_rows ? gs_rows[0] : 1.0f;"),
    "fused_driver_out_shifted": ("swiglu_out[r * inter + col] = blk[j];", "swiglu_out[r * inter + (col ^ 1)] = blk[j];"),
    "bf16_driver_ignores_gs": ("float gs = gs_rows ? gs_rows[r] : 1.0f;\n        for (int64_t b = 0; b < nb; ++b) {\n            float blk[16];\n            for (int j = 0; j < 16; ++j)\n                blk[j] = oracle_bf16_to_f32(x[",
                               "float gs = 1.0f;\n        for (int64_t b = 0; b < nb; ++b) {\n            float blk[16];\n            for (int j = 0; j < 16; ++j)\n                blk[j] = oracle_bf16_to_f32(x["),
    "f32_driver_ignores_gs": ("float gs = gs_rows ? gs_rows[r] : 1.0f;\n        for (int64_t b = 0; b < nb; ++b) {\n            float bsf;",
                              "float gs = 1.0f;\n        for (int64_t b = 0; b < nb; ++b) {\n            float bsf;"),
    "dequant_first_row_gs": ("float gs = gs_rows ? gs_rows[r] : 1.0f;\n        for (int64_t c = 0; c < cols; ++c) {",
                             "float gs = gs_rows ? gs_rows[0] : 1.0f;\n        for (int64_t c = 0; c < cols; ++c) {"),
}

FAST_PINS = [P.pin_page_facts, P.pin_fp8_decode_vs_torch, P.pin_fp8_saturation,
             P.pin_fp8_roundtrip, P.pin_e2m1_format, P.pin_e2m1_table,
             P.pin_swiglu_vs_torch, P.pin_swiglu_closed_forms,
             P.pin_quantize_vs_twin, P.pin_dequant_closed_form,
             P.pin_group_amax, P.pin_expert_global_scale, P.pin_bf16_ties,
             P.pin_swiglu_bf16_vs_torch, lambda: P.pin_bf16_vs_torch(step=9973),
             P.pin_swiglu_f32, P.pin_moe_l1_gemm,
             lambda: P.pin_fp8_encode_vs_torch(step=997),
             P.pin_quantize_rows_gs, P.pin_fused_driver]


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_mutant(name, tmp_path, monkeypatch):
    old, new = MUTANTS[name]
    src = open(B.SRC).read()
    assert src.count(old) == 1, "mutation target not found exactly once: " + name
    csrc = tmp_path / "nvfp4_oracle.c"
    csrc.write_text(src.replace(old, new))
    hdr = os.path.join(os.path.dirname(B.SRC), "nvfp4_oracle.h")
    (tmp_path / "nvfp4_oracle.h").write_text(open(hdr).read())
    so = tmp_path / "libmutant.so"
    subprocess.run(["gcc", *B.CFLAGS, str(csrc), "-o", str(so), "-lm"], check=True)

    real = oracle.lib()
    monkeypatch.setattr(B, "LIB", str(so))
    monkeypatch.setattr(oracle, "_LIB", None)
    try:
        caught = []
        for pin in FAST_PINS:
            try:
                pin()
            except AssertionError:
                caught.append(getattr(pin, "__name__", "fp8_encode_strided"))
        assert caught, "no pin caught mutant " + name
    finally:
        monkeypatch.setattr(oracle, "_LIB", real)


# The global-scale step lives in the oracle's Python front end: plant its
# mistakes by swapping in a broken function.
PY_MUTANTS = {
    "gs_6x488": lambda a: np.where(a > 0, np.asarray(a, np.float32) / np.float32(6 * 488.0),
                                   np.float32(1.0)).astype(np.float32),
    "gs_times_2688": lambda a: np.where(a > 0, np.asarray(a, np.float32) * np.float32(2688.0),
                                        np.float32(1.0)).astype(np.float32),
    "gs_zero_for_empty": lambda a: (np.asarray(a, np.float32) / np.float32(2688.0)).astype(np.float32),
    "gs_reciprocal_multiply": lambda a: np.where(
        a > 0, np.asarray(a, np.float32) * (np.float32(1.0) / np.float32(2688.0)),
        np.float32(1.0)).astype(np.float32),
    "gs_clamped": lambda a: np.where(a > 0, np.clip(np.asarray(a, np.float32) / np.float32(2688.0),
                                                    np.float32(2.0 ** -100), np.float32(2.0 ** 100)),
                                     np.float32(1.0)).astype(np.float32),
}


@pytest.mark.parametrize("name", sorted(PY_MUTANTS))
def test_pins_catch_global_scale_mutant(name, monkeypatch):
    monkeypatch.setattr(oracle, "expert_global_scale", PY_MUTANTS[name])
    with pytest.raises(AssertionError):
        P.pin_expert_global_scale()


def _gemm_left(x, w1, offsets=None, rows=None):
    """moe_l1_gemm with the expert lookup off by one at boundaries."""
    xs, ws = np.asarray(x, np.uint16), np.asarray(w1, np.uint16)
    if ws.ndim == 2:
        ws = ws[None]
    t_all = np.arange(xs.shape[0]) if rows is None else np.asarray(rows)
    e_of = (np.zeros(t_all.size, np.int64) if offsets is None else
            np.clip(np.searchsorted(np.asarray(offsets, np.int64), t_all, side="left") - 1, 0, None))
    out = np.empty((t_all.size, ws.shape[1]), np.float64)
    for e in np.unique(e_of):
        sel = np.nonzero(e_of == e)[0]
        xf = (xs[t_all[sel]].astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        wf = (ws[e].astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        out[sel] = xf @ wf.T
    return out


GEMM_MUTANTS = {
    "gemm_expert_left": _gemm_left,
    "gemm_float32": lambda x, w1, offsets=None, rows=None: _REAL_GEMM(x, w1, offsets, rows).astype(np.float32).astype(np.float64) + 1e-9,
    "gemm_untransposed_ok_shape": lambda x, w1, offsets=None, rows=None: _REAL_GEMM(x, np.asarray(w1)[..., ::-1], offsets, rows),
}
_REAL_GEMM = oracle.moe_l1_gemm


@pytest.mark.parametrize("name", sorted(GEMM_MUTANTS))
def test_pins_catch_gemm_mutant(name, monkeypatch):
    monkeypatch.setattr(oracle, "moe_l1_gemm", GEMM_MUTANTS[name])
    with pytest.raises(AssertionError):
        P.pin_moe_l1_gemm()


# the paged KV-cache write and read, mutated in the plausible ways: the row
# index used as the slot, a negative slot allowed to wrap (NumPy indexing),
# the read ignoring the slots, skipped rows not zeroed
def _paged_row_as_slot(x, slots, pc, sc, gs=None):
    return _REAL_QP(x, np.arange(len(slots)), pc, sc, gs)


def _paged_wrap(x, slots, pc, sc, gs=None):
    p, s = oracle.quantize_bf16(x, None if gs is None else np.full(x.shape[0], gs, np.float32))
    for r, slot in enumerate(slots):
        if slot < pc.shape[0]:
            pc[int(slot)] = p[r]
            sc[int(slot)] = s[r]
    return pc, sc


def _paged_read_identity(pc, sc, slots, gs=None):
    return _REAL_DP(pc, sc, np.arange(len(slots)), gs)


def _paged_read_garbage(pc, sc, slots, gs=None):
    out = _REAL_DP(pc, sc, slots, gs)
    bad = [r for r, slot in enumerate(slots) if not 0 <= slot < pc.shape[0]]
    out[bad] = 1.0
    return out


_REAL_QP = oracle.quantize_paged
_REAL_DP = oracle.dequantize_paged
PAGED_MUTANTS = {
    "paged_row_as_slot": ("quantize_paged", _paged_row_as_slot),
    "paged_negative_wraps": ("quantize_paged", _paged_wrap),
    "paged_read_ignores_slots": ("dequantize_paged", _paged_read_identity),
    "paged_read_skipped_not_zero": ("dequantize_paged", _paged_read_garbage),
}


@pytest.mark.parametrize("name", sorted(PAGED_MUTANTS))
def test_pins_catch_paged_mutant(name, monkeypatch):
    attr, fn = PAGED_MUTANTS[name]
    monkeypatch.setattr(oracle, attr, fn)
    with pytest.raises((AssertionError, IndexError)):
        P.pin_paged_kv()
