"""Code generation checks on the gfx950 ISA of the library (CPU only: hipcc
cross-compiles the device code to assembly).

* The pipelined store loops (quantize, paged write, compact SwiGLU) must never wait for
  their own output stores:
  on gfx9 the vmcnt counter covers stores as well as loads, so the loop
  that holds a wide-store quantize kernel's output stores (found from its
  backward branch) contains no `s_waitcnt vmcnt(0)`. A second one means the compiler merged
  the prologue's LDS staging into the loop and every pass drains the stores
  (measured: 5% slower on the prefill shape).
* The compact SwiGLU pass rounds with v_cvt_pk_bf16_f32 (8 per lane block).
* No scalar-memory writes or atomics anywhere in the device code: stores and
  atomics go through the vector memory path only.
* No kernel uses scratch memory (no register spills), in either source.
* The grouped GEMM's x slice loads are range-checked row by row: the buffer
  range check covers the VGPR offset, not the SGPR offset, so the x loads
  must use one VGPR offset per x row a lane loads (8), not one offset plus
  a row step in the SGPR (which would let a partial tile read past x).
* The GEMM's LDS-DMA loads are written as inline assembly that sets M0 (the
  LDS address) itself, so M0 must have no other use in those kernels: every
  M0 write is immediately followed by an LDS-DMA load and every such load
  immediately follows one.
"""
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def isa(tmp_path_factory):
    from moe_swiglu_epilogue_amd import build as B
    out = tmp_path_factory.mktemp("isa") / "moe_nvfp4.s"
    subprocess.run([B.HIPCC, *B.FLAGS, "-I", os.path.join(ROOT, "include"), "--cuda-device-only",
                    "-S", os.path.join(ROOT, "moe_swiglu_epilogue_amd", "csrc", "moe_nvfp4.hip"),
                    "-o", str(out)], check=True, capture_output=True)
    return out.read_text()


def _kernels(text):
    lines = text.split("\n")
    funcs = set(re.findall(r"\.type\s+(_Z\w+),@function", text))   # not data symbols
    out = {}
    for k, l in enumerate(lines):
        m = re.match(r"^(_Z\w+):", l)
        if m and m.group(1) in funcs:
            end = next(j for j in range(k, len(lines)) if lines[j].strip().startswith(".Lfunc_end"))
            out[m.group(1)] = [x.strip() for x in lines[k + 1:end]
                               if x.startswith("\t") or re.match(r"^\.LBB\w+:", x)]
    return out


def store_loops(body):
    """[start, end) line ranges of the loops (a backward branch to a label)
    that contain the 16-byte output stores."""
    labels = {}
    for k, l in enumerate(body):
        m = re.match(r"^(\.LBB\w+):", l)
        if m:
            labels[m.group(1)] = k
    loops = []
    for k, l in enumerate(body):
        m = re.match(r"s_(?:cbranch_\w+|branch)\s+(\.LBB\w+)", l)
        if m and labels.get(m.group(1), k + 1) < k:
            loops.append((labels[m.group(1)], k + 1))
    return [(a, b) for a, b in loops if any(l.startswith("buffer_store_dwordx4") for l in body[a:b])]


def loop_waits_for_stores(isa):
    """Names of the pipelined store kernels (wide-store quantize, compact
    SwiGLU) whose store loop has a vmcnt(0)."""
    ks = {n: body for n, body in _kernels(isa).items()
          if (("quantize_tiles_kernel" in n or "quantize_paged_kernel" in n) and "Lb1E" in n)
          or "swiglu_bf16_kernel" in n}
    assert len(ks) == 4, sorted(ks)
    bad = []
    for name, body in ks.items():
        loops = store_loops(body)
        assert loops, name
        if any("vmcnt(0)" in l for a, b in loops for l in body[a:b] if l.startswith("s_waitcnt")):
            bad.append(name)
    return bad


def test_wide_quantize_loops_do_not_wait_for_stores(isa):
    assert loop_waits_for_stores(isa) == []


def test_bf16_rounding_is_the_hardware_convert(isa):
    body = next(b for n, b in _kernels(isa).items() if "swiglu_bf16_kernel" in n)
    assert sum(l.startswith("v_cvt_pk_bf16_f32") for l in body) == 8


def test_no_scalar_memory_writes(isa):
    bad = sorted(set(re.findall(r"\bs_(?:store|atomic|buffer_store|buffer_atomic|dcache_wb|"
                                r"scratch_store)\w*", isa)))
    assert not bad, bad


def table_loads_precede_tile_loads(isa):
    """For each kernel that copies the sigmoid table: in the code before its
    set-up barrier, the table's eight 16-byte loads (plain) must all be
    issued before the first tile's 16-byte loads (non-temporal), so that the
    wait before the table's LDS writes does not also wait for the tile's HBM
    loads (loads retire in order). Returns the kernels where they do not."""
    ks = {n: body for n, body in _kernels(isa).items()
          if "FusedBlock" in n or "swiglu_bf16_kernel" in n}
    assert len(ks) == 4, sorted(ks)
    bad = []
    for name, body in ks.items():
        seen = False
        start = 0
        for k, l in enumerate(body):
            if not l.startswith("s_barrier"):
                continue
            seg = body[start:k]
            start = k + 1
            loads = [x for x in seg if x.startswith("global_load_dwordx4")]
            nt = [j for j, x in enumerate(loads) if x.endswith(" nt")]
            plain = [j for j, x in enumerate(loads) if not x.endswith(" nt")]
            if nt and len(plain) >= 8:
                seen = True
                if plain[7] > nt[0]:
                    bad.append(name)
        if not seen:
            bad.append(name + " (no set-up segment found)")
    return bad


def test_sigma_table_loads_go_out_before_the_first_tile(isa):
    assert table_loads_precede_tile_loads(isa) == []


def test_no_scratch_in_any_kernel(tmp_path):
    from moe_swiglu_epilogue_amd import build as B
    for src in (B.SRC, B.GEMM_SRC):
        out = tmp_path / (os.path.basename(src) + ".o")
        r = subprocess.run([B.HIPCC, *B.FLAGS, "-I", os.path.join(ROOT, "include"),
                            "-Rpass-analysis=kernel-resource-usage", "--cuda-device-only", "-c", src,
                            "-o", str(out)], capture_output=True, text=True, check=True)
        sizes = re.findall(r"ScratchSize \[bytes/lane\]: (\d+)", r.stderr)
        names = re.findall(r"Function Name: (\S+)", r.stderr)
        assert sizes and len(sizes) == len(names), src
        assert all(int(v) == 0 for v in sizes), list(zip(names, sizes))


@pytest.fixture(scope="module")
def gemm_isa(tmp_path_factory):
    from moe_swiglu_epilogue_amd import build as B
    out = tmp_path_factory.mktemp("isa") / "moe_gemm.s"
    subprocess.run([B.HIPCC, *B.FLAGS, "-I", os.path.join(ROOT, "include"), "--cuda-device-only",
                    "-S", B.GEMM_SRC, "-o", str(out)], check=True, capture_output=True)
    return out.read_text()


def _mfma_loop(body):
    """The lines of the loop that holds the MFMAs (the K loop): from its
    header label to the branch back to it. Within it the tile's buffer
    descriptors are loop-invariant and stay in the same SGPRs."""
    best = None
    for i, l in enumerate(body):
        m = re.match(r"(\.LBB\d+_\d+):", l)
        if not m:
            continue
        back = [k for k in range(i + 1, len(body))
                if re.match(r"s_(cbranch_\w+|branch) " + re.escape(m.group(1)) + r"$", body[k])]
        if back and any(x.startswith("v_mfma") for x in body[i:back[-1]]):
            span = (i, back[-1])
            if best is None or span[1] - span[0] < best[1] - best[0]:
                best = span
    assert best is not None
    return body[best[0]:best[1] + 1]


def test_gemm_x_rows_are_range_checked(gemm_isa):
    ks = {n: b for n, b in _kernels(gemm_isa).items() if "moe_gemm_kernel" in n}
    assert len(ks) == 2, sorted(ks)
    for name, body in ks.items():
        voffsets = {}
        for l in _mfma_loop(body):
            m = re.match(r"buffer_load_dwordx4 (?:v\[\d+:\d+\], )?(v\d+), (s\[\d+:\d+\]), \S+ offen", l)
            if m:
                voffsets.setdefault(m.group(2), set()).add(m.group(1))
        # in the K loop the x resource (in whichever SGPRs it sits) is loaded
        # through 8 distinct VGPR offsets, one per row a lane loads; w through
        # at most 2 (its row step is in the SGPR offset: every w row is inside
        # its window)
        counts = sorted(len(v) for v in voffsets.values())
        assert 8 in counts and set(counts) <= {1, 2, 8}, (name, counts)


def test_gemm_m0_only_feeds_lds_dma(gemm_isa):
    for name, body in _kernels(gemm_isa).items():
        if "moe_gemm_kernel" not in name:
            continue
        code = [l for l in body if not l.startswith(";")]
        dma = 0
        for k, l in enumerate(code):
            if re.search(r"\bm0\b", l):
                assert l.startswith("s_mov_b32 m0,"), (name, l)
                assert code[k + 1].startswith("buffer_load_dwordx4") and code[k + 1].endswith(" lds"), (name, code[k + 1])
            if l.startswith("buffer_load_dwordx4") and l.endswith(" lds"):
                assert code[k - 1].startswith("s_mov_b32 m0,"), (name, code[k - 1])
                dma += 1
        assert dma >= 16, (name, dma)
