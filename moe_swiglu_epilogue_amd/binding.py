"""ctypes binding of libmoe_nvfp4.so (include/moe_nvfp4.h).

Argument marshalling only: the functions take torch tensors that live on the
GPU, check dtypes and shapes, allocate missing outputs with ``torch.empty``,
and pass raw device pointers, sizes and torch's current HIP stream to the
C ABI. Every step of the computation runs in the library's kernels. If the
library is missing, loading it raises: there is no fallback.
"""
from __future__ import annotations

import ctypes as C
import os

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmoe_nvfp4.so")

STATUS = {0: "NVFP4_SUCCESS", 1: "NVFP4_ERROR_INVALID_VALUE",
          2: "NVFP4_ERROR_UNSUPPORTED_SHAPE", 3: "NVFP4_ERROR_MISALIGNED",
          4: "NVFP4_ERROR_LAUNCH"}

EXPORTS = ("nvfp4_quantize", "swiglu_nvfp4_quantize", "nvfp4_dequantize",
           "nvfp4_global_scale", "swiglu_nvfp4_global_scale", "swiglu_bf16",
           "moe_l1_gemm_swiglu_nvfp4", "moe_l1_gemm_bf16", "nvfp4_quantize_paged",
           "nvfp4_dequantize_paged", "nvfp4_status_string")

_LIB = None
_vp = C.c_void_p
_i64 = C.c_int64
_i32 = C.c_int32


class Nvfp4Error(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        text = _lib().nvfp4_status_string(status).decode()
        super().__init__("%s: %s (%s)" % (what, STATUS.get(status, status), text))


def library_path() -> str:
    return LIB_PATH


def _lib():
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                "libmoe_nvfp4.so is not built (%s); run "
                "`python -m moe_swiglu_epilogue_amd.build`" % LIB_PATH)
        L = C.CDLL(LIB_PATH)
        L.nvfp4_quantize.argtypes = [_vp, _i64, _i64, _i64, _vp, _vp, _i32, _vp, _vp, _vp]
        L.nvfp4_quantize.restype = C.c_int
        L.swiglu_nvfp4_quantize.argtypes = [_vp, _i64, _i64, _i64, _vp, _vp, _i32, _vp,
                                            _vp, _vp, _vp]
        L.swiglu_nvfp4_quantize.restype = C.c_int
        L.nvfp4_dequantize.argtypes = [_vp, _vp, _i64, _i64, _vp, _vp, _i32, _vp, _vp]
        L.nvfp4_dequantize.restype = C.c_int
        for fn in (L.nvfp4_global_scale, L.swiglu_nvfp4_global_scale):
            fn.argtypes = [_vp, _i64, _i64, _i64, _vp, _i32, _vp, _vp, _vp]
            fn.restype = C.c_int
        L.swiglu_bf16.argtypes = [_vp, _i64, _i64, _i64, _vp, _i64, _vp]
        L.swiglu_bf16.restype = C.c_int
        L.moe_l1_gemm_swiglu_nvfp4.argtypes = [_vp, _vp, _i64, _i64, _i64, _i64, _i64, _vp,
                                               _i32, _vp, _vp, _vp, _vp, _vp]
        L.moe_l1_gemm_swiglu_nvfp4.restype = C.c_int
        L.moe_l1_gemm_bf16.argtypes = [_vp, _vp, _i64, _i64, _i64, _i64, _i64, _vp, _i32, _vp,
                                       _i64, _vp]
        L.moe_l1_gemm_bf16.restype = C.c_int
        L.nvfp4_quantize_paged.argtypes = [_vp, _i64, _i64, _i64, _vp, _vp, _i64, _vp, _vp, _vp]
        L.nvfp4_quantize_paged.restype = C.c_int
        L.nvfp4_dequantize_paged.argtypes = [_vp, _vp, _i64, _vp, _i64, _i64, _vp, _vp, _vp]
        L.nvfp4_dequantize_paged.restype = C.c_int
        L.nvfp4_status_string.argtypes = [C.c_int]
        L.nvfp4_status_string.restype = C.c_char_p
        _LIB = L
    return _LIB


def raw():
    """The loaded ctypes library (for callers that pass raw pointers)."""
    return _lib()


# ---- marshalling helpers -----------------------------------------------------
def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream(stream):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def _bf16_matrix(t: torch.Tensor, name: str) -> torch.Tensor:
    if t.dtype == torch.bfloat16:
        t = t.view(torch.int16)
    if t.dtype not in (torch.int16, torch.uint16):
        raise TypeError("%s must be bfloat16 (or its 16-bit bit pattern)" % name)
    if not t.is_cuda:
        raise TypeError("%s must be a GPU tensor" % name)
    if t.dim() != 2 or (t.shape[1] > 1 and t.stride(1) != 1):
        raise ValueError("%s must be a 2-D tensor with unit column stride" % name)
    return t


def _pitch(t: torch.Tensor) -> int:
    return t.stride(0) if t.shape[0] > 1 else t.shape[1]


def _experts(gs, expert_offsets, device):
    if gs is not None:
        if gs.dtype != torch.float32 or gs.device != device or not gs.is_contiguous():
            raise TypeError("gs must be a contiguous float32 tensor on the input's device")
    if expert_offsets is None:
        if gs is not None and gs.numel() < 1:
            raise ValueError("gs must hold at least one value")
        return 0
    if (expert_offsets.dtype != torch.int32 or expert_offsets.device != device
            or not expert_offsets.is_contiguous()):
        raise TypeError("expert_offsets must be a contiguous int32 tensor on the input's device")
    e = expert_offsets.numel() - 1
    if e < 1:
        raise ValueError("expert_offsets must hold num_experts + 1 >= 2 entries")
    if gs is not None and gs.numel() != e:
        raise ValueError("gs must hold one value per expert")
    return e


def _out(t, shape, dtype, device, name):
    if t is None:
        return torch.empty(shape, dtype=dtype, device=device)
    if t.shape != torch.Size(shape) or t.dtype != dtype or t.device != device or not t.is_contiguous():
        raise ValueError("%s must be a contiguous %s tensor of shape %s" % (name, dtype, tuple(shape)))
    return t


def _call(fn, what, *args):
    st = fn(*args)
    if st != 0:
        raise Nvfp4Error(st, what)


# ---- entry points --------------------------------------------------------------
def nvfp4_quantize(x: torch.Tensor, gs: torch.Tensor | None = None,
                   expert_offsets: torch.Tensor | None = None, *,
                   packed: torch.Tensor | None = None, scales: torch.Tensor | None = None,
                   stream=None):
    """BF16 [rows, cols] -> (packed uint8 [rows, cols/2], scales uint8 [rows, cols/16])."""
    x = _bf16_matrix(x, "x")
    rows, cols = x.shape
    e = _experts(gs, expert_offsets, x.device)
    packed = _out(packed, (rows, cols // 2), torch.uint8, x.device, "packed")
    scales = _out(scales, (rows, cols // 16), torch.uint8, x.device, "scales")
    _call(_lib().nvfp4_quantize, "nvfp4_quantize", _ptr(x), rows, cols, _pitch(x), _ptr(gs),
          _ptr(expert_offsets), e, _ptr(packed), _ptr(scales), _stream(stream))
    return packed, scales


def swiglu_nvfp4_quantize(gate_up: torch.Tensor, gs: torch.Tensor | None = None,
                          expert_offsets: torch.Tensor | None = None, *,
                          packed: torch.Tensor | None = None,
                          scales: torch.Tensor | None = None,
                          swiglu_out: torch.Tensor | bool | None = None, stream=None):
    """Interleaved BF16 [rows, 2I] ([gate x8, up x8, ...]) -> (packed [rows, I/2],
    scales [rows, I/16]) and, when ``swiglu_out`` is True or a tensor, the FP32
    SwiGLU values [rows, I] as a third result."""
    x = _bf16_matrix(gate_up, "gate_up")
    rows, two_i = x.shape
    if two_i % 2:
        raise ValueError("gate_up must have an even number of columns")
    inter = two_i // 2
    e = _experts(gs, expert_offsets, x.device)
    packed = _out(packed, (rows, inter // 2), torch.uint8, x.device, "packed")
    scales = _out(scales, (rows, inter // 16), torch.uint8, x.device, "scales")
    y = None
    if swiglu_out is True:
        y = torch.empty((rows, inter), dtype=torch.float32, device=x.device)
    elif isinstance(swiglu_out, torch.Tensor):
        y = _out(swiglu_out, (rows, inter), torch.float32, x.device, "swiglu_out")
    _call(_lib().swiglu_nvfp4_quantize, "swiglu_nvfp4_quantize", _ptr(x), rows, inter,
          _pitch(x), _ptr(gs), _ptr(expert_offsets), e, _ptr(packed), _ptr(scales),
          _ptr(y), _stream(stream))
    return (packed, scales) if y is None else (packed, scales, y)


def nvfp4_dequantize(packed: torch.Tensor, scales: torch.Tensor,
                     gs: torch.Tensor | None = None,
                     expert_offsets: torch.Tensor | None = None, *,
                     out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """(packed uint8 [rows, cols/2], scales uint8 [rows, cols/16]) -> FP32 [rows, cols]."""
    if packed.dtype != torch.uint8 or scales.dtype != torch.uint8:
        raise TypeError("packed and scales must be uint8")
    if not packed.is_cuda or scales.device != packed.device:
        raise TypeError("packed and scales must be GPU tensors on one device")
    if not packed.is_contiguous() or not scales.is_contiguous():
        raise ValueError("packed and scales must be contiguous")
    rows, half = packed.shape
    cols = 2 * half
    if tuple(scales.shape) != (rows, cols // 16):
        raise ValueError("scales must have shape (rows, cols/16)")
    e = _experts(gs, expert_offsets, packed.device)
    out = _out(out, (rows, cols), torch.float32, packed.device, "out")
    _call(_lib().nvfp4_dequantize, "nvfp4_dequantize", _ptr(packed), _ptr(scales), rows, cols,
          _ptr(gs), _ptr(expert_offsets), e, _ptr(out), _stream(stream))
    return out


def _global_scale(fn, what, x, cols, expert_offsets, amax, gs, stream):
    rows = x.shape[0]
    e = _experts(None, expert_offsets, x.device)
    groups = e if expert_offsets is not None else 1
    gs = _out(gs, (groups,), torch.float32, x.device, "gs")
    a = None
    if amax is True:
        a = torch.empty((groups,), dtype=torch.float32, device=x.device)
    elif isinstance(amax, torch.Tensor):
        a = _out(amax, (groups,), torch.float32, x.device, "amax")
    _call(fn, what, _ptr(x), rows, cols, _pitch(x), _ptr(expert_offsets), e, _ptr(a), _ptr(gs),
          _stream(stream))
    return gs if a is None else (gs, a)


def nvfp4_global_scale(x: torch.Tensor, expert_offsets: torch.Tensor | None = None, *,
                       gs: torch.Tensor | None = None, amax: torch.Tensor | bool | None = None,
                       stream=None):
    """BF16 [rows, cols] -> gs float32 [G] (G = experts, or 1), gs = amax / (6*448)
    per expert; with ``amax`` True or a tensor also returns the FP32 amax [G]."""
    x = _bf16_matrix(x, "x")
    return _global_scale(_lib().nvfp4_global_scale, "nvfp4_global_scale", x, x.shape[1],
                         expert_offsets, amax, gs, stream)


def swiglu_nvfp4_global_scale(gate_up: torch.Tensor, expert_offsets: torch.Tensor | None = None,
                              *, gs: torch.Tensor | None = None,
                              amax: torch.Tensor | bool | None = None, stream=None):
    """Interleaved BF16 [rows, 2I] -> gs float32 [G] from the amax of the SwiGLU
    values (as swiglu_nvfp4_quantize computes them) per expert; with ``amax``
    True or a tensor also returns the FP32 amax [G]."""
    x = _bf16_matrix(gate_up, "gate_up")
    if x.shape[1] % 2:
        raise ValueError("gate_up must have an even number of columns")
    return _global_scale(_lib().swiglu_nvfp4_global_scale, "swiglu_nvfp4_global_scale", x,
                         x.shape[1] // 2, expert_offsets, amax, gs, stream)


def swiglu_bf16(gate_up: torch.Tensor, *, out: torch.Tensor | None = None, stream=None):
    """Interleaved BF16 [rows, 2I] -> compact BF16 [rows, I]: silu(gate) * up as the
    fused kernel computes it, rounded to BF16 (the first pass of the two-pass
    variant; nvfp4_quantize is the second). ``out`` may be a row-pitched view."""
    x = _bf16_matrix(gate_up, "gate_up")
    rows, two_i = x.shape
    if two_i % 2:
        raise ValueError("gate_up must have an even number of columns")
    inter = two_i // 2
    if out is None:
        out = torch.empty((rows, inter), dtype=torch.bfloat16, device=x.device)
    if (out.dtype != torch.bfloat16 or out.device != x.device or tuple(out.shape) != (rows, inter)
            or (inter > 1 and out.stride(1) != 1)):
        raise ValueError("out must be a bfloat16 tensor of shape (rows, I) with unit column stride")
    _call(_lib().swiglu_bf16, "swiglu_bf16", _ptr(x), rows, inter, _pitch(x), _ptr(out),
          _pitch(out), _stream(stream))
    return out


def _weights(w1: torch.Tensor, x: torch.Tensor):
    if w1.dtype == torch.bfloat16:
        w1 = w1.view(torch.int16)
    if w1.dtype not in (torch.int16, torch.uint16) or w1.device != x.device:
        raise TypeError("w1 must be bfloat16 on the activations' device")
    if w1.dim() == 2:
        w1 = w1.unsqueeze(0)
    # the expert stride only matters between experts (a size-1 dimension may
    # carry any stride, such as the 0 of a NumPy newaxis)
    if (w1.dim() != 3 or w1.stride(2) != 1
            or (w1.shape[0] > 1 and w1.stride(0) != w1.shape[1] * w1.stride(1))):
        raise ValueError("w1 must be [E, n, hidden] with unit column stride and packed experts")
    return w1


def moe_l1_gemm_swiglu_nvfp4(x: torch.Tensor, w1: torch.Tensor,
                             expert_offsets: torch.Tensor | None = None,
                             gs: torch.Tensor | None = None, *,
                             packed: torch.Tensor | None = None,
                             scales: torch.Tensor | None = None,
                             swiglu_out: torch.Tensor | bool | None = None, stream=None):
    """x BF16 [tokens, hidden], w1 BF16 [E, 2I, hidden] (rows = interleaved output
    columns) -> (packed [tokens, I/2], scales [tokens, I/16]) and, when
    ``swiglu_out`` is True or a tensor, y FP32 [tokens, I]."""
    x = _bf16_matrix(x, "x")
    w = _weights(w1, x)
    tokens, hidden = x.shape
    n = w.shape[1]
    if w.shape[2] != hidden:
        raise ValueError("w1 must be [E, 2I, hidden]")
    inter = n // 2
    e = _experts(gs, expert_offsets, x.device)
    packed = _out(packed, (tokens, inter // 2), torch.uint8, x.device, "packed")
    scales = _out(scales, (tokens, inter // 16), torch.uint8, x.device, "scales")
    y = None
    if swiglu_out is True:
        y = torch.empty((tokens, inter), dtype=torch.float32, device=x.device)
    elif isinstance(swiglu_out, torch.Tensor):
        y = _out(swiglu_out, (tokens, inter), torch.float32, x.device, "swiglu_out")
    _call(_lib().moe_l1_gemm_swiglu_nvfp4, "moe_l1_gemm_swiglu_nvfp4", _ptr(x), _ptr(w), tokens,
          hidden, inter, _pitch(x), w.stride(1), _ptr(expert_offsets), e, _ptr(gs), _ptr(packed),
          _ptr(scales), _ptr(y), _stream(stream))
    return (packed, scales) if y is None else (packed, scales, y)


def moe_l1_gemm_bf16(x: torch.Tensor, w1: torch.Tensor,
                     expert_offsets: torch.Tensor | None = None, *,
                     out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """x BF16 [tokens, hidden], w1 BF16 [E, n, hidden] -> BF16 [tokens, n]: the L1
    GEMM output (interleaved [gate x8, up x8, ...]) of the unfused flow."""
    x = _bf16_matrix(x, "x")
    w = _weights(w1, x)
    tokens, hidden = x.shape
    n = w.shape[1]
    if w.shape[2] != hidden:
        raise ValueError("w1 must be [E, n, hidden]")
    e = _experts(None, expert_offsets, x.device)
    if out is None:
        out = torch.empty((tokens, n), dtype=torch.bfloat16, device=x.device)
    if (out.dtype != torch.bfloat16 or out.device != x.device or tuple(out.shape) != (tokens, n)
            or (n > 1 and out.stride(1) != 1)):
        raise ValueError("out must be a bfloat16 tensor of shape (tokens, n) with unit column stride")
    _call(_lib().moe_l1_gemm_bf16, "moe_l1_gemm_bf16", _ptr(x), _ptr(w), tokens, hidden, n,
          _pitch(x), w.stride(1), _ptr(expert_offsets), e, _ptr(out), _pitch(out),
          _stream(stream))
    return out


def _slots(t: torch.Tensor, rows: int, device, name: str) -> torch.Tensor:
    if t.dtype != torch.int64 or t.device != device or not t.is_contiguous():
        raise TypeError("%s must be a contiguous int64 tensor on the input's device" % name)
    if t.numel() != rows:
        raise ValueError("%s must hold one slot per row" % name)
    return t


def _cache(packed_cache, scales_cache, cols):
    for t, name in ((packed_cache, "packed_cache"), (scales_cache, "scales_cache")):
        if t.dtype != torch.uint8 or not t.is_cuda or t.dim() != 2 or not t.is_contiguous():
            raise TypeError("%s must be a contiguous 2-D uint8 GPU tensor" % name)
    n = packed_cache.shape[0]
    if (tuple(packed_cache.shape) != (n, cols // 2)
            or tuple(scales_cache.shape) != (n, cols // 16)):
        raise ValueError("caches must be [num_slots, cols/2] and [num_slots, cols/16]")
    return n


def nvfp4_quantize_paged(x: torch.Tensor, slot_mapping: torch.Tensor, packed_cache: torch.Tensor,
                         scales_cache: torch.Tensor, gs: torch.Tensor | None = None, *,
                         stream=None):
    """BF16 [rows, cols] -> NVFP4 rows written into cache rows slot_mapping[r]
    of packed_cache [num_slots, cols/2] and scales_cache [num_slots, cols/16]
    (in place; slots outside [0, num_slots) are skipped)."""
    x = _bf16_matrix(x, "x")
    rows, cols = x.shape
    _experts(gs, None, x.device)
    slot_mapping = _slots(slot_mapping, rows, x.device, "slot_mapping")
    n = _cache(packed_cache, scales_cache, cols)
    _call(_lib().nvfp4_quantize_paged, "nvfp4_quantize_paged", _ptr(x), rows, cols, _pitch(x),
          _ptr(gs), _ptr(slot_mapping), n, _ptr(packed_cache), _ptr(scales_cache),
          _stream(stream))
    return packed_cache, scales_cache


def nvfp4_dequantize_paged(packed_cache: torch.Tensor, scales_cache: torch.Tensor,
                           slots: torch.Tensor, gs: torch.Tensor | None = None, *,
                           out: torch.Tensor | None = None, stream=None):
    """Cache rows slots[r] -> FP32 [rows, cols] (zeros for slots outside
    [0, num_slots))."""
    cols = packed_cache.shape[1] * 2 if packed_cache.dim() == 2 else 0
    n = _cache(packed_cache, scales_cache, cols)
    device = packed_cache.device
    _experts(gs, None, device)
    rows = slots.numel()
    slots = _slots(slots, rows, device, "slots")
    out = _out(out, (rows, cols), torch.float32, device, "out")
    _call(_lib().nvfp4_dequantize_paged, "nvfp4_dequantize_paged", _ptr(packed_cache),
          _ptr(scales_cache), n, _ptr(slots), rows, cols, _ptr(gs), _ptr(out), _stream(stream))
    return out
