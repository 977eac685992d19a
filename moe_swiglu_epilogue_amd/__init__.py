"""MI355X (gfx950) fused SwiGLU + NVFP4 block quantization.

The compute lives in ``libmoe_nvfp4.so`` (hand-written HIP kernels behind a
C ABI, declared in ``include/moe_nvfp4.h``); this package is a thin binding:
``nvfp4_quantize``, ``swiglu_nvfp4_quantize`` and ``nvfp4_dequantize`` take
torch tensors on the GPU, marshal pointers, sizes and the current stream, and
call the library. Importing the package does not load the library; the first
call does, and raises if it is missing.
"""
import importlib

__all__ = ["nvfp4_quantize", "swiglu_nvfp4_quantize", "nvfp4_dequantize",
           "nvfp4_global_scale", "swiglu_nvfp4_global_scale", "swiglu_bf16",
           "moe_l1_gemm_swiglu_nvfp4", "moe_l1_gemm_bf16", "nvfp4_quantize_paged",
           "nvfp4_dequantize_paged", "Nvfp4Error", "library_path"]


def __getattr__(name):
    if name == "binding" or name in __all__:
        binding = importlib.import_module(__name__ + ".binding")
        return binding if name == "binding" else getattr(binding, name)
    raise AttributeError(name)
