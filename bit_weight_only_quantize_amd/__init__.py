"""MI355X-native AWQ W4A16: group-quantized linear layer and alpha-grid scale search.

The compute lives in libawq355.so (HIP kernels for gfx950 behind a C ABI,
include/awq355.h); this package is its ctypes binding.  Build the library with
``python -m bit_weight_only_quantize_amd.build``.  Accessing any API name
loads the library and raises ImportError if it is not built.
"""

_API = (
    "awq_quantize_pack", "awq_dequantize", "awq_linear", "awq_linear_ex", "awq_linear_ws", "awq_linear_noalloc",
    "awq_linear_fused", "awq_linear_fused_workspace_size", "AWQ_EPILOGUE_NONE",
    "AWQ_EPILOGUE_SILU_MUL", "AWQ_MAX_PARTS",
    "awq_linear_workspace_size", "awq_scale_search",
    "awq_scale_search_workspace_size", "AwqError", "config", "empty_packed", "lib",
    "AWQ_F16", "AWQ_BF16", "AWQ_F32", "AWQ_KERNEL_AUTO", "AWQ_KERNEL_GEMV",
    "AWQ_KERNEL_GEMM", "AWQ_KERNEL_BATCHED", "AWQ_GEMV_MAX_M", "AWQ_BATCHED_MAX_M", "EXPORTS",
    "LIB_PATH",
)

__all__ = list(_API)


def __getattr__(name):
    if name in _API:
        from . import binding
        return getattr(binding, name)
    raise AttributeError(name)
