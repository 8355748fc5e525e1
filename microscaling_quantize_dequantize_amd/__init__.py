"""libmxqdq: MX (MXFP4 / MXFP8) quantize-dequantize on AMD Instinct MI355X.

The compute path is the C-ABI HIP library ``libmxqdq.so`` (built for gfx950
from ``csrc/``); ``binding`` is a thin ctypes layer over it with the same
entry-point names.  The binding is loaded on first use so that importing
``workloads`` does not need the library.
"""

__all__ = ["mx_qdq", "mx_quantize", "mx_dequantize", "mx_rotate", "mx_matmul",
           "mx_blocked_scales_bytes", "mx_scales_to_blocked", "mx_quantize_blocked",
           "mx_nvfp4_quantize", "mx_nvfp4_qdq", "mx_nvfp4_dequantize",
           "mx_set_stream", "mx_status_string", "MXError",
           "E2M1", "E4M3", "BF16", "F32", "ROWMAJOR", "BLOCKED"]


def __getattr__(name):
    if name in __all__:
        from . import binding
        return getattr(binding, name)
    raise AttributeError(name)
