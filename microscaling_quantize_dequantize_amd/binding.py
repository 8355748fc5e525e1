"""Thin ctypes binding over libmxqdq.so (argument marshalling only).

Every function has the name of the C entry point it calls and takes torch
tensors on the GPU: it checks that they are contiguous device tensors of the
expected dtype and shape, points the library at torch's current stream, and
passes raw pointers.  All computation happens in the HIP kernels; there is
no fallback: if the library is missing the import fails.

Tensor conventions: bf16 data is ``torch.bfloat16``; codes and scales are
``torch.uint8``; the rotation is an r x r tensor in the source dtype.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.environ.get("LIBMXQDQ", os.path.join(_HERE, "libmxqdq.so"))

if not os.path.exists(LIB_PATH):
    raise ImportError(f"libmxqdq.so not found at {LIB_PATH}; build it with "
                      "`python -m microscaling_quantize_dequantize_amd.build`")

_lib = ctypes.CDLL(LIB_PATH)

E2M1, E4M3 = 0, 1
BF16, F32 = 0, 1
ROWMAJOR, BLOCKED = 0, 1
_DTYPE = {torch.bfloat16: BF16, torch.float32: F32}

_vp, _i64, _int = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
_lib.mx_qdq.argtypes = [_int, _vp, _int, _i64, _i64, _vp, _int, _vp]
_lib.mx_quantize.argtypes = [_int, _vp, _i64, _i64, _vp, _int, _vp, _vp]
_lib.mx_dequantize.argtypes = [_int, _vp, _vp, _i64, _i64, _int, _vp]
_lib.mx_rotate.argtypes = [_vp, _int, _i64, _i64, _vp, _int, _vp]
_lib.mx_matmul.argtypes = [_int, _vp, _vp, _vp, _vp, _int, _i64, _i64, _i64, ctypes.c_float, _int, _vp]
_lib.mx_blocked_scales_bytes.argtypes = [_i64, _i64]
_lib.mx_blocked_scales_bytes.restype = _i64
_lib.mx_scales_to_blocked.argtypes = [_vp, _i64, _i64, _vp]
_lib.mx_quantize_blocked.argtypes = [_int, _vp, _i64, _i64, _vp, _int, _vp, _vp]
_lib.mx_nvfp4_quantize.argtypes = [_vp, _i64, _i64, _vp, _int, _vp, _vp, _vp]
_lib.mx_nvfp4_qdq.argtypes = [_vp, _i64, _i64, _vp, _int, _vp, _vp]
_lib.mx_nvfp4_dequantize.argtypes = [_vp, _vp, _i64, _i64, _vp, _int, _vp]
_lib.mx_set_stream.argtypes = [_vp]
_lib.mx_get_stream.restype = _vp
_lib.mx_status_string.argtypes = [_int]
_lib.mx_status_string.restype = ctypes.c_char_p
for _f in (_lib.mx_qdq, _lib.mx_quantize, _lib.mx_dequantize, _lib.mx_rotate, _lib.mx_matmul,
           _lib.mx_scales_to_blocked, _lib.mx_quantize_blocked, _lib.mx_nvfp4_quantize, _lib.mx_nvfp4_qdq,
           _lib.mx_nvfp4_dequantize):
    _f.restype = _int


class MXError(RuntimeError):
    def __init__(self, status: int):
        self.status = status
        super().__init__(f"libmxqdq status {status}: {mx_status_string(status)}")


def mx_status_string(status: int) -> str:
    return _lib.mx_status_string(int(status)).decode()


def mx_set_stream(stream) -> None:
    """Point the calling thread's library calls at a torch stream or a raw
    hipStream_t (int)."""
    _lib.mx_set_stream(ctypes.c_void_p(stream if isinstance(stream, int) else stream.cuda_stream))


def _dev(t: torch.Tensor, name: str) -> int:
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


def _rot(rot, dtype):
    if rot is None:
        return None, 0
    if rot.dtype != dtype or rot.dim() != 2 or rot.shape[0] != rot.shape[1]:
        raise ValueError("rotation must be a square matrix in the source dtype")
    return _dev(rot, "rot"), rot.shape[0]


def _mk(src: torch.Tensor) -> tuple[int, int]:
    if src.dim() != 2:
        raise ValueError("expected a 2-D [M, K] tensor")
    return src.shape[0], src.shape[1]


def _call(status: int) -> None:
    if status != 0:
        raise MXError(status)


def _stream() -> None:
    _lib.mx_set_stream(ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))


def mx_qdq(fmt: int, src: torch.Tensor, rot: torch.Tensor | None = None,
           dst: torch.Tensor | None = None) -> torch.Tensor:
    """Fused MX quantize-dequantize of src [M, K] (bf16 or fp32) into dst."""
    M, K = _mk(src)
    if src.dtype not in _DTYPE:
        raise TypeError("src must be bfloat16 or float32")
    if dst is None:
        dst = torch.empty_like(src)
    if dst.dtype != src.dtype or dst.shape != src.shape:
        raise ValueError("dst must match src in dtype and shape")
    rp, r = _rot(rot, src.dtype)
    _stream()
    _call(_lib.mx_qdq(fmt, _dev(src, "src"), _DTYPE[src.dtype], M, K, rp, r, _dev(dst, "dst")))
    return dst


def mx_quantize(fmt: int, src: torch.Tensor, rot: torch.Tensor | None = None,
                codes: torch.Tensor | None = None, scales: torch.Tensor | None = None):
    """Quantize bf16 src [M, K] -> (codes uint8 [M, K/2 or K], scales uint8 [M, K/32])."""
    M, K = _mk(src)
    if src.dtype != torch.bfloat16:
        raise TypeError("mx_quantize takes bfloat16 input")
    if codes is None:
        codes = torch.empty((M, K // 2 if fmt == E2M1 else K), dtype=torch.uint8, device=src.device)
    if scales is None:
        scales = torch.empty((M, K // 32), dtype=torch.uint8, device=src.device)
    rp, r = _rot(rot, src.dtype)
    _stream()
    _call(_lib.mx_quantize(fmt, _dev(src, "src"), M, K, rp, r, _dev(codes, "codes"),
                           _dev(scales, "scales")))
    return codes, scales


def mx_dequantize(fmt: int, codes: torch.Tensor, scales: torch.Tensor, K: int,
                  dtype: torch.dtype = torch.bfloat16, dst: torch.Tensor | None = None):
    """Dequantize codes + scales into a [M, K] tensor of `dtype`."""
    M = scales.shape[0]
    if dst is None:
        dst = torch.empty((M, K), dtype=dtype, device=codes.device)
    _stream()
    _call(_lib.mx_dequantize(fmt, _dev(codes, "codes"), _dev(scales, "scales"), M, K,
                             _DTYPE[dst.dtype], _dev(dst, "dst")))
    return dst


def mx_rotate(src: torch.Tensor, rot: torch.Tensor, dst: torch.Tensor | None = None):
    """The rotation step alone: fp32 [M, K] of per-chunk src . rot."""
    M, K = _mk(src)
    if dst is None:
        dst = torch.empty((M, K), dtype=torch.float32, device=src.device)
    rp, r = _rot(rot, src.dtype)
    _stream()
    _call(_lib.mx_rotate(_dev(src, "src"), _DTYPE[src.dtype], M, K, rp, r, _dev(dst, "dst")))
    return dst


def mx_blocked_scales_bytes(M: int, K: int) -> int:
    n = _lib.mx_blocked_scales_bytes(M, K)
    if n < 0:
        raise MXError(n)
    return n


def mx_scales_to_blocked(scales: torch.Tensor, K: int, blocked: torch.Tensor | None = None) -> torch.Tensor:
    """Row-major [M, K/32] scales -> the blocked layout (flat uint8)."""
    M = scales.shape[0]
    if blocked is None:
        blocked = torch.empty(mx_blocked_scales_bytes(M, K), dtype=torch.uint8, device=scales.device)
    _stream()
    _call(_lib.mx_scales_to_blocked(_dev(scales, "scales"), M, K, _dev(blocked, "blocked")))
    return blocked


def mx_quantize_blocked(fmt: int, src: torch.Tensor, rot: torch.Tensor | None = None,
                        codes: torch.Tensor | None = None, blocked: torch.Tensor | None = None):
    """Quantize bf16 src [M, K] -> (codes, scales in the blocked layout)."""
    M, K = _mk(src)
    if src.dtype != torch.bfloat16:
        raise TypeError("mx_quantize_blocked takes bfloat16 input")
    if codes is None:
        codes = torch.empty((M, K // 2 if fmt == E2M1 else K), dtype=torch.uint8, device=src.device)
    if blocked is None:
        blocked = torch.empty(mx_blocked_scales_bytes(M, K), dtype=torch.uint8, device=src.device)
    rp, r = _rot(rot, src.dtype)
    _stream()
    _call(_lib.mx_quantize_blocked(fmt, _dev(src, "src"), M, K, rp, r, _dev(codes, "codes"),
                                   _dev(blocked, "blocked")))
    return codes, blocked


def mx_matmul(fmt: int, a_codes: torch.Tensor, a_scales: torch.Tensor, b_codes: torch.Tensor,
              b_scales: torch.Tensor, K: int, alpha: float = 1.0, dtype: torch.dtype = torch.bfloat16,
              c: torch.Tensor | None = None, scale_layout: int = ROWMAJOR):
    """[M, N] = alpha * A_dq . B_dq^T from MX codes and scales (A [M, K], B [N, K]);
    the row counts come from the codes."""
    M, N = a_codes.shape[0], b_codes.shape[0]
    if c is None:
        c = torch.empty((M, N), dtype=dtype, device=a_codes.device)
    if c.dtype not in _DTYPE or tuple(c.shape) != (M, N):
        raise ValueError("c must be a bfloat16 or float32 [M, N] tensor")
    _stream()
    _call(_lib.mx_matmul(fmt, _dev(a_codes, "a_codes"), _dev(a_scales, "a_scales"), _dev(b_codes, "b_codes"),
                         _dev(b_scales, "b_scales"), scale_layout, M, N, K, float(alpha), _DTYPE[c.dtype],
                         _dev(c, "c")))
    return c


def _gscale(global_scale: torch.Tensor) -> int:
    if global_scale.dtype != torch.float32 or global_scale.numel() != 1:
        raise ValueError("global_scale must be a one-element float32 tensor")
    return _dev(global_scale, "global_scale")


def mx_nvfp4_quantize(src: torch.Tensor, global_scale: torch.Tensor, rot: torch.Tensor | None = None,
                      codes: torch.Tensor | None = None, scales: torch.Tensor | None = None):
    """NVFP4 quantize of bf16 src [M, K] -> (E2M1 codes [M, K/2], E4M3 scale bytes [M, K/16])."""
    M, K = _mk(src)
    if src.dtype != torch.bfloat16:
        raise TypeError("mx_nvfp4_quantize takes bfloat16 input")
    if codes is None:
        codes = torch.empty((M, K // 2), dtype=torch.uint8, device=src.device)
    if scales is None:
        scales = torch.empty((M, K // 16), dtype=torch.uint8, device=src.device)
    rp, r = _rot(rot, src.dtype)
    _stream()
    _call(_lib.mx_nvfp4_quantize(_dev(src, "src"), M, K, rp, r, _gscale(global_scale), _dev(codes, "codes"),
                                 _dev(scales, "scales")))
    return codes, scales


def mx_nvfp4_qdq(src: torch.Tensor, global_scale: torch.Tensor, rot: torch.Tensor | None = None,
                 dst: torch.Tensor | None = None) -> torch.Tensor:
    """NVFP4 quantize-dequantize of bf16 src [M, K] into bf16 dst."""
    M, K = _mk(src)
    if src.dtype != torch.bfloat16:
        raise TypeError("mx_nvfp4_qdq takes bfloat16 input")
    if dst is None:
        dst = torch.empty_like(src)
    if dst.dtype != src.dtype or dst.shape != src.shape:
        raise ValueError("dst must match src in dtype and shape")
    rp, r = _rot(rot, src.dtype)
    _stream()
    _call(_lib.mx_nvfp4_qdq(_dev(src, "src"), M, K, rp, r, _gscale(global_scale), _dev(dst, "dst")))
    return dst


def mx_nvfp4_dequantize(codes: torch.Tensor, scales: torch.Tensor, K: int, global_scale: torch.Tensor,
                        dtype: torch.dtype = torch.bfloat16, dst: torch.Tensor | None = None):
    """NVFP4 codes + E4M3 scales -> [M, K] of `dtype`."""
    M = scales.shape[0]
    if dst is None:
        dst = torch.empty((M, K), dtype=dtype, device=codes.device)
    _stream()
    _call(_lib.mx_nvfp4_dequantize(_dev(codes, "codes"), _dev(scales, "scales"), M, K, _gscale(global_scale),
                                   _DTYPE[dst.dtype], _dev(dst, "dst")))
    return dst


def raw():
    """The ctypes library handle (for callers passing raw pointers)."""
    return _lib
