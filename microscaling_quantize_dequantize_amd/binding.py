"""Thin ctypes binding over libmxqdq.so (argument marshalling only).

Every function has the name of the C entry point it calls and takes torch
tensors on the GPU.  Before anything is enqueued it checks every tensor it
is handed: dtype and exact shape first (codes [M, K/2] or [M, K], scales
[M, K/32] or [M, K/16] for NVFP4, blocked scales at least the blocked size,
outputs [M, K] in the stated dtype), then that each is a contiguous tensor
on the current device; a mismatch raises ValueError or TypeError.  It then points the
library at torch's current stream and passes raw pointers.  All computation
happens in the HIP kernels; there is no fallback: if the library is missing
the import fails.

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
    if t.device.index != torch.cuda.current_device():
        # the library launches on the current device (and torch's stream there)
        raise ValueError(f"{name} is on {t.device}, the current device is cuda:{torch.cuda.current_device()}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


def _want(t, name: str, dtype: torch.dtype, shape) -> None:
    """t must be a tensor of exactly this dtype and shape (checked before any
    pointer is taken, so that a wrong buffer never reaches a kernel)."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


def _want_blocked(t, name: str, M: int, K: int) -> None:
    """Blocked scales: a flat uint8 tensor of at least the blocked size."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if t.dtype != torch.uint8 or t.dim() != 1:
        raise ValueError(f"{name} must be a flat uint8 tensor")
    need = mx_blocked_scales_bytes(M, K)
    if t.numel() < need:
        raise ValueError(f"{name} holds {t.numel()} bytes; the blocked layout of {M} x {K} needs {need}")


def _rot(rot, dtype):
    if rot is None:
        return None, 0
    if not isinstance(rot, torch.Tensor) or rot.dtype != dtype or rot.dim() != 2 or rot.shape[0] != rot.shape[1]:
        raise ValueError("rotation must be a square matrix in the source dtype")
    return _dev(rot, "rot"), rot.shape[0]


def _mk(src: torch.Tensor) -> tuple[int, int]:
    if not isinstance(src, torch.Tensor):
        raise TypeError("expected a torch tensor")
    if src.dim() != 2:
        raise ValueError("expected a 2-D [M, K] tensor")
    return src.shape[0], src.shape[1]


def _code_cols(fmt: int, K: int) -> int:
    return K // 2 if fmt == E2M1 else K


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
    _want(dst, "dst", src.dtype, (M, K))
    ps, pd = _dev(src, "src"), _dev(dst, "dst")
    rp, r = _rot(rot, src.dtype)
    _stream()
    _call(_lib.mx_qdq(fmt, ps, _DTYPE[src.dtype], M, K, rp, r, pd))
    return dst


def mx_quantize(fmt: int, src: torch.Tensor, rot: torch.Tensor | None = None,
                codes: torch.Tensor | None = None, scales: torch.Tensor | None = None):
    """Quantize bf16 src [M, K] -> (codes uint8 [M, K/2 or K], scales uint8 [M, K/32])."""
    M, K = _mk(src)
    if src.dtype != torch.bfloat16:
        raise TypeError("mx_quantize takes bfloat16 input")
    if codes is None:
        codes = torch.empty((M, _code_cols(fmt, K)), dtype=torch.uint8, device=src.device)
    if scales is None:
        scales = torch.empty((M, K // 32), dtype=torch.uint8, device=src.device)
    _want(codes, "codes", torch.uint8, (M, _code_cols(fmt, K)))
    _want(scales, "scales", torch.uint8, (M, K // 32))
    ps, pc, pq = _dev(src, "src"), _dev(codes, "codes"), _dev(scales, "scales")
    rp, r = _rot(rot, src.dtype)
    _stream()
    _call(_lib.mx_quantize(fmt, ps, M, K, rp, r, pc, pq))
    return codes, scales


def mx_dequantize(fmt: int, codes: torch.Tensor, scales: torch.Tensor, K: int,
                  dtype: torch.dtype = torch.bfloat16, dst: torch.Tensor | None = None):
    """Dequantize codes [M, K/2 or K] + row-major scales [M, K/32] into a
    [M, K] tensor of `dtype`."""
    if not isinstance(scales, torch.Tensor) or scales.dim() != 2:
        raise ValueError("scales must be a 2-D [M, K/32] uint8 tensor")
    M = scales.shape[0]
    _want(scales, "scales", torch.uint8, (M, K // 32))
    _want(codes, "codes", torch.uint8, (M, _code_cols(fmt, K)))
    if dst is None:
        dst = torch.empty((M, K), dtype=dtype, device=codes.device)
    if dst.dtype not in _DTYPE:
        raise ValueError("dst must be bfloat16 or float32")
    _want(dst, "dst", dst.dtype, (M, K))
    pc, pq, pd = _dev(codes, "codes"), _dev(scales, "scales"), _dev(dst, "dst")
    _stream()
    _call(_lib.mx_dequantize(fmt, pc, pq, M, K, _DTYPE[dst.dtype], pd))
    return dst


def mx_rotate(src: torch.Tensor, rot: torch.Tensor, dst: torch.Tensor | None = None):
    """The rotation step alone: fp32 [M, K] of per-chunk src . rot."""
    M, K = _mk(src)
    if src.dtype not in _DTYPE:
        raise TypeError("src must be bfloat16 or float32")
    if dst is None:
        dst = torch.empty((M, K), dtype=torch.float32, device=src.device)
    _want(dst, "dst", torch.float32, (M, K))
    ps, pd = _dev(src, "src"), _dev(dst, "dst")
    rp, r = _rot(rot, src.dtype)
    _stream()
    _call(_lib.mx_rotate(ps, _DTYPE[src.dtype], M, K, rp, r, pd))
    return dst


def mx_blocked_scales_bytes(M: int, K: int) -> int:
    n = _lib.mx_blocked_scales_bytes(M, K)
    if n < 0:
        raise MXError(n)
    return n


def mx_scales_to_blocked(scales: torch.Tensor, K: int, blocked: torch.Tensor | None = None) -> torch.Tensor:
    """Row-major [M, K/32] scales -> the blocked layout (flat uint8)."""
    if not isinstance(scales, torch.Tensor) or scales.dim() != 2:
        raise ValueError("scales must be a 2-D [M, K/32] uint8 tensor")
    M = scales.shape[0]
    _want(scales, "scales", torch.uint8, (M, K // 32))
    if blocked is None:
        blocked = torch.empty(mx_blocked_scales_bytes(M, K), dtype=torch.uint8, device=scales.device)
    _want_blocked(blocked, "blocked", M, K)
    pq, pb = _dev(scales, "scales"), _dev(blocked, "blocked")
    _stream()
    _call(_lib.mx_scales_to_blocked(pq, M, K, pb))
    return blocked


def mx_quantize_blocked(fmt: int, src: torch.Tensor, rot: torch.Tensor | None = None,
                        codes: torch.Tensor | None = None, blocked: torch.Tensor | None = None):
    """Quantize bf16 src [M, K] -> (codes, scales in the blocked layout)."""
    M, K = _mk(src)
    if src.dtype != torch.bfloat16:
        raise TypeError("mx_quantize_blocked takes bfloat16 input")
    if codes is None:
        codes = torch.empty((M, _code_cols(fmt, K)), dtype=torch.uint8, device=src.device)
    if blocked is None:
        blocked = torch.empty(mx_blocked_scales_bytes(M, K), dtype=torch.uint8, device=src.device)
    _want(codes, "codes", torch.uint8, (M, _code_cols(fmt, K)))
    _want_blocked(blocked, "blocked", M, K)
    ps, pc, pb = _dev(src, "src"), _dev(codes, "codes"), _dev(blocked, "blocked")
    rp, r = _rot(rot, src.dtype)
    _stream()
    _call(_lib.mx_quantize_blocked(fmt, ps, M, K, rp, r, pc, pb))
    return codes, blocked


def _want_scales(t, name: str, layout: int, rows: int, K: int) -> None:
    if layout == BLOCKED:
        _want_blocked(t, name, rows, K)
    else:
        _want(t, name, torch.uint8, (rows, K // 32))


def mx_matmul(fmt: int, a_codes: torch.Tensor, a_scales: torch.Tensor, b_codes: torch.Tensor,
              b_scales: torch.Tensor, K: int, alpha: float = 1.0, dtype: torch.dtype = torch.bfloat16,
              c: torch.Tensor | None = None, scale_layout: int = ROWMAJOR):
    """[M, N] = alpha * A_dq . B_dq^T from MX codes and scales (A [M, K], B [N, K]);
    the row counts come from the codes."""
    for t, name in ((a_codes, "a_codes"), (b_codes, "b_codes")):
        if not isinstance(t, torch.Tensor) or t.dim() != 2:
            raise ValueError(f"{name} must be a 2-D uint8 tensor")
    M, N = a_codes.shape[0], b_codes.shape[0]
    _want(a_codes, "a_codes", torch.uint8, (M, _code_cols(fmt, K)))
    _want(b_codes, "b_codes", torch.uint8, (N, _code_cols(fmt, K)))
    if scale_layout in (ROWMAJOR, BLOCKED):
        _want_scales(a_scales, "a_scales", scale_layout, M, K)
        _want_scales(b_scales, "b_scales", scale_layout, N, K)
    if c is None:
        c = torch.empty((M, N), dtype=dtype, device=a_codes.device)
    if not isinstance(c, torch.Tensor) or c.dtype not in _DTYPE or tuple(c.shape) != (M, N):
        raise ValueError("c must be a bfloat16 or float32 [M, N] tensor")
    pa, pas, pb, pbs, pc = (_dev(a_codes, "a_codes"), _dev(a_scales, "a_scales"), _dev(b_codes, "b_codes"),
                            _dev(b_scales, "b_scales"), _dev(c, "c"))
    _stream()
    _call(_lib.mx_matmul(fmt, pa, pas, pb, pbs, scale_layout, M, N, K, float(alpha), _DTYPE[c.dtype], pc))
    return c


def _want_g(global_scale) -> None:
    if not isinstance(global_scale, torch.Tensor) or global_scale.dtype != torch.float32 \
            or global_scale.numel() != 1:
        raise ValueError("global_scale must be a one-element float32 tensor")


def _gscale(global_scale: torch.Tensor) -> int:
    _want_g(global_scale)
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
    _want(codes, "codes", torch.uint8, (M, K // 2))
    _want(scales, "scales", torch.uint8, (M, K // 16))
    _want_g(global_scale)
    ps, pc, pq, pg = _dev(src, "src"), _dev(codes, "codes"), _dev(scales, "scales"), _gscale(global_scale)
    rp, r = _rot(rot, src.dtype)
    _stream()
    _call(_lib.mx_nvfp4_quantize(ps, M, K, rp, r, pg, pc, pq))
    return codes, scales


def mx_nvfp4_qdq(src: torch.Tensor, global_scale: torch.Tensor, rot: torch.Tensor | None = None,
                 dst: torch.Tensor | None = None) -> torch.Tensor:
    """NVFP4 quantize-dequantize of bf16 src [M, K] into bf16 dst."""
    M, K = _mk(src)
    if src.dtype != torch.bfloat16:
        raise TypeError("mx_nvfp4_qdq takes bfloat16 input")
    if dst is None:
        dst = torch.empty_like(src)
    _want(dst, "dst", torch.bfloat16, (M, K))
    _want_g(global_scale)
    ps, pd, pg = _dev(src, "src"), _dev(dst, "dst"), _gscale(global_scale)
    rp, r = _rot(rot, src.dtype)
    _stream()
    _call(_lib.mx_nvfp4_qdq(ps, M, K, rp, r, pg, pd))
    return dst


def mx_nvfp4_dequantize(codes: torch.Tensor, scales: torch.Tensor, K: int, global_scale: torch.Tensor,
                        dtype: torch.dtype = torch.bfloat16, dst: torch.Tensor | None = None):
    """NVFP4 codes [M, K/2] + E4M3 scales [M, K/16] -> [M, K] of `dtype`."""
    if not isinstance(scales, torch.Tensor) or scales.dim() != 2:
        raise ValueError("scales must be a 2-D [M, K/16] uint8 tensor")
    M = scales.shape[0]
    _want(scales, "scales", torch.uint8, (M, K // 16))
    _want(codes, "codes", torch.uint8, (M, K // 2))
    if dst is None:
        dst = torch.empty((M, K), dtype=dtype, device=codes.device)
    if dst.dtype not in _DTYPE:
        raise ValueError("dst must be bfloat16 or float32")
    _want(dst, "dst", dst.dtype, (M, K))
    _want_g(global_scale)
    pc, pq, pd, pg = _dev(codes, "codes"), _dev(scales, "scales"), _dev(dst, "dst"), _gscale(global_scale)
    _stream()
    _call(_lib.mx_nvfp4_dequantize(pc, pq, M, K, pg, _DTYPE[dst.dtype], pd))
    return dst


def raw():
    """The ctypes library handle (for callers passing raw pointers)."""
    return _lib
