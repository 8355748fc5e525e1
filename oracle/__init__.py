"""CPU oracle for MX quantize / dequantize (plain scalar C in IEEE double).

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and
the CPU-baseline leg of ``bench.py`` may import this package.  The product
path (the HIP library and its Python binding) never imports, links or calls
it, and the two share no code.

This module builds ``mxoracle.c`` with gcc into ``libmxoracle.so`` and wraps
it with ctypes over numpy arrays.  ``threads > 1`` splits rows over a thread
pool; each thread runs the unchanged scalar C code on its own row range
(ctypes releases the GIL during the call).

What each C function computes, and which passage of the pages it follows, is
stated in ``mxoracle.h``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "mxoracle.c")
_LIB = os.path.join(_HERE, "libmxoracle.so")

E2M1, E4M3 = 0, 1
BF16, F32 = 0, 1

_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (strict IEEE: no -ffast-math)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.check_call([
            "gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-Wall", "-Wextra",
            "-fno-fast-math", "-ffp-contract=off", "-o", tmp, _SRC, "-lm",
        ])
        os.replace(tmp, _LIB)
    return _LIB


def lib():
    global _lib
    if _lib is None:
        path = os.environ.get("MXORACLE_LIB")  # mutation tests load a planted copy
        if path is None:
            if not os.path.exists(_LIB):
                build(force=False)
            path = _LIB
        L = ctypes.CDLL(path)
        vp, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
        L.orc_bf16_value.argtypes = [ctypes.c_uint16]
        L.orc_bf16_value.restype = ctypes.c_double
        L.orc_f32_value.argtypes = [ctypes.c_uint32]
        L.orc_f32_value.restype = ctypes.c_double
        L.orc_bf16_from_double.argtypes = [ctypes.c_double]
        L.orc_bf16_from_double.restype = ctypes.c_uint16
        L.orc_f32_from_double.argtypes = [ctypes.c_double]
        L.orc_f32_from_double.restype = ctypes.c_uint32
        L.orc_scale_exponent.argtypes = [i32, ctypes.c_double]
        L.orc_scale_exponent.restype = i32
        L.orc_encode.argtypes = [i32, ctypes.c_double, i32]
        L.orc_encode.restype = i32
        L.orc_decode.argtypes = [i32, i32]
        L.orc_decode.restype = ctypes.c_double
        L.orc_scale_exponent_n.argtypes = [i32, vp, i64, vp]
        L.orc_scale_exponent_n.restype = None
        L.orc_encode_n.argtypes = [i32, vp, vp, i64, vp]
        L.orc_encode_n.restype = None
        L.orc_qdq_value_n.argtypes = [i32, vp, vp, i64, vp]
        L.orc_qdq_value_n.restype = None
        L.orc_rotate.argtypes = [vp, i32, i64, i64, vp, i32, vp, vp]
        L.orc_rotate.restype = i32
        L.orc_qdq.argtypes = [i32, vp, i32, i64, i64, vp, i32, vp]
        L.orc_qdq.restype = i32
        L.orc_quantize.argtypes = [i32, vp, i64, i64, vp, i32, vp, vp]
        L.orc_quantize.restype = i32
        L.orc_dequantize.argtypes = [i32, vp, vp, i64, i64, i32, vp]
        L.orc_dequantize.restype = i32
        L.orc_dequantize_f64.argtypes = [i32, vp, vp, i64, i64, vp]
        L.orc_dequantize_f64.restype = i32
        L.orc_blocked_size.argtypes = [i64, i64]
        L.orc_blocked_size.restype = i64
        L.orc_scales_to_blocked.argtypes = [vp, i64, i64, vp]
        L.orc_scales_to_blocked.restype = i32
        f32 = ctypes.c_float
        L.orc_nv_scale_byte_n.argtypes = [f32, vp, i64, vp]
        L.orc_nv_scale_byte_n.restype = None
        L.orc_nv_code_n.argtypes = [f32, vp, vp, i64, vp]
        L.orc_nv_code_n.restype = None
        L.orc_nv_value_n.argtypes = [f32, vp, vp, i64, vp]
        L.orc_nv_value_n.restype = None
        L.orc_nv_quantize.argtypes = [vp, i64, i64, vp, i32, f32, vp, vp]
        L.orc_nv_quantize.restype = i32
        L.orc_nv_qdq.argtypes = [vp, i64, i64, vp, i32, f32, vp]
        L.orc_nv_qdq.restype = i32
        L.orc_nv_dequantize.argtypes = [vp, vp, i64, i64, f32, i32, vp]
        L.orc_nv_dequantize.restype = i32
        _lib = L
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data


def _dtype_code(a: np.ndarray) -> int:
    if a.dtype == np.uint16:
        return BF16
    if a.dtype in (np.uint32, np.float32):
        return F32
    raise TypeError(f"oracle source must be bf16 bits (uint16) or float32, got {a.dtype}")


def _row_ranges(M: int, threads: int):
    threads = max(1, min(threads, M)) if M > 0 else 1
    step = (M + threads - 1) // threads if M > 0 else 0
    return [(r0, min(M, r0 + step)) for r0 in range(0, M, step)] if M > 0 else []


def _run_rows(fn, M: int, threads: int):
    ranges = _row_ranges(M, threads)
    if len(ranges) <= 1:
        for r0, r1 in ranges:
            fn(r0, r1)
        return
    with ThreadPoolExecutor(max_workers=len(ranges)) as ex:
        list(ex.map(lambda rr: fn(*rr), ranges))


# ---- scalar / batch element steps -----------------------------------------

def bf16_value(bits: int) -> float:
    return lib().orc_bf16_value(int(bits))


def f32_value(bits: int) -> float:
    return lib().orc_f32_value(int(bits))


def bf16_from_double(x: float) -> int:
    return lib().orc_bf16_from_double(float(x))


def f32_from_double(x: float) -> int:
    return lib().orc_f32_from_double(float(x))


def scale_exponent(fmt: int, amax: float) -> int:
    return lib().orc_scale_exponent(fmt, float(amax))


def encode(fmt: int, y: float, s: int) -> int:
    return lib().orc_encode(fmt, float(y), int(s))


def decode(fmt: int, code: int) -> float:
    return lib().orc_decode(fmt, int(code))


def scale_exponent_n(fmt: int, amax: np.ndarray) -> np.ndarray:
    amax = np.ascontiguousarray(amax, dtype=np.float64)
    out = np.empty(amax.shape, dtype=np.int32)
    lib().orc_scale_exponent_n(fmt, _ptr(amax), amax.size, _ptr(out))
    return out


def encode_n(fmt: int, y: np.ndarray, s: np.ndarray) -> np.ndarray:
    y = np.ascontiguousarray(y, dtype=np.float64)
    s = np.ascontiguousarray(np.broadcast_to(s, y.shape), dtype=np.int32)
    out = np.empty(y.shape, dtype=np.uint8)
    lib().orc_encode_n(fmt, _ptr(y), _ptr(s), y.size, _ptr(out))
    return out


def qdq_value_n(fmt: int, y: np.ndarray, s: np.ndarray) -> np.ndarray:
    y = np.ascontiguousarray(y, dtype=np.float64)
    s = np.ascontiguousarray(np.broadcast_to(s, y.shape), dtype=np.int32)
    out = np.empty(y.shape, dtype=np.float64)
    lib().orc_qdq_value_n(fmt, _ptr(y), _ptr(s), y.size, _ptr(out))
    return out


# ---- whole-matrix operations ----------------------------------------------

def _check_rot(rot, rot_size, dt):
    if rot_size == 0:
        return None
    rot = np.ascontiguousarray(rot)
    if _dtype_code(rot) != dt or rot.size != rot_size * rot_size:
        raise ValueError("rotation must be r x r in the source dtype")
    return rot


def rotate(src: np.ndarray, rot=None, rot_size: int = 0, threads: int = 1):
    """Rotated values y (float64) and band weights beta, shaped like src."""
    src = np.ascontiguousarray(src)
    dt = _dtype_code(src)
    M, K = src.shape
    rot = _check_rot(rot, rot_size, dt)
    y = np.empty((M, K), dtype=np.float64)
    beta = np.empty((M, K), dtype=np.float64)

    def run(r0, r1):
        rc = lib().orc_rotate(src[r0:].ctypes.data, dt, r1 - r0, K, _ptr(rot),
                              rot_size, y[r0:].ctypes.data, beta[r0:].ctypes.data)
        if rc != 0:
            raise ValueError("oracle rejected the arguments")

    _run_rows(run, M, threads)
    return y, beta


def qdq(fmt: int, src: np.ndarray, rot=None, rot_size: int = 0, threads: int = 1):
    """Fused quantize-dequantize; returns an array of src's dtype."""
    src = np.ascontiguousarray(src)
    dt = _dtype_code(src)
    M, K = src.shape
    rot = _check_rot(rot, rot_size, dt)
    dst = np.empty_like(src)

    def run(r0, r1):
        rc = lib().orc_qdq(fmt, src[r0:].ctypes.data, dt, r1 - r0, K, _ptr(rot),
                           rot_size, dst[r0:].ctypes.data)
        if rc != 0:
            raise ValueError("oracle rejected the arguments")

    _run_rows(run, M, threads)
    return dst


def quantize(fmt: int, src: np.ndarray, rot=None, rot_size: int = 0, threads: int = 1):
    """Quantize bf16 bits [M,K] -> (codes, scales)."""
    src = np.ascontiguousarray(src)
    if src.dtype != np.uint16:
        raise TypeError("quantize takes bf16 bits (uint16)")
    M, K = src.shape
    rot = _check_rot(rot, rot_size, BF16)
    codes = np.empty((M, K // 2 if fmt == E2M1 else K), dtype=np.uint8)
    scales = np.empty((M, K // 32), dtype=np.uint8)

    def run(r0, r1):
        rc = lib().orc_quantize(fmt, src[r0:].ctypes.data, r1 - r0, K, _ptr(rot),
                                rot_size, codes[r0:].ctypes.data,
                                scales[r0:].ctypes.data)
        if rc != 0:
            raise ValueError("oracle rejected the arguments")

    _run_rows(run, M, threads)
    return codes, scales


def dequantize(fmt: int, codes: np.ndarray, scales: np.ndarray, K: int,
               dst_dtype: int = BF16, threads: int = 1):
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.uint8)
    M = scales.shape[0]
    dst = np.empty((M, K), dtype=np.uint16 if dst_dtype == BF16 else np.uint32)

    def run(r0, r1):
        rc = lib().orc_dequantize(fmt, codes[r0:].ctypes.data,
                                  scales[r0:].ctypes.data, r1 - r0, K, dst_dtype,
                                  dst[r0:].ctypes.data)
        if rc != 0:
            raise ValueError("oracle rejected the arguments")

    _run_rows(run, M, threads)
    return dst


def dequantize_f64(fmt: int, codes: np.ndarray, scales: np.ndarray, K: int, threads: int = 1):
    """Exact dequantized values (float64 [M, K]), not rounded to a storage type."""
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.uint8)
    M = scales.shape[0]
    dst = np.empty((M, K), dtype=np.float64)

    def run(r0, r1):
        rc = lib().orc_dequantize_f64(fmt, codes[r0:].ctypes.data, scales[r0:].ctypes.data,
                                      r1 - r0, K, dst[r0:].ctypes.data)
        if rc != 0:
            raise ValueError("oracle rejected the arguments")

    _run_rows(run, M, threads)
    return dst


def matmul(fmt: int, a_codes, a_scales, b_codes, b_scales, K: int, threads: int = 1):
    """MX GEMM reference: float64 A_dq . B_dq^T for A [M, K] and B [N, K] in the
    quantized layout ("Add QuTLASS support to vLLM", review of the MXFP4 test:
    the kernel's output is compared with the dequantized operands multiplied in
    high precision).  The two exact dequantizations are followed by one library
    matmul in float64."""
    a = dequantize_f64(fmt, a_codes, a_scales, K, threads)
    b = dequantize_f64(fmt, b_codes, b_scales, K, threads)
    return a @ b.T


def blocked_size(M: int, K: int) -> int:
    return int(lib().orc_blocked_size(M, K))


def scales_to_blocked(scales: np.ndarray, K: int) -> np.ndarray:
    """Row-major [M, K/32] E8M0 scales -> the blocked layout (uint8, flat)."""
    scales = np.ascontiguousarray(scales, dtype=np.uint8)
    M = scales.shape[0]
    out = np.empty(blocked_size(M, K), dtype=np.uint8)
    if lib().orc_scales_to_blocked(scales.ctypes.data, M, K, out.ctypes.data) != 0:
        raise ValueError("oracle rejected the arguments")
    return out


# ---- NVFP4 (a reading; steps in mxoracle.h) -----------------------------------

def nv_scale_byte_n(g: float, amax: np.ndarray) -> np.ndarray:
    amax = np.ascontiguousarray(amax, dtype=np.float32)
    out = np.empty(amax.shape, dtype=np.uint8)
    lib().orc_nv_scale_byte_n(float(np.float32(g)), amax.ctypes.data, amax.size, out.ctypes.data)
    return out


def nv_code_n(g: float, sb: np.ndarray, x: np.ndarray) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float32)
    sb = np.ascontiguousarray(np.broadcast_to(sb, x.shape), dtype=np.uint8)
    out = np.empty(x.shape, dtype=np.uint8)
    lib().orc_nv_code_n(float(np.float32(g)), sb.ctypes.data, x.ctypes.data, x.size, out.ctypes.data)
    return out


def nv_value_n(g: float, sb: np.ndarray, codes: np.ndarray) -> np.ndarray:
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    sb = np.ascontiguousarray(np.broadcast_to(sb, codes.shape), dtype=np.uint8)
    out = np.empty(codes.shape, dtype=np.float32)
    lib().orc_nv_value_n(float(np.float32(g)), sb.ctypes.data, codes.ctypes.data, codes.size, out.ctypes.data)
    return out


def nv_quantize(src: np.ndarray, g: float, rot=None, rot_size: int = 0, threads: int = 1):
    """NVFP4 quantize of bf16 bits [M, K] -> (codes [M, K/2], E4M3 scale bytes [M, K/16])."""
    src = np.ascontiguousarray(src, dtype=np.uint16)
    M, K = src.shape
    codes = np.empty((M, K // 2), dtype=np.uint8)
    scales = np.empty((M, K // 16), dtype=np.uint8)
    rp = None if rot is None else np.ascontiguousarray(rot, dtype=np.uint16)

    def run(r0, r1):
        rc = lib().orc_nv_quantize(src[r0:].ctypes.data, r1 - r0, K, None if rp is None else rp.ctypes.data,
                                   rot_size, float(np.float32(g)), codes[r0:].ctypes.data, scales[r0:].ctypes.data)
        if rc != 0:
            raise ValueError("oracle rejected the arguments")

    _run_rows(run, M, threads)
    return codes, scales


def nv_qdq(src: np.ndarray, g: float, rot=None, rot_size: int = 0, threads: int = 1) -> np.ndarray:
    """NVFP4 quantize-dequantize of bf16 bits [M, K] -> bf16 bits."""
    src = np.ascontiguousarray(src, dtype=np.uint16)
    M, K = src.shape
    dst = np.empty((M, K), dtype=np.uint16)
    rp = None if rot is None else np.ascontiguousarray(rot, dtype=np.uint16)

    def run(r0, r1):
        rc = lib().orc_nv_qdq(src[r0:].ctypes.data, r1 - r0, K, None if rp is None else rp.ctypes.data,
                              rot_size, float(np.float32(g)), dst[r0:].ctypes.data)
        if rc != 0:
            raise ValueError("oracle rejected the arguments")

    _run_rows(run, M, threads)
    return dst


def nv_dequantize(codes: np.ndarray, scales: np.ndarray, K: int, g: float, dst_dtype: int = BF16,
                  threads: int = 1) -> np.ndarray:
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.uint8)
    M = scales.shape[0]
    dst = np.empty((M, K), dtype=np.uint16 if dst_dtype == BF16 else np.uint32)

    def run(r0, r1):
        rc = lib().orc_nv_dequantize(codes[r0:].ctypes.data, scales[r0:].ctypes.data, r1 - r0, K,
                                     float(np.float32(g)), dst_dtype, dst[r0:].ctypes.data)
        if rc != 0:
            raise ValueError("oracle rejected the arguments")

    _run_rows(run, M, threads)
    return dst
