"""The C-ABI library loads, exports every declared symbol, and rejects bad
arguments on the host before any GPU work (CPU only: no kernel is launched)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "libmxqdq.h")
LIB = os.path.join(ROOT, "microscaling_quantize_dequantize_amd", "libmxqdq.so")

MX_OK, MX_EFMT, MX_EDTYPE, MX_ESHAPE, MX_EROT, MX_ENULL, MX_EALIGN, MX_ELAUNCH, MX_ELAYOUT = 0, -1, -2, -3, -4, -5, -6, -7, -8


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        from microscaling_quantize_dequantize_amd import build
        build.build()
    L = ctypes.CDLL(LIB)
    vp, i64, i = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    L.mx_qdq.argtypes = [i, vp, i, i64, i64, vp, i, vp]
    L.mx_quantize.argtypes = [i, vp, i64, i64, vp, i, vp, vp]
    L.mx_dequantize.argtypes = [i, vp, vp, i64, i64, i, vp]
    L.mx_rotate.argtypes = [vp, i, i64, i64, vp, i, vp]
    L.mx_matmul.argtypes = [i, vp, vp, vp, vp, i, i64, i64, i64, ctypes.c_float, i, vp]
    L.mx_blocked_scales_bytes.argtypes = [i64, i64]
    L.mx_blocked_scales_bytes.restype = i64
    L.mx_scales_to_blocked.argtypes = [vp, i64, i64, vp]
    L.mx_quantize_blocked.argtypes = [i, vp, i64, i64, vp, i, vp, vp]
    L.mx_nvfp4_quantize.argtypes = [vp, i64, i64, vp, i, vp, vp, vp]
    L.mx_nvfp4_qdq.argtypes = [vp, i64, i64, vp, i, vp, vp]
    L.mx_nvfp4_dequantize.argtypes = [vp, vp, i64, i64, vp, i, vp]
    L.mx_set_stream.argtypes = [vp]
    L.mx_get_stream.restype = vp
    L.mx_status_string.argtypes = [i]
    L.mx_status_string.restype = ctypes.c_char_p
    return L


def declared_symbols():
    text = open(HEADER).read()
    return re.findall(r"MX_API\s+[\w\s\*]+?\b(mx_\w+)\s*\(", text)


def test_header_declares_the_boundary():
    names = set(declared_symbols())
    assert {"mx_qdq", "mx_quantize", "mx_dequantize", "mx_rotate", "mx_matmul", "mx_blocked_scales_bytes",
            "mx_scales_to_blocked", "mx_quantize_blocked", "mx_nvfp4_quantize", "mx_nvfp4_qdq",
            "mx_nvfp4_dequantize", "mx_set_stream",
            "mx_get_stream", "mx_status_string"} <= names


def test_library_exports_every_declared_symbol(lib):
    for name in declared_symbols():
        assert hasattr(lib, name), name


def test_header_compiles_as_c():
    import subprocess
    import tempfile
    with tempfile.TemporaryDirectory() as d:
        src = os.path.join(d, "t.c")
        open(src, "w").write('#include "libmxqdq.h"\nint main(void){return MX_OK;}\n')
        subprocess.check_call(["gcc", "-std=c99", "-Wall", "-Werror", "-I", os.path.dirname(HEADER),
                               "-c", src, "-o", os.path.join(d, "t.o")])


A = 1 << 20  # a 16-byte aligned fake address; never dereferenced (validation fails first)


def test_qdq_argument_errors(lib):
    q = lib.mx_qdq
    assert q(2, A, 0, 4, 64, None, 0, A) == MX_EFMT
    assert q(-1, A, 0, 4, 64, None, 0, A) == MX_EFMT
    assert q(0, A, 2, 4, 64, None, 0, A) == MX_EDTYPE
    assert q(0, A, 0, 4, 48, None, 0, A) == MX_ESHAPE
    assert q(0, A, 0, -1, 64, None, 0, A) == MX_ESHAPE
    assert q(0, A, 0, 4, -32, None, 0, A) == MX_ESHAPE
    assert q(0, A, 0, 1 << 40, 1 << 20, None, 0, A) == MX_ESHAPE
    assert q(0, A, 0, 4, 64, A, 8, A) == MX_EROT
    assert q(0, A, 0, 4, 64, A, 256, A) == MX_EROT
    assert q(0, A, 0, 4, 96, A, 64, A) == MX_EROT      # K % r != 0
    assert q(0, A, 0, 4, 64, None, 16, A) == MX_EROT   # NULL matrix
    assert q(0, None, 0, 4, 64, None, 0, A) == MX_ENULL
    assert q(0, A, 0, 4, 64, None, 0, None) == MX_ENULL
    assert q(0, A + 8, 0, 4, 64, None, 0, A) == MX_EALIGN
    assert q(0, A, 0, 4, 64, None, 0, A + 2) == MX_EALIGN
    assert q(0, A, 0, 4, 64, A + 4, 16, A) == MX_EALIGN


def test_quantize_argument_errors(lib):
    q = lib.mx_quantize
    assert q(5, A, 4, 64, None, 0, A, A) == MX_EFMT
    assert q(0, A, 4, 33, None, 0, A, A) == MX_ESHAPE
    assert q(0, A, 4, 64, A, 12, A, A) == MX_EROT
    assert q(0, A, 4, 64, None, 0, None, A) == MX_ENULL
    assert q(0, A, 4, 64, None, 0, A, None) == MX_ENULL
    assert q(0, A, 4, 64, None, 0, A + 4, A) == MX_EALIGN
    assert q(1, A, 4, 64, None, 0, A, A + 2) == MX_EALIGN


def test_dequantize_and_rotate_argument_errors(lib):
    assert lib.mx_dequantize(3, A, A, 4, 64, 0, A) == MX_EFMT
    assert lib.mx_dequantize(0, A, A, 4, 64, 7, A) == MX_EDTYPE
    assert lib.mx_dequantize(0, A, A, 4, 40, 0, A) == MX_ESHAPE
    assert lib.mx_dequantize(0, None, A, 4, 64, 0, A) == MX_ENULL
    assert lib.mx_dequantize(0, A, A, 4, 64, 0, A + 8) == MX_EALIGN
    assert lib.mx_rotate(A, 0, 4, 64, A, 0, A) == MX_EROT  # rotation is required
    assert lib.mx_rotate(A, 3, 4, 64, A, 16, A) == MX_EDTYPE
    assert lib.mx_rotate(A, 0, 4, 64, A, 16, None) == MX_ENULL


def test_matmul_argument_errors(lib):
    F = 1.0
    assert lib.mx_matmul(2, A, A, A, A, 0, 4, 4, 64, F, 0, A) == MX_EFMT
    assert lib.mx_matmul(0, A, A, A, A, 0, 4, 4, 64, F, 5, A) == MX_EDTYPE
    assert lib.mx_matmul(0, A, A, A, A, 0, 4, 4, 48, F, 0, A) == MX_ESHAPE
    assert lib.mx_matmul(0, A, A, A, A, 0, -1, 4, 64, F, 0, A) == MX_ESHAPE
    assert lib.mx_matmul(0, A, A, A, A, 0, 4, -4, 64, F, 0, A) == MX_ESHAPE
    assert lib.mx_matmul(1, A, A, A, A, 0, 65535 * 128 + 1, 4, 64, F, 1, A) == MX_ESHAPE
    assert lib.mx_matmul(1, A, A, A, A, 0, 4, 4, (1 << 23) + 32, F, 0, A) == MX_ESHAPE  # 32-bit offsets
    assert lib.mx_matmul(0, A, A, A, A, 0, 4, 4, (1 << 24) + 32, F, 0, A) == MX_ESHAPE
    assert lib.mx_matmul(0, A, A, A, A, 2, 4, 4, 64, F, 0, A) == MX_ELAYOUT
    assert lib.mx_matmul(0, A, A, A, A, 0, 4, 4, 64, F, 0, None) == MX_ENULL
    assert lib.mx_matmul(0, A, None, A, A, 0, 4, 4, 64, F, 0, A) == MX_ENULL
    assert lib.mx_matmul(0, A, A, None, A, 1, 4, 4, 64, F, 0, A) == MX_ENULL
    assert lib.mx_matmul(0, A + 4, A, A, A, 0, 4, 4, 64, F, 0, A) == MX_EALIGN
    assert lib.mx_matmul(0, A, A, A + 8, A, 0, 4, 4, 64, F, 0, A) == MX_EALIGN
    assert lib.mx_matmul(0, A, A, A, A, 0, 4, 4, 64, F, 1, A + 4) == MX_EALIGN
    assert lib.mx_matmul(0, A, A + 2, A, A, 1, 4, 4, 64, F, 1, A) == MX_EALIGN  # blocked scales: 4 bytes


def test_blocked_scales_size_and_errors(lib):
    assert lib.mx_blocked_scales_bytes(2, 64) == 256
    assert lib.mx_blocked_scales_bytes(33, 288) == 1024
    assert lib.mx_blocked_scales_bytes(8192, 28672) == 256 * 112 * 256
    assert lib.mx_blocked_scales_bytes(0, 64) == 0
    assert lib.mx_blocked_scales_bytes(4, 48) == MX_ESHAPE
    assert lib.mx_scales_to_blocked(A, 4, 48, A) == MX_ESHAPE
    assert lib.mx_scales_to_blocked(None, 4, 64, A) == MX_ENULL
    assert lib.mx_scales_to_blocked(A, 4, 64, A + 2) == MX_EALIGN
    assert lib.mx_quantize_blocked(2, A, 4, 64, None, 0, A, A) == MX_EFMT
    assert lib.mx_quantize_blocked(0, A, 4, 64, A, 48, A, A) == MX_EROT
    assert lib.mx_quantize_blocked(0, A, 4, 64, None, 0, A, None) == MX_ENULL
    assert lib.mx_quantize_blocked(0, A, 4, 64, None, 0, A, A + 1) == MX_EALIGN
    assert lib.mx_quantize_blocked(1, A + 8, 4, 64, None, 0, A, A) == MX_EALIGN


def test_nvfp4_argument_errors(lib):
    assert lib.mx_nvfp4_quantize(A, 4, 40, None, 0, A, A, A) == MX_ESHAPE
    assert lib.mx_nvfp4_quantize(A, -1, 32, None, 0, A, A, A) == MX_ESHAPE
    assert lib.mx_nvfp4_quantize(A, 4, 48, A, 16, A, A, A) == MX_EROT  # a rotation needs K % 32 == 0
    assert lib.mx_nvfp4_quantize(A, 4, 64, A, 48, A, A, A) == MX_EROT
    assert lib.mx_nvfp4_quantize(A, 4, 64, None, 16, A, A, A) == MX_EROT
    assert lib.mx_nvfp4_quantize(A, 4, 48, None, 0, None, A, A) == MX_ENULL
    assert lib.mx_nvfp4_quantize(A, 4, 48, None, 0, A, A, None) == MX_ENULL
    assert lib.mx_nvfp4_quantize(A + 8, 4, 48, None, 0, A, A, A) == MX_EALIGN
    assert lib.mx_nvfp4_quantize(A, 4, 48, None, 0, A + 2, A, A) == MX_EALIGN
    assert lib.mx_nvfp4_quantize(A, 4, 48, None, 0, A, A, A + 2) == MX_EALIGN
    assert lib.mx_nvfp4_qdq(A, 4, 24, None, 0, A, A) == MX_ESHAPE
    assert lib.mx_nvfp4_qdq(A, 4, 48, None, 0, A, A + 4) == MX_EALIGN
    assert lib.mx_nvfp4_dequantize(A, A, 4, 48, A, 3, A) == MX_EDTYPE
    assert lib.mx_nvfp4_dequantize(A, A, 4, 40, A, 0, A) == MX_ESHAPE
    assert lib.mx_nvfp4_dequantize(A, None, 4, 48, A, 0, A) == MX_ENULL


def test_empty_is_a_noop(lib):
    # no pointer is touched and no kernel is launched for M == 0 or K == 0
    assert lib.mx_qdq(0, None, 0, 0, 64, None, 0, None) == MX_OK
    assert lib.mx_qdq(1, None, 1, 5, 0, None, 0, None) == MX_OK
    assert lib.mx_quantize(0, None, 0, 128, None, 0, None, None) == MX_OK
    assert lib.mx_dequantize(1, None, None, 0, 32, 0, None) == MX_OK
    assert lib.mx_rotate(None, 0, 0, 128, A, 128, None) == MX_OK
    assert lib.mx_matmul(0, None, None, None, None, 0, 0, 8, 64, 1.0, 0, None) == MX_OK
    assert lib.mx_matmul(1, None, None, None, None, 1, 8, 0, 64, 1.0, 1, None) == MX_OK
    assert lib.mx_scales_to_blocked(None, 0, 64, None) == MX_OK
    assert lib.mx_quantize_blocked(0, None, 5, 0, None, 0, None, None) == MX_OK
    assert lib.mx_nvfp4_quantize(None, 0, 48, None, 0, None, None, None) == MX_OK
    assert lib.mx_nvfp4_qdq(None, 7, 0, None, 0, None, None) == MX_OK
    assert lib.mx_nvfp4_dequantize(None, None, 0, 16, None, 1, None) == MX_OK


def test_status_strings_and_stream(lib):
    for code in (MX_OK, MX_EFMT, MX_EDTYPE, MX_ESHAPE, MX_EROT, MX_ENULL, MX_EALIGN, MX_ELAUNCH, MX_ELAYOUT):
        s = lib.mx_status_string(code).decode()
        assert s and s != "unknown status"
    assert lib.mx_status_string(-99).decode() == "unknown status"
    lib.mx_set_stream(ctypes.c_void_p(0x1234))
    assert lib.mx_get_stream() == 0x1234
    lib.mx_set_stream(None)
    assert not lib.mx_get_stream()


def test_stream_is_thread_local(lib):
    """A stream set in one thread is not the stream of another."""
    import threading
    seen = {}

    def worker(name, value):
        lib.mx_set_stream(ctypes.c_void_p(value))
        barrier.wait()
        seen[name] = lib.mx_get_stream()
        lib.mx_set_stream(None)

    barrier = threading.Barrier(2)
    ts = [threading.Thread(target=worker, args=("a", 0x1000)), threading.Thread(target=worker, args=("b", 0x2000))]
    for t in ts:
        t.start()
    for t in ts:
        t.join()
    assert seen == {"a": 0x1000, "b": 0x2000}
    assert not lib.mx_get_stream()


def test_library_does_not_reference_the_oracle():
    """The product library links nothing from oracle/ (no orc_ symbols)."""
    import subprocess
    out = subprocess.run(["nm", "-D", LIB], capture_output=True, text=True).stdout
    assert "orc_" not in out
