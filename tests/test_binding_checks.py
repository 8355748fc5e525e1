"""The Python binding rejects wrong buffers before anything reaches the
library: a tensor of the wrong dtype or shape raises ValueError (and a
right-shaped one that is not on the GPU raises TypeError) without any
compute entry point being called (CPU only: the tensors are host tensors and
the library's compute entry points are replaced by a stub that fails)."""
import os

import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "microscaling_quantize_dequantize_amd", "libmxqdq.so")


@pytest.fixture(scope="module")
def b():
    if not os.path.exists(LIB):
        from microscaling_quantize_dequantize_amd import build
        build.build()
    from microscaling_quantize_dequantize_amd import binding
    return binding


class NoCompute:
    """Stands in for the library: only the size query may be called."""

    def __init__(self, real):
        self.real = real

    def __getattr__(self, name):
        if name in ("mx_blocked_scales_bytes", "mx_status_string"):
            return getattr(self.real, name)
        raise AssertionError(f"{name} was called")


@pytest.fixture
def mx(b, monkeypatch):
    monkeypatch.setattr(b, "_lib", NoCompute(b._lib))
    return b


def u8(*shape):
    return torch.zeros(shape, dtype=torch.uint8)


def bf(*shape):
    return torch.zeros(shape, dtype=torch.bfloat16)


M, K = 4, 64


@pytest.mark.parametrize("fmt", [0, 1])
def test_quantize_buffers(mx, fmt):
    cols = K // 2 if fmt == 0 else K
    src = bf(M, K)
    for codes, scales in ((u8(M, cols + 1), u8(M, 2)), (u8(M - 1, cols), u8(M, 2)), (u8(M, cols), u8(M, 1)),
                          (u8(M, cols), u8(M * 2)), (torch.zeros((M, cols), dtype=torch.int8), u8(M, 2))):
        with pytest.raises(ValueError):
            mx.mx_quantize(fmt, src, codes=codes, scales=scales)
    with pytest.raises(TypeError):
        mx.mx_quantize(fmt, src, codes=u8(M, cols), scales=u8(M, 2))
    with pytest.raises(ValueError):
        mx.mx_quantize_blocked(fmt, src, codes=u8(M, cols), blocked=u8(mx.mx_blocked_scales_bytes(M, K) - 1))
    with pytest.raises(ValueError):
        mx.mx_quantize_blocked(fmt, src, codes=u8(M, cols + 2), blocked=u8(mx.mx_blocked_scales_bytes(M, K)))
    with pytest.raises(TypeError):
        mx.mx_quantize_blocked(fmt, src, codes=u8(M, cols), blocked=u8(mx.mx_blocked_scales_bytes(M, K)))


def test_qdq_and_rotate_outputs(mx):
    src = bf(M, K)
    for dst in (bf(M, K + 32), bf(M + 1, K), torch.zeros((M, K), dtype=torch.float32)):
        with pytest.raises(ValueError):
            mx.mx_qdq(0, src, dst=dst)
    with pytest.raises(TypeError):
        mx.mx_qdq(0, src, dst=bf(M, K))
    with pytest.raises(ValueError):
        mx.mx_rotate(src, bf(32, 32), dst=bf(M, K))
    with pytest.raises(ValueError):
        mx.mx_rotate(src, bf(32, 32), dst=torch.zeros((M, K + 32), dtype=torch.float32))


@pytest.mark.parametrize("fmt", [0, 1])
def test_dequantize_buffers(mx, fmt):
    cols = K // 2 if fmt == 0 else K
    bad = [
        (u8(M, cols), u8(M * 2), None),                 # flat (blocked-like) scales
        (u8(M, cols), u8(M, 3), None),                  # scales of another K
        (u8(M - 1, cols), u8(M, 2), None),              # fewer code rows than scale rows
        (u8(M, cols - 1), u8(M, 2), None),              # short code rows
        (u8(M, cols), u8(M, 2), bf(M, K - 32)),         # short output
        (u8(M, cols), u8(M, 2), torch.zeros((M, K), dtype=torch.int16)),
    ]
    for codes, scales, dst in bad:
        with pytest.raises(ValueError):
            mx.mx_dequantize(fmt, codes, scales, K, dst=dst)
    with pytest.raises(TypeError):
        mx.mx_dequantize(fmt, u8(M, cols), u8(M, 2), K)


def test_scales_to_blocked_buffers(mx):
    with pytest.raises(ValueError):
        mx.mx_scales_to_blocked(u8(M, 3), K)
    with pytest.raises(ValueError):
        mx.mx_scales_to_blocked(u8(M, 2), K, blocked=u8(16))
    with pytest.raises(ValueError):
        mx.mx_scales_to_blocked(u8(M, 2), K, blocked=u8(2, 256))
    with pytest.raises(TypeError):
        mx.mx_scales_to_blocked(u8(M, 2), K, blocked=u8(mx.mx_blocked_scales_bytes(M, K)))


@pytest.mark.parametrize("fmt", [0, 1])
def test_matmul_buffers(mx, fmt):
    cols = K // 2 if fmt == 0 else K
    N = 8
    a, b_ = u8(M, cols), u8(N, cols)
    sa, sb = u8(M, 2), u8(N, 2)
    for args in ((u8(M, cols - 1), sa, b_, sb), (a, sa, u8(N, cols + 1), sb), (a, u8(M, 1), b_, sb),
                 (a, sa, b_, u8(N - 1, 2))):
        with pytest.raises(ValueError):
            mx.mx_matmul(fmt, *args, K)
    with pytest.raises(ValueError):
        mx.mx_matmul(fmt, a, u8(10), b_, u8(mx.mx_blocked_scales_bytes(N, K)), K, scale_layout=mx.BLOCKED)
    with pytest.raises(ValueError):
        mx.mx_matmul(fmt, a, sa, b_, sb, K, c=torch.zeros((M, N + 1), dtype=torch.float32))
    with pytest.raises(TypeError):
        mx.mx_matmul(fmt, a, sa, b_, sb, K)


def test_nvfp4_buffers(mx):
    src = bf(M, K)
    g = torch.ones(1, dtype=torch.float32)
    for codes, scales in ((u8(M, K // 2 + 1), u8(M, K // 16)), (u8(M, K // 2), u8(M, K // 32))):
        with pytest.raises(ValueError):
            mx.mx_nvfp4_quantize(src, g, codes=codes, scales=scales)
    with pytest.raises(ValueError):
        mx.mx_nvfp4_qdq(src, g, dst=bf(M, K // 2))
    with pytest.raises(ValueError):
        mx.mx_nvfp4_qdq(src, torch.ones(2, dtype=torch.float32))
    with pytest.raises(ValueError):
        mx.mx_nvfp4_dequantize(u8(M, K // 2), u8(M, K // 32), K, g)
    with pytest.raises(ValueError):
        mx.mx_nvfp4_dequantize(u8(M, K // 2 - 1), u8(M, K // 16), K, g)
    with pytest.raises(TypeError):
        mx.mx_nvfp4_quantize(src, g)
