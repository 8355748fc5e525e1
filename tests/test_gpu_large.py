"""Tensors of more than 2^31 elements: every step kernel indexes with 64 bits.

A 65540 x 32768 bf16 tensor (2^31 + 131072 elements, 4.3 GB) drawn on the
GPU from a seeded generator; the first and last four rows (the last ones
lie past element 2^31) are compared with the oracle, which treats rows
independently: unrotated QDQ, quantize and dequantize (bf16 and fp32 out)
bit for bit, the rotated forms (r = 16 on 64-element blocks, r = 64 on the
persistent grid, r = 128 on the 16-block and the lane-owned kernels,
blocked scales by whole units) within the band, and NVFP4 (its per-tensor
multiplier passed in, so rows stay independent) bit for bit unrotated and
within its band at r = 128.  The oracle runs on those rows only.
"""
import numpy as np
import pytest

import oracle
from _parity import (E2M1, E4M3, THREADS, assert_bits_equal, band_check, bf16_values, bits_of,
                     nv_band_check, unpack_codes)
from oracle import BF16, F32
from microscaling_quantize_dequantize_amd import workloads as W

pytestmark = pytest.mark.gpu

M, K = 65540, 32768
ROWS = list(range(4)) + list(range(M - 4, M))


@pytest.fixture(scope="module")
def big():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from microscaling_quantize_dequantize_amd import binding
    assert M * K > 2 ** 31
    g = torch.Generator(device="cuda")
    g.manual_seed(2031)
    x = (torch.randn((M, K), generator=g, device="cuda", dtype=torch.float32) * 0.02).to(torch.bfloat16)
    rows = bits_of(x[ROWS])
    return binding, x, rows


def _rot(r):
    import torch
    return torch.from_numpy(W.hadamard_rotation(r).view(np.int16)).view(torch.bfloat16).cuda()


def test_unrotated_beyond_2_31(big):
    import torch
    mx, x, rows = big
    for fmt in (E2M1, E4M3):
        out = mx.mx_qdq(fmt, x)
        codes, scales = mx.mx_quantize(fmt, x)
        torch.cuda.synchronize()
        assert_bits_equal(bits_of(out[ROWS]), oracle.qdq(fmt, rows, threads=THREADS), f"qdq fmt{fmt}")
        c_ref, s_ref = oracle.quantize(fmt, rows, threads=THREADS)
        assert_bits_equal(bits_of(codes[ROWS]), c_ref, f"codes fmt{fmt}")
        assert_bits_equal(bits_of(scales[ROWS]), s_ref, f"scales fmt{fmt}")
        del out, codes, scales


@pytest.mark.parametrize("r", [16, 64, 128])
def test_rotated_beyond_2_31(big, r):
    import torch
    mx, x, rows = big
    Rb = W.hadamard_rotation(r)
    R = _rot(r)
    y, beta = oracle.rotate(rows, Rb, r, threads=THREADS)
    for fmt in (E2M1, E4M3):
        out = mx.mx_qdq(fmt, x, rot=R)
        torch.cuda.synchronize()
        band_check(fmt, y, beta, deq_gpu=bf16_values(bits_of(out[ROWS])))
        del out
        codes, scales = mx.mx_quantize(fmt, x, rot=R)
        torch.cuda.synchronize()
        band_check(fmt, y, beta, codes_gpu=unpack_codes(fmt, bits_of(codes[ROWS]), K), scales_gpu=bits_of(scales[ROWS]))
        if r == 128:
            bcodes, blocked = mx.mx_quantize_blocked(fmt, x, rot=R)
            torch.cuda.synchronize()
            assert torch.equal(bcodes[ROWS], codes[ROWS]), f"blocked codes fmt{fmt}"
            s_blk = mx.mx_scales_to_blocked(scales, K)
            torch.cuda.synchronize()
            assert torch.equal(blocked, s_blk), f"blocked scales fmt{fmt}"
            del bcodes, blocked, s_blk
        del codes, scales


def test_dequantize_beyond_2_31(big):
    import torch
    mx, x, rows = big
    for fmt in (E2M1, E4M3):
        codes, scales = mx.mx_quantize(fmt, x)
        torch.cuda.synchronize()
        c_rows, s_rows = bits_of(codes[ROWS]), bits_of(scales[ROWS])
        for dt, odt in ((torch.bfloat16, BF16), (torch.float32, F32)):
            d = mx.mx_dequantize(fmt, codes, scales, K, dtype=dt)
            torch.cuda.synchronize()
            assert_bits_equal(bits_of(d[ROWS]), oracle.dequantize(fmt, c_rows, s_rows, K, dst_dtype=odt, threads=THREADS),
                              f"dequantize fmt{fmt} {dt}")
            del d
        del codes, scales


def test_nvfp4_beyond_2_31(big):
    import torch
    mx, x, rows = big
    g = float(np.float32(448.0 * 6.0 / float(x.abs().max().float())))
    gs = torch.tensor([g], dtype=torch.float32, device="cuda")
    codes, scales = mx.mx_nvfp4_quantize(x, gs)
    qdq = mx.mx_nvfp4_qdq(x, gs)
    torch.cuda.synchronize()
    c_ref, s_ref = oracle.nv_quantize(rows, g, threads=THREADS)
    assert_bits_equal(bits_of(scales[ROWS]), s_ref, "nvfp4 scales")
    assert_bits_equal(bits_of(codes[ROWS]), c_ref, "nvfp4 codes")
    assert_bits_equal(bits_of(qdq[ROWS]), oracle.nv_qdq(rows, g, threads=THREADS), "nvfp4 qdq")
    del qdq
    d = mx.mx_nvfp4_dequantize(codes, scales, K, gs)
    torch.cuda.synchronize()
    assert_bits_equal(bits_of(d[ROWS]), oracle.nv_dequantize(c_ref, s_ref, K, g, threads=THREADS), "nvfp4 dequantize")
    del d, codes, scales
    Rb = W.hadamard_rotation(128)
    y, beta = oracle.rotate(rows, Rb, 128, threads=THREADS)
    codes, scales = mx.mx_nvfp4_quantize(x, gs, rot=_rot(128))
    qdq = mx.mx_nvfp4_qdq(x, gs, rot=_rot(128))
    torch.cuda.synchronize()
    nv_band_check(y, beta, g, codes_gpu=unpack_codes(E2M1, bits_of(codes[ROWS]), K), scales_gpu=bits_of(scales[ROWS]))
    nv_band_check(y, beta, g, deq_gpu=qdq[ROWS].float().cpu().numpy().astype(np.float64))
