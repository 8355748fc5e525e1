"""The rotated-path comparator accepts the oracle's own results and rejects
planted mistakes (CPU only; the mistakes are planted in oracle outputs)."""
import numpy as np
import pytest

import oracle
from _parity import E2M1, E4M3, band_check, bf16_values, rotate_within_beta, unpack_codes
from microscaling_quantize_dequantize_amd import workloads as W


@pytest.fixture(scope="module")
def case():
    x = W.random_bf16((16, 512), seed=77)
    R = W.hadamard_rotation(64)
    y, beta = oracle.rotate(x, R, 64)
    return x, R, y, beta


@pytest.mark.parametrize("fmt", [E2M1, E4M3])
def test_accepts_oracle_output(case, fmt):
    x, R, y, beta = case
    d = bf16_values(oracle.qdq(fmt, x, R, 64))
    assert band_check(fmt, y, beta, deq_gpu=d)["differ"] == 0
    codes, scales = oracle.quantize(fmt, x, R, 64)
    st = band_check(fmt, y, beta, codes_gpu=unpack_codes(fmt, codes, x.shape[1]), scales_gpu=scales)
    assert st["differ"] == 0


@pytest.mark.parametrize("fmt", [E2M1, E4M3])
def test_rejects_planted_value(case, fmt):
    x, R, y, beta = case
    d = bf16_values(oracle.qdq(fmt, x, R, 64))
    big = np.argmax(np.abs(d))
    d.ravel()[big] *= 0.5          # a whole code step or more, far from any tie
    with pytest.raises(AssertionError):
        band_check(fmt, y, beta, deq_gpu=d)


@pytest.mark.parametrize("fmt", [E2M1, E4M3])
def test_rejects_planted_scale(case, fmt):
    x, R, y, beta = case
    codes, scales = oracle.quantize(fmt, x, R, 64)
    scales = scales.copy()
    scales[3, 5] += 1
    with pytest.raises(AssertionError):
        band_check(fmt, y, beta, codes_gpu=unpack_codes(fmt, codes, x.shape[1]), scales_gpu=scales)


def test_rejects_too_many_tie_flips(case):
    """Even in-band differences are capped at 0.01% of the elements."""
    x, R, y, beta = case
    wide = beta * 1e4                                    # makes many elements ambiguous
    d = bf16_values(oracle.qdq(E2M1, x, R, 64))
    lo = oracle.qdq_value_n(E2M1, (y - wide).ravel(), np.repeat(
        oracle.scale_exponent_n(E2M1, np.abs(y).reshape(-1, 32).max(1)), 32))
    d2 = np.where(lo.reshape(d.shape) != d, lo.reshape(d.shape), d)
    d2 = bf16_values(W.f32_to_bf16_bits(d2.astype(np.float32)))
    with pytest.raises(AssertionError):
        band_check(E2M1, y, wide, deq_gpu=d2)


def test_rotate_tolerance_check(case):
    x, R, y, beta = case
    rotate_within_beta(y.astype(np.float32), y, beta)     # fp32 rounding of y is inside
    bad = y.astype(np.float32).copy()
    i = np.argmax(beta)
    bad.ravel()[i] += np.float32(3 * beta.ravel()[i])
    with pytest.raises(AssertionError):
        rotate_within_beta(bad, y, beta)


# ---- the NVFP4 band ------------------------------------------------------------

from _parity import nv_band_check  # noqa: E402

G_NV = 37.5


def test_nvfp4_accepts_oracle_output(case):
    x, R, y, beta = case
    d = bf16_values(oracle.nv_qdq(x, G_NV, R, 64))
    assert nv_band_check(y, beta, G_NV, deq_gpu=d)["differ"] == 0
    codes, scales = oracle.nv_quantize(x, G_NV, R, 64)
    st = nv_band_check(y, beta, G_NV, codes_gpu=unpack_codes(E2M1, codes, x.shape[1]), scales_gpu=scales)
    assert st["differ"] == 0


def test_nvfp4_rejects_planted_value(case):
    x, R, y, beta = case
    d = bf16_values(oracle.nv_qdq(x, G_NV, R, 64))
    big = np.argmax(np.abs(d))
    d.ravel()[big] *= 0.5
    with pytest.raises(AssertionError):
        nv_band_check(y, beta, G_NV, deq_gpu=d)


def test_nvfp4_rejects_planted_scale_and_code(case):
    x, R, y, beta = case
    codes, scales = oracle.nv_quantize(x, G_NV, R, 64)
    bad = scales.copy()
    bad[2, 7] += 1
    with pytest.raises(AssertionError):
        nv_band_check(y, beta, G_NV, codes_gpu=unpack_codes(E2M1, codes, x.shape[1]), scales_gpu=bad)
    u = unpack_codes(E2M1, codes, x.shape[1]).copy()
    k = int(np.argmax(np.abs(y)))
    u.ravel()[k] = (u.ravel()[k] & 8) | max(0, (u.ravel()[k] & 7) - 2)  # two grid steps smaller
    with pytest.raises(AssertionError):
        nv_band_check(y, beta, G_NV, codes_gpu=u, scales_gpu=scales)
