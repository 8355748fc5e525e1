"""The whole-tensor C comparator (tests/bandcheck.c) decides exactly as the
numpy comparator of tests/_parity.py: the same differing-element counts and
the same rejections, on the oracle's own results and on planted in-band and
out-of-band changes (CPU only; every change is planted in oracle outputs)."""
import numpy as np
import pytest

import oracle
from _bandcheck import check_mx, check_nv
from _parity import E2M1, E4M3, band_check, bf16_values, nv_band_check, unpack_codes
from microscaling_quantize_dequantize_amd import workloads as W


def identity_bits(r):
    return W.f32_to_bf16_bits(np.eye(r, dtype=np.float32))


def tie_case(fmt):
    """Identity rotation (y = x exactly, beta = 1e-5 |x|) on groups whose
    abs-max fixes s = 0 and whose other elements sit on rounding ties."""
    M, K = 160, 256
    top, ties = (6.0, [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]) if fmt == E2M1 else \
        (448.0, [1.0625, 1.1875, 2.125, 3.125, 5.75, 13.5, 200.0])
    rng = np.random.default_rng(5 + fmt)
    v = rng.choice(ties, size=(M, K)) * rng.choice([-1.0, 1.0], size=(M, K))
    v[:, ::32] = top
    return W.f32_to_bf16_bits(v.astype(np.float32)), identity_bits(32)


def numpy_stats(fmt, x, R, r, deq=None, codes=None, scales=None):
    y, beta = oracle.rotate(x, R, r)
    if deq is not None:
        return band_check(fmt, y, beta, deq_gpu=bf16_values(deq))
    return band_check(fmt, y, beta, codes_gpu=unpack_codes(fmt, codes, x.shape[1]), scales_gpu=scales)


def c_stats(fmt, x, R, r, deq=None, codes=None, scales=None):
    res = {"fmt": fmt, "deq": deq} if deq is not None else {"fmt": fmt, "codes": codes, "scales": scales}
    return check_mx(x, R, r, [res], threads=3)[0]


def both(fmt, x, R, r, **kw):
    """(numpy stats or None if it rejected, C stats or None if it rejected)."""
    out = []
    for f in (numpy_stats, c_stats):
        try:
            out.append(f(fmt, x, R, r, **kw))
        except AssertionError:
            out.append(None)
    return out


@pytest.mark.parametrize("fmt", [E2M1, E4M3])
@pytest.mark.parametrize("r", [16, 32, 64, 128])
def test_accepts_oracle_results(fmt, r):
    x = W.random_bf16((9, 1024), seed=r + fmt)
    R = W.hadamard_rotation(r)
    deq = oracle.qdq(fmt, x, R, r)
    codes, scales = oracle.quantize(fmt, x, R, r)
    for kw in ({"deq": deq}, {"codes": codes, "scales": scales}):
        a, b = both(fmt, x, R, r, **kw)
        assert a is not None and b is not None
        assert a["differ"] == b["differ"] == 0
        assert a["ambiguous_scale_groups"] == b["ambiguous_scale_groups"]
        assert b["elements"] == x.size


@pytest.mark.parametrize("fmt", [E2M1, E4M3])
def test_in_band_tie_flips_counted_alike(fmt):
    x, R = tie_case(fmt)
    deq = oracle.qdq(fmt, x, R, 32)
    vals = bf16_values(deq)
    top = 6.0 if fmt == E2M1 else 448.0
    # the next grid value up from each tie's rounded value, for a few elements
    flips = [(1, 3), (2, 40), (5, 77), (7, 250)]
    d2 = deq.copy()
    for i, k in flips:
        t = abs(float(bf16_values(x[i:i + 1, k:k + 1])[0, 0]))
        down = abs(vals[i, k])
        up = 2 * t - down          # a tie is the midpoint of its two neighbours
        assert up != down and up <= top
        d2[i, k] = W.f32_to_bf16_bits(np.array([np.copysign(up, vals[i, k])], dtype=np.float32))[0]
    a, b = both(fmt, x, R, 32, deq=d2)
    assert a is not None and b is not None
    assert a["differ"] == b["differ"] == len(flips)
    codes, scales = oracle.quantize(fmt, x, R, 32)
    u = unpack_codes(fmt, codes, x.shape[1]).copy()
    for i, k in flips:
        u[i, k] = oracle.encode(fmt, float(np.copysign(2 * abs(float(bf16_values(x[i:i + 1, k:k + 1])[0, 0]))
                                                       - abs(vals[i, k]), vals[i, k])), 0)
    if fmt == E2M1:
        packed = (u[:, 0::2] | (u[:, 1::2] << 4)).astype(np.uint8)
    else:
        packed = u.astype(np.uint8)
    a, b = both(fmt, x, R, 32, codes=packed, scales=scales)
    assert a is not None and b is not None
    assert a["differ"] == b["differ"] == len(flips)


@pytest.mark.parametrize("fmt", [E2M1, E4M3])
def test_out_of_band_changes_rejected_alike(fmt):
    x = W.random_bf16((12, 512), seed=40 + fmt)
    R = W.hadamard_rotation(64)
    deq = oracle.qdq(fmt, x, R, 64)
    vals = bf16_values(deq)
    big = np.unravel_index(np.argmax(np.abs(vals)), vals.shape)
    d2 = deq.copy()
    d2[big] = W.f32_to_bf16_bits(np.float32(vals[big] * 0.5))[0]
    assert both(fmt, x, R, 64, deq=d2) == [None, None]
    codes, scales = oracle.quantize(fmt, x, R, 64)
    s2 = scales.copy()
    s2[3, 5] += 1
    assert both(fmt, x, R, 64, codes=codes, scales=s2) == [None, None]
    c2 = codes.copy()
    c2[big[0], big[1] // (2 if fmt == E2M1 else 1)] ^= 0x02
    assert both(fmt, x, R, 64, codes=c2, scales=scales) == [None, None]


def test_ambiguous_scale_accepted_alike():
    """A group whose abs-max is exactly 8 (E2M1: s = 1) may take s = 0 within
    beta; under s = 0 every element saturates or rounds as the band allows."""
    x = np.zeros((80, 4096), dtype=np.uint16)  # 32 differing elements stay under 0.01%
    x[0, :32] = W.f32_to_bf16_bits(np.float32(0.5))
    x[0, 7] = W.f32_to_bf16_bits(np.float32(8.0))[0]
    R = identity_bits(32)
    codes, scales = oracle.quantize(E2M1, x, R, 32)
    assert scales[0, 0] == 128
    s2 = scales.copy()
    s2[0, 0] = 127
    u = unpack_codes(E2M1, codes, x.shape[1]).copy()
    u[0, :32] = [oracle.encode(E2M1, float(v), 0) for v in bf16_values(x[0, :32])]
    packed = (u[:, 0::2] | (u[:, 1::2] << 4)).astype(np.uint8)
    a, b = both(E2M1, x, R, 32, codes=packed, scales=s2)
    assert a is not None and b is not None and a["differ"] == b["differ"] == 32
    assert a["ambiguous_scale_groups"] == b["ambiguous_scale_groups"] == 1


def test_too_many_differences_rejected():
    x, R = tie_case(E4M3)
    deq = oracle.qdq(E4M3, x, R, 32)
    vals = bf16_values(deq)
    xs = np.abs(bf16_values(x))
    d2 = deq.copy()
    flip = (xs != 448.0) & (np.arange(x.shape[1])[None, :] % 7 == 0)
    up = 2 * xs - np.abs(vals)
    d2[flip] = W.f32_to_bf16_bits(np.copysign(up, vals)[flip].astype(np.float32))
    assert flip.sum() > 1e-4 * x.size
    st = check_mx(x, R, 32, [{"fmt": E4M3, "deq": d2}], check=False)[0]
    assert st["violations"] == 0 and st["differ"] == flip.sum()
    with pytest.raises(AssertionError):
        check_mx(x, R, 32, [{"fmt": E4M3, "deq": d2}])


# ---- NVFP4 ---------------------------------------------------------------------

G_NV = 37.5


def nv_both(x, R, r, **kw):
    y, beta = oracle.rotate(x, R, r)
    out = []
    try:
        if "deq" in kw:
            out.append(nv_band_check(y, beta, G_NV, deq_gpu=bf16_values(kw["deq"])))
        else:
            out.append(nv_band_check(y, beta, G_NV, codes_gpu=unpack_codes(E2M1, kw["codes"], x.shape[1]),
                                     scales_gpu=kw["scales"]))
    except AssertionError:
        out.append(None)
    try:
        out.append(check_nv(x, R, r, G_NV, [kw], threads=3)[0])
    except AssertionError:
        out.append(None)
    return out


@pytest.mark.parametrize("r", [16, 64, 128])
def test_nvfp4_alike(r):
    x = W.random_bf16((10, 1024), seed=90 + r)
    R = W.hadamard_rotation(r)
    deq = oracle.nv_qdq(x, G_NV, R, r)
    codes, scales = oracle.nv_quantize(x, G_NV, R, r)
    for kw in ({"deq": deq}, {"codes": codes, "scales": scales}):
        a, b = nv_both(x, R, r, **kw)
        assert a is not None and b is not None and a["differ"] == b["differ"] == 0
        assert a["ambiguous_scale_groups"] == b["ambiguous_scale_groups"]
    vals = bf16_values(deq)
    big = np.unravel_index(np.argmax(np.abs(vals)), vals.shape)
    d2 = deq.copy()
    d2[big] = W.f32_to_bf16_bits(np.float32(vals[big] * 0.5))[0]
    assert nv_both(x, R, r, deq=d2) == [None, None]
    s2 = scales.copy()
    s2[2, 7] += 1
    assert nv_both(x, R, r, codes=codes, scales=s2) == [None, None]
