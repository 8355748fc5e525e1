"""GPU parity of NVFP4 (the reading of the pages' fusedQuantizeNv: 16-groups,
E4M3 block scales, E2M1 codes and a per-tensor fp32 multiplier g, with the
steps fixed as fp32 operations) against the CPU oracle, through the C ABI.

Bars: unrotated codes, scale bytes, QDQ output and dequantized values are
bit-exact; rotated results satisfy the NVFP4 band (tests/_parity.py), as the
MX rotated path does.
"""
import numpy as np
import pytest

import oracle
from _bandcheck import check_nv
from _parity import THREADS, assert_bits_equal, bits_of, nv_band_check, to_gpu_bf16, unpack_codes
from microscaling_quantize_dequantize_amd import workloads as W

pytestmark = pytest.mark.gpu

E2M1 = 0


@pytest.fixture(scope="module")
def mx():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from microscaling_quantize_dequantize_amd import binding
    return binding


def gscale(g):
    import torch
    return torch.tensor([g], dtype=torch.float32, device="cuda")


def tensor_g(bits):
    """448 * 6 / amax of the tensor (the usual per-tensor choice), in fp32."""
    amax = float(np.abs(W.bf16_bits_to_f32(bits)).max())
    return float(np.float32(448.0 * 6.0 / amax)) if amax > 0 else 1.0


def check_unrotated(mx, x, g, what):
    import torch
    xs = to_gpu_bf16(x)
    codes, scales = mx.mx_nvfp4_quantize(xs, gscale(g))
    qdq = mx.mx_nvfp4_qdq(xs, gscale(g))
    torch.cuda.synchronize()
    c_ref, s_ref = oracle.nv_quantize(x, g, threads=THREADS)
    assert_bits_equal(bits_of(scales), s_ref, f"{what} scales")
    assert_bits_equal(bits_of(codes), c_ref, f"{what} codes")
    assert_bits_equal(bits_of(qdq), oracle.nv_qdq(x, g, threads=THREADS), f"{what} qdq")
    # dequantize of the oracle's codes, bf16 and fp32
    K = x.shape[1]
    for dt, odt in ((torch.bfloat16, 0), (torch.float32, 1)):
        d = mx.mx_nvfp4_dequantize(torch.from_numpy(c_ref).cuda(), torch.from_numpy(s_ref).cuda(), K, gscale(g),
                                   dtype=dt)
        torch.cuda.synchronize()
        assert_bits_equal(bits_of(d), oracle.nv_dequantize(c_ref, s_ref, K, g, dst_dtype=odt, threads=THREADS),
                          f"{what} dequantize {dt}")


@pytest.mark.parametrize("shape", [(1, 16), (3, 48), (64, 80), (130, 1024), (257, 4112)],
                         ids=lambda s: f"{s[0]}x{s[1]}")
def test_unrotated_matches_oracle(mx, shape):
    M, K = shape
    x = W.random_bf16(shape, seed=M * 7 + K)
    for g in (1.0, tensor_g(x), 0.37, 3.0e4):
        check_unrotated(mx, x, g, f"{shape} g={g}")


def test_unrotated_special_groups(mx):
    rng = np.random.default_rng(5)
    M, K = 64, 256
    x = rng.standard_t(3, (M, K)).astype(np.float32)
    x = x.reshape(M, K // 16, 16)
    x[0, 0] = 0.0                               # zero group
    x[1, 1] = -0.0                              # negative zero group
    x[2, 2] *= 2.0 ** -20                       # scale rounds to 0 under g = 1 (q <= 2^-10)
    x[3, 3] *= 2.0 ** -9                        # E4M3-subnormal scales
    x[4, 4] *= 2.0 ** 14                        # saturating scale (q > 448) under g = 1
    x[5, 5, :] = np.float32(0.75)               # ties in the element grid
    x[6, 6, 0] = 6.0                            # scale exactly 1
    x[7, 7] = rng.standard_normal(16) * 2.0 ** -130  # bf16 subnormals
    bits = W.f32_to_bf16_bits(x.reshape(M, K))
    for g in (1.0, 2688.0, 6.0 * 2.0 ** -5):
        check_unrotated(mx, bits, g, f"special g={g}")


@pytest.mark.parametrize("e", [60, -60, 61, -61, 100, -100])
def test_unrotated_multiplier_range(mx, e):
    """g = 2^e on both sides of the range in which the kernels form g / v
    and v / g without a division, the input scaled by 2^-e so that the group
    scales stay in range: bit-exact either way."""
    M, K = 33, 160
    x = W.random_bf16((M, K), seed=200 + e)
    xs = W.f32_to_bf16_bits(W.bf16_bits_to_f32(x) * np.float32(2.0 ** -e))
    check_unrotated(mx, xs, float(2.0 ** e), f"g=2^{e}")


@pytest.mark.parametrize("g", [1.0, 2688.0, 2.0 ** 70])
def test_dequantize_every_scale_byte(mx, g):
    """Dequantize of every scale byte 0..255 (negative scales and the NaN
    bytes 0x7F/0xFF included) with every E2M1 code: bit-exact against the
    oracle's E4M3 decode where it gives a number, NaN where it gives NaN."""
    import torch
    K = 16 * 16
    sb = np.arange(256, dtype=np.uint8).reshape(16, 16)   # 16 rows x 16 groups
    nib = np.tile(np.arange(16, dtype=np.uint8), K // 16)
    codes = np.tile((nib[0::2] | (nib[1::2] << 4))[None, :], (16, 1))
    for dt, odt in ((torch.bfloat16, 0), (torch.float32, 1)):
        d = mx.mx_nvfp4_dequantize(torch.from_numpy(codes).cuda(), torch.from_numpy(sb).cuda(), K, gscale(g),
                                   dtype=dt)
        torch.cuda.synchronize()
        got = d.float().cpu().numpy()
        want = oracle.nv_dequantize(codes, sb, K, g, dst_dtype=odt, threads=THREADS)
        want_f = W.bf16_bits_to_f32(want) if odt == 0 else want.view(np.float32)
        nan = np.isnan(want_f)
        assert nan.sum() == 2 * 16, "the 0x7F and 0xFF groups"
        assert np.array_equal(np.isnan(got), nan), f"NaN positions {dt}"
        assert_bits_equal(bits_of(d)[~nan], want[~nan], f"every scale byte {dt} g={g}")


def test_unrotated_full_size(mx):
    """The 8192 x 28672 down-projection input (Student-t, nu = 3), the
    configuration the bench times: every code, scale byte and QDQ output
    bit-exact against the oracle."""
    import torch
    x = W.generate("c4")
    g = tensor_g(x)
    xs = to_gpu_bf16(x)
    codes, scales = mx.mx_nvfp4_quantize(xs, gscale(g))
    qdq = mx.mx_nvfp4_qdq(xs, gscale(g))
    torch.cuda.synchronize()
    c_ref, s_ref = oracle.nv_quantize(x, g, threads=THREADS)
    assert_bits_equal(bits_of(scales), s_ref, "full-size scales")
    assert_bits_equal(bits_of(codes), c_ref, "full-size codes")
    del c_ref, s_ref
    assert_bits_equal(bits_of(qdq), oracle.nv_qdq(x, g, threads=THREADS), "full-size qdq")


@pytest.mark.parametrize("r,shape", [(16, (64, 256)), (16, (6, 96)), (32, (33, 288)), (32, (10, 160)), (64, (45, 384)),
                                     (128, (129, 1152))], ids=lambda v: str(v))
def test_rotated_within_band(mx, r, shape):
    import torch
    M, K = shape
    x = W.random_bf16(shape, seed=r + M)
    Rb = W.hadamard_rotation(r)
    y, beta = oracle.rotate(x, Rb, r, threads=THREADS)
    for g in (1.0, tensor_g(x) * 0.9):
        xs, R = to_gpu_bf16(x), to_gpu_bf16(Rb)
        codes, scales = mx.mx_nvfp4_quantize(xs, gscale(g), rot=R)
        qdq = mx.mx_nvfp4_qdq(xs, gscale(g), rot=R)
        torch.cuda.synchronize()
        nv_band_check(y, beta, g, codes_gpu=unpack_codes(E2M1, bits_of(codes), K), scales_gpu=bits_of(scales))
        nv_band_check(y, beta, g, deq_gpu=qdq.float().cpu().numpy().astype(np.float64))


@pytest.mark.parametrize("r", [16, 32, 64, 128])
def test_dense_nonsymmetric_rotation(mx, r):
    """A dense matrix with no symmetry (seeded normal entries times r^-0.5,
    rounded to bf16) on several tiles with a partial last one: quantize and
    QDQ within the NVFP4 band of the oracle."""
    import torch
    rng = np.random.default_rng(950 + r)
    Rb = W.f32_to_bf16_bits((rng.standard_normal((r, r)) / np.sqrt(r)).astype(np.float32))
    x = W.random_bf16((300, 1152), seed=r + 11)
    K = x.shape[1]
    y, beta = oracle.rotate(x, Rb, r, threads=THREADS)
    for g in (1.0, tensor_g(x) * 0.9):
        xs, R = to_gpu_bf16(x), to_gpu_bf16(Rb)
        codes, scales = mx.mx_nvfp4_quantize(xs, gscale(g), rot=R)
        qdq = mx.mx_nvfp4_qdq(xs, gscale(g), rot=R)
        torch.cuda.synchronize()
        nv_band_check(y, beta, g, codes_gpu=unpack_codes(E2M1, bits_of(codes), K), scales_gpu=bits_of(scales))
        nv_band_check(y, beta, g, deq_gpu=qdq.float().cpu().numpy().astype(np.float64))


@pytest.mark.parametrize("r", [0, 16, 64, 128])
def test_in_place_matches_out_of_place(mx, r):
    """dst == src gives the bits of the out-of-place QDQ, on the unrotated,
    the 32-block and the lane-owned kernels."""
    import torch
    x = W.random_bf16((2048, 4096), seed=31 + r)
    g = tensor_g(x)
    R = to_gpu_bf16(W.hadamard_rotation(r)) if r else None
    src = to_gpu_bf16(x)
    ref = mx.mx_nvfp4_qdq(src, gscale(g), rot=R)
    t = src.clone()
    mx.mx_nvfp4_qdq(t, gscale(g), rot=R, dst=t)
    torch.cuda.synchronize()
    assert np.array_equal(bits_of(t), bits_of(ref)), f"nvfp4 in place r={r}"


def test_rotated_full_size(mx):
    """Rotation 128 on the 8192 x 28672 layer: codes, scales and QDQ output
    of every row within the NVFP4 band of the oracle (tests/bandcheck.c), the
    cap of 0.01% differing elements on the whole tensor."""
    import torch
    x = W.generate("c4")
    g = tensor_g(x)
    Rb = W.hadamard_rotation(128)
    xs, R = to_gpu_bf16(x), to_gpu_bf16(Rb)
    codes, scales = mx.mx_nvfp4_quantize(xs, gscale(g), rot=R)
    qdq = mx.mx_nvfp4_qdq(xs, gscale(g), rot=R)
    torch.cuda.synchronize()
    results = [{"codes": bits_of(codes), "scales": bits_of(scales)}, {"deq": bits_of(qdq)}]
    stats = check_nv(x, Rb, 128, g, results, what="nvfp4 c4 r=128")
    print("nvfp4 c4 rotation 128 (quantize, qdq):", stats)
    assert all(st["elements"] == x.size for st in stats)


@pytest.mark.parametrize("e", [None, 70, -70])
def test_identity_rotation_equals_unrotated(mx, e):
    """Rotation by the identity changes nothing, also for g outside the range
    of the division-free quotients (g = 2^e, input scaled by 2^-e)."""
    import torch
    M, K = 64, 512
    x = W.random_bf16((M, K), seed=3)
    eye = W.f32_to_bf16_bits(np.eye(32, dtype=np.float32))
    if e is None:
        g = tensor_g(x)
    else:
        x = W.f32_to_bf16_bits(W.bf16_bits_to_f32(x) * np.float32(2.0 ** -e))
        g = float(2.0 ** e)
    xs = to_gpu_bf16(x)
    c1, s1 = mx.mx_nvfp4_quantize(xs, gscale(g), rot=to_gpu_bf16(eye))
    c0, s0 = mx.mx_nvfp4_quantize(xs, gscale(g))
    q1 = mx.mx_nvfp4_qdq(xs, gscale(g), rot=to_gpu_bf16(eye))
    q0 = mx.mx_nvfp4_qdq(xs, gscale(g))
    torch.cuda.synchronize()
    assert torch.equal(c1, c0) and torch.equal(s1, s0) and torch.equal(q1, q0)


def test_empty_and_errors(mx):
    import torch
    e = torch.empty((0, 32), dtype=torch.bfloat16, device="cuda")
    c, s = mx.mx_nvfp4_quantize(e, gscale(1.0))
    assert c.shape == (0, 16) and s.shape == (0, 2)
    with pytest.raises(mx.MXError):
        mx.mx_nvfp4_quantize(torch.zeros((4, 40), dtype=torch.bfloat16, device="cuda"), gscale(1.0))
    with pytest.raises(ValueError):
        mx.mx_nvfp4_qdq(torch.zeros((4, 32), dtype=torch.bfloat16, device="cuda"),
                        torch.ones(2, dtype=torch.float32, device="cuda"))
