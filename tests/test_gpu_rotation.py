"""GPU parity of the rotated path (runtime rotation on MFMA, then MX).

Exact where the rotation itself is exact (identity, signed permutations,
diagonal matrices); otherwise within the stated band: rotated values within
beta = 1e-5 * sum|x R|, and at most 0.01% of elements differing from the
oracle, each only where a value within beta would round differently."""
import numpy as np
import pytest

import oracle
from _bandcheck import check_mx
from _parity import (E2M1, E4M3, THREADS, assert_bits_equal, band_check, bf16_values, bits_of,
                     rotate_within_beta, to_gpu_bf16, to_gpu_f32, unpack_codes)
from microscaling_quantize_dequantize_amd import workloads as W

pytestmark = pytest.mark.gpu

RS = [16, 32, 64, 128]


@pytest.fixture(scope="module")
def mx():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from microscaling_quantize_dequantize_amd import binding
    return binding


def no_negative_zero(x):
    """An exactly rotated zero is +0 (IEEE sum), while the unrotated path keeps
    -0; bit-exact comparisons across the two use inputs without -0."""
    x = x.copy()
    x[x == 0x8000] = 0
    return x


def bf16_exact(v):
    f = np.asarray(v, dtype=np.float32)
    assert np.array_equal(f.astype(np.float64), np.asarray(v, dtype=np.float64))
    return (f.view(np.uint32) >> 16).astype(np.uint16)


@pytest.mark.parametrize("r", RS)
def test_rotate_step_within_tolerance(mx, r):
    import torch
    rng = np.random.default_rng(r)
    x = W.generate("c3", rows=(0, 64))[:, :4096]
    for R in (W.hadamard_rotation(r), W.f32_to_bf16_bits(rng.standard_normal((r, r)).astype(np.float32))):
        yg = mx.mx_rotate(to_gpu_bf16(x), to_gpu_bf16(R))
        torch.cuda.synchronize()
        y, beta = oracle.rotate(x, R, r, threads=THREADS)
        rotate_within_beta(bits_of(yg).view(np.float32), y, beta)
    xf = W.random_f32((32, 2048), seed=r)
    Rf = rng.standard_normal((r, r)).astype(np.float32)
    yg = mx.mx_rotate(to_gpu_f32(xf), to_gpu_f32(Rf))
    torch.cuda.synchronize()
    y, beta = oracle.rotate(xf, Rf, r)
    rotate_within_beta(bits_of(yg).view(np.float32), y, beta)


@pytest.mark.parametrize("r", RS)
def test_identity_rotation_is_bit_exact(mx, r):
    import torch
    x = no_negative_zero(W.generate("c5a", rows=(0, 64)))
    xg = to_gpu_bf16(x)
    I = to_gpu_bf16(bf16_exact(np.eye(r)))
    for fmt in (E2M1, E4M3):
        a = mx.mx_qdq(fmt, xg, rot=I)
        b = mx.mx_qdq(fmt, xg)
        ca, sa = mx.mx_quantize(fmt, xg, rot=I)
        torch.cuda.synchronize()
        assert_bits_equal(bits_of(a), bits_of(b), f"identity r={r} fmt{fmt}")
        c_ref, s_ref = oracle.quantize(fmt, x, threads=THREADS)
        assert_bits_equal(bits_of(sa), s_ref, "identity scales")
        assert_bits_equal(bits_of(ca), c_ref, "identity codes")


@pytest.mark.parametrize("r", RS)
def test_exact_rotations_are_bit_exact(mx, r):
    """Signed permutations and diagonal matrices make y exact in fp32, so the
    GPU must match the oracle bit for bit (this also pins the fp32 inputs of
    the hardware conversions)."""
    import torch
    rng = np.random.default_rng(300 + r)
    x = no_negative_zero(W.generate("c5a", rows=(64, 128))[:, :4096])
    perm = rng.permutation(r)
    P = np.zeros((r, r))
    P[np.arange(r), perm] = rng.choice([-1.0, 1.0], size=r)
    D = np.diag(W.bf16_bits_to_f32(W.f32_to_bf16_bits(
        (rng.uniform(0.5, 2.0, size=r) * rng.choice([-1, 1], size=r)).astype(np.float32))).astype(np.float64))
    for R in (P, D):
        Rb = bf16_exact(R)
        for fmt in (E2M1, E4M3):
            out = mx.mx_qdq(fmt, to_gpu_bf16(x), rot=to_gpu_bf16(Rb))
            codes, scales = mx.mx_quantize(fmt, to_gpu_bf16(x), rot=to_gpu_bf16(Rb))
            torch.cuda.synchronize()
            assert_bits_equal(bits_of(out), oracle.qdq(fmt, x, Rb, r, threads=THREADS), f"exact R r={r}")
            c_ref, s_ref = oracle.quantize(fmt, x, Rb, r, threads=THREADS)
            assert_bits_equal(bits_of(scales), s_ref, "exact R scales")
            assert_bits_equal(bits_of(codes), c_ref, "exact R codes")


def _qdq_band(mx, fmt, x, R, r):
    import torch
    out = mx.mx_qdq(fmt, to_gpu_bf16(x), rot=to_gpu_bf16(R))
    torch.cuda.synchronize()
    y, beta = oracle.rotate(np.ascontiguousarray(x), R, r, threads=THREADS)
    return band_check(fmt, y, beta, deq_gpu=bf16_values(bits_of(out)))


def _quant_band(mx, fmt, x, R, r):
    import torch
    codes, scales = mx.mx_quantize(fmt, to_gpu_bf16(x), rot=to_gpu_bf16(R))
    torch.cuda.synchronize()
    y, beta = oracle.rotate(np.ascontiguousarray(x), R, r, threads=THREADS)
    return band_check(fmt, y, beta, codes_gpu=unpack_codes(fmt, bits_of(codes), x.shape[1]),
                      scales_gpu=bits_of(scales))


@pytest.mark.parametrize("fmt", [E2M1, E4M3])
@pytest.mark.parametrize("r", RS)
def test_hadamard_small_shapes(mx, fmt, r):
    for shape in [(3, 128), (7, 384), (33, 1024 + 128)]:
        x = W.random_bf16(shape, seed=shape[0] + r)
        R = W.hadamard_rotation(r)
        _qdq_band(mx, fmt, x, R, r)
        _quant_band(mx, fmt, x, R, r)


@pytest.mark.parametrize("fmt", [E2M1, E4M3])
@pytest.mark.parametrize("r", RS)
def test_dense_nonsymmetric_rotation(mx, fmt, r):
    """A dense matrix with no symmetry (seeded normal entries times r^-0.5,
    rounded to bf16), so that R and its transpose rotate differently by far
    more than the band: QDQ and quantize on every kernel of the rotation, on
    shapes of several tiles with a partial last one, within the band."""
    rng = np.random.default_rng(900 + r)
    R = W.f32_to_bf16_bits((rng.standard_normal((r, r)) / np.sqrt(r)).astype(np.float32))
    for shape in [(37, 1024), (300, 1152)]:
        x = W.random_bf16(shape, seed=shape[0] + r + 7 * fmt)
        y, beta = oracle.rotate(x, R, r, threads=THREADS)
        yt, _ = oracle.rotate(x, np.ascontiguousarray(R.T), r, threads=THREADS)
        assert (np.abs(yt - y) > beta).mean() > 0.5  # the transpose lies outside the band
        _qdq_band(mx, fmt, x, R, r)
        _quant_band(mx, fmt, x, R, r)


@pytest.mark.parametrize("r", [0] + RS)
def test_in_place_matches_out_of_place(mx, r):
    """dst == src: every QDQ kernel reads each element before its own wave
    writes it, so QDQ in place gives the bits it gives out of place (bf16 on
    every rotation kernel, small and many-workgroup shapes; fp32 sources)."""
    import torch
    for shape in [(300, 1152), (4096, 8192)]:
        x = W.random_bf16(shape, seed=77 + r + shape[0])
        xf = W.random_f32(shape, seed=78 + r + shape[0])
        R = to_gpu_bf16(W.hadamard_rotation(r)) if r else None
        Rf = to_gpu_f32(W.hadamard_rotation(r, "f32")) if r else None
        for fmt in (E2M1, E4M3):
            for src, rot in ((to_gpu_bf16(x), R), (to_gpu_f32(xf), Rf)):
                ref = mx.mx_qdq(fmt, src, rot=rot)
                t = src.clone()
                mx.mx_qdq(fmt, t, rot=rot, dst=t)
                torch.cuda.synchronize()
                assert np.array_equal(bits_of(t), bits_of(ref)), f"in place {shape} fmt{fmt} {src.dtype} r={r}"


@pytest.mark.parametrize("fmt", [E2M1, E4M3])
@pytest.mark.parametrize("shape", [(255, 128), (256, 128), (257, 128), (511, 128), (512, 128), (513, 128),
                                   (31, 4224), (16, 8192), (3, 22016)],
                         ids=lambda s: f"{s[0]}x{s[1]}")
def test_rot128_qdq_work_unit_edges(mx, fmt, shape):
    """QDQ with r = 128 runs in workgroups of 16 tiles of 16 blocks (256
    rotation blocks): tensors of a workgroup less one block, one, one plus a
    block, two less one block, two, two plus a block, and partial last
    tiles, all within the band of the oracle."""
    x = W.random_bf16(shape, seed=shape[0] * 7 + fmt)
    _qdq_band(mx, fmt, x, W.hadamard_rotation(128), 128)


@pytest.mark.parametrize("fmt", [E2M1, E4M3])
@pytest.mark.parametrize("r", [16, 32])
def test_rot_le32_qdq_work_unit_edges(mx, fmt, r):
    """QDQ with r = 16 or 32 runs on 64-element blocks in workgroups of 4
    tiles of 16 blocks: one block, a tile less one block, one tile, a tile
    plus one block, a workgroup less one block, one workgroup, a workgroup
    plus one block, and longer rows with a partial last tile, all within the
    band of the oracle."""
    R = W.hadamard_rotation(r)
    for shape in [(1, 64), (15, 64), (16, 64), (17, 64), (63, 64), (64, 64), (65, 64), (3, 4160), (31, 2112)]:
        x = W.random_bf16(shape, seed=shape[0] * 13 + shape[1] + r + fmt)
        _qdq_band(mx, fmt, x, R, r)


@pytest.mark.parametrize("shape", [(1, 128), (16, 2048), (1931, 2176)], ids=lambda s: f"{s[0]}x{s[1]}")
def test_rot128_lane_kernel_grid_edges(mx, shape):
    """Quantize (MX and NVFP4) and NVFP4 QDQ at r = 128 run on a persistent
    grid of one wave per workgroup, 8 per CU, whose waves take interleaved
    16-block tiles: one partial tile, exactly 16 tiles, and 2052 tiles (the
    last one partial) so that the first waves take a second tile.  MX
    quantize and NVFP4 QDQ and quantize of every row within the band of the
    oracle."""
    import torch
    from _bandcheck import check_nv
    x = W.random_bf16(shape, seed=shape[0] + 17)
    R = W.hadamard_rotation(128)
    xg, Rg = to_gpu_bf16(x), to_gpu_bf16(R)
    results = []
    for fmt in (E2M1, E4M3):
        codes, scales = mx.mx_quantize(fmt, xg, rot=Rg)
        results.append({"fmt": fmt, "codes": bits_of(codes), "scales": bits_of(scales)})
    check_mx(x, R, 128, results, what=f"lane kernel {shape}")
    g = 448.0 * 6.0 / float(np.abs(W.bf16_bits_to_f32(x)).max())
    gt = torch.tensor([g], dtype=torch.float32, device="cuda")
    c, sc = mx.mx_nvfp4_quantize(xg, gt, rot=Rg)
    q = mx.mx_nvfp4_qdq(xg, gt, rot=Rg)
    torch.cuda.synchronize()
    check_nv(x, R, 128, float(np.float32(g)), [{"codes": bits_of(c), "scales": bits_of(sc)}, {"deq": bits_of(q)}],
             what=f"lane kernel nvfp4 {shape}")


@pytest.mark.parametrize("fmt", [E2M1, E4M3])
@pytest.mark.parametrize("r,shape", [(16, (6, 96)), (16, (10, 160)), (32, (6, 96)), (32, (10, 160)), (16, (5, 96))],
                         ids=lambda v: str(v))
def test_small_rotations_across_rows(mx, fmt, r, shape):
    """Rotations of 16 and 32 run on 64-element blocks (two or four copies of
    R on the diagonal) when the tensor is a whole number of them, so with K
    not a multiple of 64 a block holds the end of one row and the start of
    the next: QDQ and quantize stay within the oracle's band.  (5, 96) is not
    a whole number of 64-blocks and takes the 32-element blocks."""
    x = W.random_bf16(shape, seed=shape[0] * 13 + r + fmt)
    R = W.hadamard_rotation(r)
    _qdq_band(mx, fmt, x, R, r)
    _quant_band(mx, fmt, x, R, r)


def full_tensor_rotated(mx, name, rs):
    """Every row of a full-size layer, for each rotation size: MXFP4 and MXFP8
    QDQ and quantize, each checked against the oracle's rotation of the same
    row within the band (tests/bandcheck.c), and the cap of 0.01% differing
    elements asserted on the whole tensor; on the GPU, QDQ equals the
    dequantize of the quantize bit for bit."""
    import torch
    x = W.generate(name)
    M, K = x.shape
    xg = to_gpu_bf16(x)
    for r in rs:
        R = W.hadamard_rotation(r)
        Rg = to_gpu_bf16(R)
        results = []
        for fmt in (E2M1, E4M3):
            print(f"{name} {M}x{K} rotation {r} fmt {fmt}: launching", flush=True)
            q = mx.mx_qdq(fmt, xg, rot=Rg)
            codes, scales = mx.mx_quantize(fmt, xg, rot=Rg)
            d = mx.mx_dequantize(fmt, codes, scales, K)
            assert torch.equal(d.view(torch.int16), q.view(torch.int16)), "qdq != dequantize(quantize)"
            results.append({"fmt": fmt, "deq": bits_of(q)})
            results.append({"fmt": fmt, "codes": bits_of(codes), "scales": bits_of(scales)})
            del q, codes, scales, d
        stats = check_mx(x, R, r, results, what=f"{name} r={r}")
        for res, st in zip(results, stats):
            print(name, r, res["fmt"], "qdq" if "deq" in res else "quantize", st, flush=True)
            assert st["elements"] == M * K


def test_c3_mxfp4_qdq_rot32(mx):
    """4096 x 8192, columns scaled LogNormal(0, 1), rotation 32."""
    full_tensor_rotated(mx, "c3", (32,))


def test_c4_quantize_rot128(mx):
    """8192 x 28672 down-projection input, Student-t (nu = 3), rotation 128
    (the MXFP4 quantize of the layer, and its MXFP8 and QDQ siblings)."""
    full_tensor_rotated(mx, "c4", (128,))


@pytest.mark.parametrize("name,rs", [("c5a", (16, 64)), ("c5b", (16, 64, 128)), ("c5c", (16, 64))])
def test_c5_layers_rotated(mx, name, rs):
    """The three Llama-3.1-70B layer shapes (N(0, 0.02^2) weights with
    subnormal-range and saturating groups), every rotation of the sweep."""
    full_tensor_rotated(mx, name, rs)


@pytest.mark.parametrize("fmt", [E2M1, E4M3])
@pytest.mark.parametrize("r", RS)
def test_fp32_source_rotated(mx, fmt, r):
    import torch
    rng = np.random.default_rng(500 + r)
    x = W.random_f32((48, 1024), seed=r)
    R = (W.sylvester_hadamard(r) / np.sqrt(r)).astype(np.float32)
    out = mx.mx_qdq(fmt, to_gpu_f32(x), rot=to_gpu_f32(R))
    torch.cuda.synchronize()
    y, beta = oracle.rotate(x, R, r)
    band_check(fmt, y, beta, deq_gpu=bits_of(out).view(np.float32).astype(np.float64), dst_bf16=False)
    Pm = np.zeros((r, r), dtype=np.float32)
    Pm[np.arange(r), rng.permutation(r)] = 1.0
    out = mx.mx_qdq(fmt, to_gpu_f32(x), rot=to_gpu_f32(Pm))
    torch.cuda.synchronize()
    assert_bits_equal(bits_of(out), oracle.qdq(fmt, x, Pm, r), "f32 permutation")


@pytest.mark.parametrize("fmt,r", [(E2M1, 16), (E4M3, 64), (E2M1, 128), (E4M3, 128)])
def test_fp32_source_rotated_many_steps(mx, fmt, r):
    """fp32 sources on a tensor of more 16 KiB steps than the grid has
    workgroups (so workgroups loop) and a partial last step: QDQ within the
    band of the oracle on every element, and the rotation alone within
    beta."""
    import torch
    M, K = 8200, 1152
    x = W.random_f32((M, K), seed=700 + r)
    R = (W.sylvester_hadamard(r) / np.sqrt(r)).astype(np.float32)
    out = mx.mx_qdq(fmt, to_gpu_f32(x), rot=to_gpu_f32(R))
    yg = mx.mx_rotate(to_gpu_f32(x), to_gpu_f32(R))
    torch.cuda.synchronize()
    y, beta = oracle.rotate(x, R, r, threads=THREADS)
    band_check(fmt, y, beta, deq_gpu=bits_of(out).view(np.float32).astype(np.float64), dst_bf16=False)
    rotate_within_beta(bits_of(yg).view(np.float32), y, beta)


@pytest.mark.parametrize("r", [16, 64, 128])
def test_rotate_bf16_many_steps(mx, r):
    """The rotation alone of bf16 sources on a tensor of more steps than the
    grid has workgroups and a partial last step, within beta everywhere."""
    import torch
    M, K = 8200, 1152
    x = W.random_bf16((M, K), seed=800 + r)
    R = W.hadamard_rotation(r)
    yg = mx.mx_rotate(to_gpu_bf16(x), to_gpu_bf16(R))
    torch.cuda.synchronize()
    y, beta = oracle.rotate(x, R, r, threads=THREADS)
    rotate_within_beta(bits_of(yg).view(np.float32), y, beta)


def _spread_mask(nonfinite, block):
    """Groups [M, K/32] and elements [M, K] of every `block`-element block of a
    row that holds a non-finite input."""
    M, K = nonfinite.shape
    bad = nonfinite.reshape(M, K // block, block).any(axis=2)
    return np.repeat(bad, block // 32, axis=1), np.repeat(bad, block, axis=1)


@pytest.mark.parametrize("r", RS)
def test_nonfinite_inputs_rotated(mx, r):
    """NaN and Inf inputs through every rotated bf16 kernel.  The kernels
    rotate blocks of max(r, 64) elements here (r = 16 and 32 as a
    block-diagonal 64 x 64 matrix whose zeros turn an Inf into NaN), so every
    group of such a block is non-finite: scale byte 0xFF, codes 0x7F (E4M3) or
    0x0 (E2M1), dequantized NaN.  The oracle's non-finite groups are the
    r-chunks' own, a subset; outside the marked blocks an exact rotation (a
    signed permutation) must match the oracle bit for bit, and a Hadamard
    rotation must leave no group non-finite."""
    import torch
    x = no_negative_zero(W.generate("c5a", rows=(0, 64))[:, :4096])
    x[0, 5] = 0x7FC0      # NaN
    x[3, 300] = 0x7F80    # +Inf
    x[7, 1000] = 0xFF80   # -Inf and +Inf in one chunk
    x[7, 1001] = 0x7F80
    x[20, 2047] = 0x7F80  # the last element of a 128-block
    x[63, 4095] = 0xFFC0  # a negative NaN, the tensor's last element
    M, K = x.shape
    gbad, ebad = _spread_mask((x & 0x7FFF) >= 0x7F80, max(r, 64))
    rng = np.random.default_rng(700 + r)
    P = np.zeros((r, r))
    P[np.arange(r), rng.permutation(r)] = rng.choice([-1.0, 1.0], size=r)
    xg = to_gpu_bf16(x)
    for name, R in (("permutation", bf16_exact(P)), ("hadamard", W.hadamard_rotation(r))):
        Rg = to_gpu_bf16(R)
        for fmt in (E2M1, E4M3):
            nan_code = 0x7F if fmt == E4M3 else 0x0
            out = mx.mx_qdq(fmt, xg, rot=Rg)
            codes, scales = mx.mx_quantize(fmt, xg, rot=Rg)
            bcodes, blocked = mx.mx_quantize_blocked(fmt, xg, rot=Rg)
            torch.cuda.synchronize()
            tag = f"r={r} {name} fmt{fmt}"
            s, o = bits_of(scales), bits_of(out)
            c = unpack_codes(fmt, bits_of(codes), K)
            assert np.array_equal(s == 0xFF, gbad), f"non-finite groups {tag}"
            assert np.all(c[ebad] == nan_code), f"non-finite codes {tag}"
            assert np.array_equal((o & 0x7FFF) > 0x7F80, ebad), f"NaN outputs {tag}"
            assert_bits_equal(bits_of(bcodes), bits_of(codes), f"blocked codes {tag}")
            assert_bits_equal(bits_of(blocked), oracle.scales_to_blocked(s, K), f"blocked scales {tag}")
            if name == "permutation":
                c_ref, s_ref = oracle.quantize(fmt, x, R, r, threads=THREADS)
                assert np.all(gbad[s_ref == 0xFF]), f"oracle non-finite groups inside the blocks {tag}"
                assert_bits_equal(s[~gbad], s_ref[~gbad], f"scales {tag}")
                assert_bits_equal(c[~ebad], unpack_codes(fmt, c_ref, K)[~ebad], f"codes {tag}")
                o_ref = oracle.qdq(fmt, x, R, r, threads=THREADS)
                assert_bits_equal(o[~ebad], o_ref[~ebad], f"qdq {tag}")


@pytest.mark.parametrize("r", RS)
def test_nonfinite_inputs_rotated_fp32(mx, r):
    """fp32 sources rotate in blocks of max(r, 32) elements; the same rule."""
    import torch
    x = W.random_f32((16, 1024), seed=40 + r)
    x[0, 5] = np.nan
    x[3, 300] = np.inf
    x[7, 600] = -np.inf
    x[15, 1023] = np.nan
    gbad, ebad = _spread_mask(~np.isfinite(x), max(r, 32))
    rng = np.random.default_rng(800 + r)
    P = np.zeros((r, r), dtype=np.float32)
    P[np.arange(r), rng.permutation(r)] = rng.choice([-1.0, 1.0], size=r)
    for fmt in (E2M1, E4M3):
        out = mx.mx_qdq(fmt, to_gpu_f32(x), rot=to_gpu_f32(P))
        torch.cuda.synchronize()
        o = bits_of(out)
        assert np.array_equal((o & 0x7FFFFFFF) > 0x7F800000, ebad), f"NaN outputs r={r} fmt{fmt}"
        o_ref = oracle.qdq(fmt, x, P, r).view(np.uint32)
        assert_bits_equal(o[~ebad], o_ref[~ebad], f"f32 permutation r={r} fmt{fmt}")
