"""Parity helpers shared by the GPU tests: tensor transfer, bit-exact
comparison, and the tolerance band of the rotated path.

Rotated path bar (stated tolerance): a rotated value may differ from the
exact one by at most beta = 1e-5 * sum_t |x[t] R[t][j]| (fp32 accumulation;
the products are exact for bf16 sources and rounded once to fp32 for fp32
sources, at most 2^-24 |x[t] R[t][j]| each, well inside beta); at most 0.01%
of the elements may differ from the oracle's
result, and each difference must be one that some rotated value within beta
would produce:
  - a group's scale may be any of those the abs-max can take within the band
    (floor(log2) of max(|y|-beta) ... max(|y|+beta));
  - under the scale the GPU chose, each element must lie between the
    quantize-dequantize of y-beta and of y+beta (the rounding is monotone).
Every element outside those ambiguity bands is therefore bit-exact.
"""
from __future__ import annotations

import os

import numpy as np

import oracle

THREADS = max(1, min(16, os.cpu_count() or 1))
E2M1, E4M3 = 0, 1
SIGN_BIT = {E2M1: 0x8, E4M3: 0x80}


# ---- transfer ------------------------------------------------------------

def to_gpu_bf16(bits: np.ndarray):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def to_gpu_f32(a: np.ndarray):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()


def bits_of(t) -> np.ndarray:
    """bf16 tensor -> uint16 bits; fp32 tensor -> uint32 bits; uint8 as is."""
    import torch
    c = t.detach().cpu().contiguous()
    if c.dtype == torch.bfloat16:
        return c.view(torch.int16).numpy().view(np.uint16)
    if c.dtype == torch.float32:
        return c.numpy().view(np.uint32)
    return c.numpy()


def bf16_values(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def f64_to_bf16_values(v: np.ndarray) -> np.ndarray:
    """Round doubles that are exact in fp32 to bf16 (nearest-even) and return
    the values (used for band bounds, which are code values times 2^s)."""
    f = v.astype(np.float32)
    u = f.view(np.uint32)
    r = ((u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)) << np.uint32(16)
    out = r.view(np.float32).astype(np.float64)
    return np.where(np.isnan(v), np.nan, out)


def _as_bits(a: np.ndarray) -> np.ndarray:
    a = np.asarray(a)
    if a.dtype == np.float32:
        return a.view(np.uint32)
    if a.dtype == np.float64:
        return a.view(np.uint64)
    return a


def assert_bits_equal(got: np.ndarray, want: np.ndarray, what: str) -> None:
    got, want = _as_bits(got), _as_bits(want)
    assert got.shape == want.shape, (what, got.shape, want.shape)
    bad = np.flatnonzero(got.ravel() != want.ravel())
    if bad.size:
        i = bad[:8]
        raise AssertionError(f"{what}: {bad.size} of {got.size} differ; first at flat {i.tolist()}: "
                             f"got {got.ravel()[i].tolist()} want {want.ravel()[i].tolist()}")


def unpack_codes(fmt: int, codes: np.ndarray, K: int) -> np.ndarray:
    if fmt == E4M3:
        return codes
    M = codes.shape[0]
    return np.stack([codes & 0xF, codes >> 4], axis=2).reshape(M, K)


def code_values(fmt: int, codes: np.ndarray) -> np.ndarray:
    table = np.array([oracle.decode(fmt, c) for c in range(16 if fmt == E2M1 else 256)])
    return table[codes]


# ---- the band of the rotated path -----------------------------------------

def _bounds(fmt, y, beta, s):
    lo = oracle.qdq_value_n(fmt, y - beta, s)
    hi = oracle.qdq_value_n(fmt, y + beta, s)
    return lo, hi


def band_check(fmt: int, y: np.ndarray, beta: np.ndarray, *, deq_gpu=None, dst_bf16=True,
               codes_gpu=None, scales_gpu=None) -> dict:
    """Check GPU results for rows of a rotated matrix against the band.

    y, beta: [M, K] float64 from the oracle.  Pass either deq_gpu (QDQ output
    values as float64) or codes_gpu (unpacked, [M, K]) with scales_gpu
    ([M, K/32] bytes).  Row blocks are checked on a thread pool; returns
    counters and raises on a violation."""
    from concurrent.futures import ThreadPoolExecutor
    M = y.shape[0]
    step = max(1, (M + THREADS - 1) // THREADS)

    def part(r0):
        r1 = min(M, r0 + step)
        return _band_rows(fmt, y[r0:r1], beta[r0:r1],
                          deq_gpu=None if deq_gpu is None else deq_gpu[r0:r1], dst_bf16=dst_bf16,
                          codes_gpu=None if codes_gpu is None else codes_gpu[r0:r1],
                          scales_gpu=None if scales_gpu is None else scales_gpu[r0:r1])

    with ThreadPoolExecutor(max_workers=THREADS) as ex:
        parts = list(ex.map(part, range(0, M, step)))
    out = {"elements": sum(p["elements"] for p in parts), "differ": sum(p["differ"] for p in parts),
           "ambiguous_scale_groups": sum(p["ambiguous_scale_groups"] for p in parts)}
    frac = out["differ"] / max(1, out["elements"])
    assert frac <= 1e-4, f"{out['differ']} elements ({frac:.2e}) differ from the oracle (limit 1e-4)"
    return out


def _band_rows(fmt, y, beta, *, deq_gpu, dst_bf16, codes_gpu, scales_gpu) -> dict:
    M, K = y.shape
    G = M * K // 32
    yg = y.reshape(G, 32)
    bg = beta.reshape(G, 32)
    amax_lo = np.max(np.maximum(np.abs(yg) - bg, 0.0), axis=1)
    amax_hi = np.max(np.abs(yg) + bg, axis=1)
    s_lo = oracle.scale_exponent_n(fmt, amax_lo)
    s_hi = oracle.scale_exponent_n(fmt, amax_hi)
    s_exact = oracle.scale_exponent_n(fmt, np.max(np.abs(yg), axis=1))
    ref = np.repeat(s_exact, 32)
    exact_val = oracle.qdq_value_n(fmt, yg.ravel(), ref).reshape(G, 32)

    if codes_gpu is not None:
        s_gpu = scales_gpu.reshape(G).astype(np.int32) - 127
        bad_scale = (s_gpu < s_lo) | (s_gpu > s_hi)
        assert not bad_scale.any(), f"{bad_scale.sum()} scales outside the band"
        v_gpu = (code_values(fmt, codes_gpu.reshape(G, 32)) * np.exp2(s_gpu.astype(np.float64))[:, None])
        lo, hi = _bounds(fmt, yg.ravel(), bg.ravel(), np.repeat(s_gpu, 32))
        lo, hi = lo.reshape(G, 32), hi.reshape(G, 32)
        ok = (v_gpu >= lo) & (v_gpu <= hi)
        assert ok.all(), f"{(~ok).sum()} codes outside the band, e.g. group {np.flatnonzero(~ok.all(1))[:4]}"
        differ = (v_gpu != exact_val) | (s_gpu != s_exact)[:, None]
    else:
        d = deq_gpu.reshape(G, 32)
        group_ok = np.zeros(G, dtype=bool)
        for s_c in np.unique(np.concatenate([s_lo, s_hi])):
            sel = (s_lo <= s_c) & (s_c <= s_hi)
            if not sel.any():
                continue
            idx = np.flatnonzero(sel)
            lo, hi = _bounds(fmt, yg[idx].ravel(), bg[idx].ravel(), np.int32(s_c))
            if dst_bf16:
                lo, hi = f64_to_bf16_values(lo), f64_to_bf16_values(hi)
            lo, hi = lo.reshape(-1, 32), hi.reshape(-1, 32)
            group_ok[idx] |= ((d[idx] >= lo) & (d[idx] <= hi)).all(axis=1)
        assert group_ok.all(), f"{(~group_ok).sum()} groups outside the band, e.g. {np.flatnonzero(~group_ok)[:4]}"
        ev = f64_to_bf16_values(exact_val) if dst_bf16 else exact_val
        differ = d != ev
    return {"elements": M * K, "differ": int(differ.sum()), "ambiguous_scale_groups": int((s_lo != s_hi).sum())}


def rotate_within_beta(y_gpu: np.ndarray, y: np.ndarray, beta: np.ndarray) -> float:
    """Check |y_gpu - y| <= beta elementwise; return the largest ratio."""
    err = np.abs(y_gpu.astype(np.float64) - y)
    ratio = np.where(beta > 0, err / np.where(beta > 0, beta, 1.0), np.where(err > 0, np.inf, 0.0))
    worst = float(ratio.max()) if ratio.size else 0.0
    assert worst <= 1.0, f"rotated values exceed the tolerance: worst |err|/beta = {worst}"
    return worst


# ---- the band of the rotated NVFP4 path ---------------------------------------

def _f32_down(v):
    f = np.asarray(v, dtype=np.float64).astype(np.float32)
    return np.where(f.astype(np.float64) > v, np.nextafter(f, np.float32(-np.inf)), f).astype(np.float32)


def _f32_up(v):
    f = np.asarray(v, dtype=np.float64).astype(np.float32)
    return np.where(f.astype(np.float64) < v, np.nextafter(f, np.float32(np.inf)), f).astype(np.float32)


def nv_band_check(y: np.ndarray, beta: np.ndarray, g: float, *, deq_gpu=None, codes_gpu=None,
                  scales_gpu=None) -> dict:
    """The band of the rotated path for NVFP4: with |y_gpu - y| <= beta, a
    16-group's E4M3 scale byte lies between those of its smallest and largest
    possible abs-max (the scale is monotone in amax), and under the GPU's
    scale each element lies between the values of y - beta and y + beta (the
    code is monotone in x).  Pass deq_gpu (QDQ output values, bf16 as
    float64) or codes_gpu (unpacked [M, K]) with scales_gpu ([M, K/16])."""
    M, K = y.shape
    G = M * K // 16
    yg, bg = y.reshape(G, 16), beta.reshape(G, 16)
    sb_lo = oracle.nv_scale_byte_n(g, _f32_down(np.max(np.maximum(np.abs(yg) - bg, 0.0), axis=1)))
    sb_hi = oracle.nv_scale_byte_n(g, _f32_up(np.max(np.abs(yg) + bg, axis=1)))
    y32 = yg.astype(np.float32)
    sb_ex = oracle.nv_scale_byte_n(g, np.abs(y32).max(axis=1))
    code_ex = oracle.nv_code_n(g, np.repeat(sb_ex, 16).reshape(G, 16), y32)
    lo_x, hi_x = _f32_down(yg - bg), _f32_up(yg + bg)
    if codes_gpu is not None:
        sb = scales_gpu.reshape(G)
        bad = (sb < sb_lo) | (sb > sb_hi)
        assert not bad.any(), f"{bad.sum()} NVFP4 scales outside the band"
        sbr = np.repeat(sb, 16).reshape(G, 16)
        c = codes_gpu.reshape(G, 16)
        v, vlo, vhi = (code_values(E2M1, cc) for cc in (c, oracle.nv_code_n(g, sbr, lo_x),
                                                        oracle.nv_code_n(g, sbr, hi_x)))
        ok = (v >= vlo) & (v <= vhi)
        assert ok.all(), f"{(~ok).sum()} NVFP4 codes outside the band"
        differ = (c != code_ex) | (sb != sb_ex)[:, None]
    else:
        d = deq_gpu.reshape(G, 16)
        group_ok = np.zeros(G, dtype=bool)
        for cand in range(int(sb_lo.min()), int(sb_hi.max()) + 1):
            idx = np.flatnonzero((sb_lo <= cand) & (cand <= sb_hi))
            if idx.size == 0:
                continue
            sbr = np.full((idx.size, 16), cand, dtype=np.uint8)
            vlo = f64_to_bf16_values(oracle.nv_value_n(g, sbr, oracle.nv_code_n(g, sbr, lo_x[idx])).astype(np.float64))
            vhi = f64_to_bf16_values(oracle.nv_value_n(g, sbr, oracle.nv_code_n(g, sbr, hi_x[idx])).astype(np.float64))
            group_ok[idx] |= ((d[idx] >= vlo) & (d[idx] <= vhi)).all(axis=1)
        assert group_ok.all(), f"{(~group_ok).sum()} NVFP4 groups outside the band"
        ev = f64_to_bf16_values(oracle.nv_value_n(g, np.repeat(sb_ex, 16).reshape(G, 16), code_ex).astype(np.float64))
        differ = d != ev
    out = {"elements": M * K, "differ": int(differ.sum()), "ambiguous_scale_groups": int((sb_lo != sb_hi).sum())}
    frac = out["differ"] / max(1, out["elements"])
    assert frac <= 1e-4, f"{out['differ']} NVFP4 elements ({frac:.2e}) differ from the oracle (limit 1e-4)"
    return out


# ---- the scaled-MFMA GEMM error bound ----------------------------------------

def gemm_error_bound(fmt: int, a_dq: np.ndarray, b_dq: np.ndarray) -> np.ndarray:
    """Bound on |C - A_dq . B_dq^T| for the gfx950 scaled MFMA with fp32
    accumulation (before alpha and the output rounding), from two sources:
      * fp32 accumulation with faithful additions: each 64-deep k-step's
        sum is added to the accumulator rounded to nearest-even within a
        short window of guard bits and with no sticky bit (characterised on
        gfx950, test_accumulation_across_steps_is_faithful: a tail 7 bits
        below the ulp is dropped, so a sum just above a midpoint can round
        down), so each addition errs by less than one ulp of its result and
        the bound is K * 2^-23 * sum_k |a_k b_k|, twice the
        round-to-nearest one;
      * E4M3 only: the matrix core sums the products of each 8-element
        chunk of k in a window of 14 bits below the chunk's largest
        product, dropping lower bits (characterised on gfx950; the
        characterisation test pins it), so each chunk adds at most
        8 * 2^(floor(log2 max_k |a_k b_k|) - 13).  E2M1 products span at
        most 2^7 (0.25 .. 36) and always fit the window.
    """
    K = a_dq.shape[1]
    bound = K * 2.0 ** -23 * (np.abs(a_dq) @ np.abs(b_dq).T)
    if fmt == E4M3:
        for c in range(K // 8):
            p = np.abs(a_dq[:, None, 8 * c:8 * c + 8] * b_dq[None, :, 8 * c:8 * c + 8]).max(-1)
            _, e = np.frexp(p)  # p = f * 2^e with f in [0.5, 1): floor(log2 p) = e - 1
            bound += np.where(p > 0, 8.0 * np.exp2(e - 1 - 13), 0.0)
    return bound
