"""Seeded synthetic inputs for MX quantize / dequantize.

This module only draws inputs: it holds none of the quantization arithmetic,
and it imports neither the HIP binding nor the CPU oracle, so both sides can
read the same buffers.  Every array is returned as bf16 bit patterns
(``uint16``) or ``float32``; values are drawn in float32/float64 and rounded
once to bf16 (nearest-even).

The shapes stand in for the layers the pages benchmark: the Llama-3.1-70B
layer shapes (8192, 8192), (8192, 57344) and (28672, 8192) listed in the
benchmark script reviewed on "Add QuTLASS support to vLLM" (review of
benchmarks/kernels/bench_mxfp4_qutlass.py), read literally as M x K.  The
rotation is the normalised Sylvester Hadamard matrix H_r * r^-0.5 built in the
activation dtype, as in that benchmark's ``hadamard(group_size) *
group_size**-0.5`` (same page, same review).

Generation is split in row blocks, each with its own generator seeded from
(seed, block), so any block can be regenerated on its own.
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np

ROW_BLOCK = 64


# ---- bf16 helpers (input preparation only) --------------------------------

def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (nearest-even) and return the bits."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


# ---- rotation matrices ---------------------------------------------------

def sylvester_hadamard(r: int) -> np.ndarray:
    """Sylvester Hadamard matrix of order r (entries +-1), float64."""
    if r < 1 or r & (r - 1):
        raise ValueError("order must be a power of two")
    h = np.ones((1, 1))
    while h.shape[0] < r:
        h = np.block([[h, h], [h, -h]])
    return h


def hadamard_rotation(r: int, dtype: str = "bf16") -> np.ndarray:
    """H_r * r^-0.5 rounded once into the activation dtype.

    bf16 is returned as bit patterns (uint16), f32 as float32."""
    m = sylvester_hadamard(r) * (1.0 / math.sqrt(r))
    if dtype == "f32":
        return m.astype(np.float32)
    return f32_to_bf16_bits(_f64_to_f32_for_bf16(m))


def _f64_to_f32_for_bf16(m: np.ndarray) -> np.ndarray:
    # Rounding float64 -> float32 -> bf16 rounds twice; the second rounding
    # only differs from a direct one when the first lands exactly on a bf16
    # halfway point, which does not happen for +-r^-0.5 (checked by a test).
    return m.astype(np.float32)


# ---- the workloads --------------------------------------------------------

@dataclass(frozen=True)
class Workload:
    name: str
    M: int
    K: int
    seed: int
    description: str


WORKLOADS = {
    "c1": Workload("c1", 128, 4096, 101,
                   "N(0,1); 0.1% of entries x50; 4 all-zero groups"),
    "c2": Workload("c2", 8192, 8192, 102,
                   "Student-t nu=4 x0.5; rows i%64==0 x1000"),
    "c3": Workload("c3", 4096, 8192, 103,
                   "N(0,1) x per-column LogNormal(0,1) scale"),
    "c4": Workload("c4", 8192, 28672, 104, "Student-t nu=3"),
    "c5a": Workload("c5a", 8192, 8192, 105,
                    "N(0, 0.02^2); 1/1024 subnormal-range and 1/1024 saturating groups"),
    "c5b": Workload("c5b", 8192, 57344, 106,
                    "N(0, 0.02^2); 1/1024 subnormal-range and 1/1024 saturating groups"),
    "c5c": Workload("c5c", 28672, 8192, 107,
                    "N(0, 0.02^2); 1/1024 subnormal-range and 1/1024 saturating groups"),
}

C1_ZERO_GROUPS = ((0, 0), (31, 64), (64, 127), (127, 5))


def _rng(seed: int, block: int) -> np.random.Generator:
    return np.random.default_rng([seed, block])


def _c1(w: Workload) -> np.ndarray:
    rng = _rng(w.seed, 0)
    x = rng.standard_normal((w.M, w.K), dtype=np.float32)
    zero = np.zeros((w.M, w.K), dtype=bool)
    for row, g in C1_ZERO_GROUPS:
        zero[row, g * 32:(g + 1) * 32] = True
    candidates = np.flatnonzero(~zero.ravel())
    n_out = int(round(0.001 * w.M * w.K))
    pos = rng.choice(candidates, size=n_out, replace=False)
    flat = x.ravel()
    flat[pos] *= np.float32(50.0)
    x[zero] = 0.0
    return f32_to_bf16_bits(x)


def _block_values(w: Workload, r0: int, r1: int, col_scale=None) -> np.ndarray:
    rng = _rng(w.seed, r0 // ROW_BLOCK)
    shape = (r1 - r0, w.K)
    if w.name == "c2":
        x = (0.5 * rng.standard_t(4, size=shape)).astype(np.float32)
        rows = np.arange(r0, r1)
        x[rows % 64 == 0] *= np.float32(1000.0)
    elif w.name == "c3":
        x = rng.standard_normal(shape, dtype=np.float32) * col_scale[None, :]
    elif w.name == "c4":
        x = rng.standard_t(3, size=shape).astype(np.float32)
    elif w.name.startswith("c5"):
        x = rng.standard_normal(shape, dtype=np.float32) * np.float32(0.02)
        _c5_special_groups(rng, x)
    else:
        raise KeyError(w.name)
    return x


def _c5_special_groups(rng: np.random.Generator, x: np.ndarray) -> None:
    """1/1024 of the groups in the block get values of magnitude below
    2^-120 (N(0,1) clipped to |z| <= 3.9, times 2^-124, some bf16
    subnormal); another 1/1024 get their largest element set to
    +-1.96875 * 2^floor(log2 amax), a mantissa that saturates both formats."""
    rows, K = x.shape
    groups = x.reshape(rows * K // 32, 32)
    n = groups.shape[0] // 1024
    if n == 0:
        return
    pick = rng.choice(groups.shape[0], size=2 * n, replace=False)
    sub, sat = pick[:n], pick[n:]
    z = np.clip(rng.standard_normal((n, 32), dtype=np.float32), -3.9, 3.9)
    groups[sub] = z * np.float32(2.0 ** -124)
    g = groups[sat]
    # amax is taken on the bf16-rounded group, as the method will see it
    gb = bf16_bits_to_f32(f32_to_bf16_bits(g))
    j = np.argmax(np.abs(gb), axis=1)
    amax = np.abs(gb[np.arange(n), j]).astype(np.float64)
    _, ex = np.frexp(amax)  # amax = f * 2^ex, f in [0.5, 1)
    val = np.ldexp(1.96875, ex - 1) * np.sign(gb[np.arange(n), j])
    g[np.arange(n), j] = val.astype(np.float32)
    groups[sat] = g


def generate(name: str, rows: tuple[int, int] | None = None) -> np.ndarray:
    """bf16 bits [M, K] of a named workload (or of rows [r0, r1), which must
    start on a multiple of ROW_BLOCK unless the workload is c1)."""
    w = WORKLOADS[name]
    if name == "c1":
        x = _c1(w)
        return x if rows is None else x[rows[0]:rows[1]].copy()
    r0, r1 = (0, w.M) if rows is None else rows
    if r0 % ROW_BLOCK:
        raise ValueError("row range must start on a block boundary")
    col_scale = None
    if name == "c3":
        col_scale = np.random.default_rng([w.seed, 1 << 30]).lognormal(
            0.0, 1.0, size=w.K).astype(np.float32)
    out = np.empty((r1 - r0, w.K), dtype=np.uint16)
    for b0 in range(r0, r1, ROW_BLOCK):
        b1 = min(r1, b0 - b0 % ROW_BLOCK + ROW_BLOCK)
        blk0 = b0 - b0 % ROW_BLOCK
        vals = _block_values(w, blk0, min(w.M, blk0 + ROW_BLOCK), col_scale)
        out[b0 - r0:b1 - r0] = f32_to_bf16_bits(vals[b0 - blk0:b1 - blk0])
    return out


def random_bf16(shape, seed: int, scale: float = 1.0) -> np.ndarray:
    """Plain N(0, scale^2) bf16 bits, for small parity and edge cases."""
    rng = np.random.default_rng([seed, 7])
    return f32_to_bf16_bits(rng.standard_normal(shape, dtype=np.float32) * np.float32(scale))


def random_f32(shape, seed: int, scale: float = 1.0) -> np.ndarray:
    rng = np.random.default_rng([seed, 8])
    return rng.standard_normal(shape, dtype=np.float32) * np.float32(scale)
