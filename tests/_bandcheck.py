"""Whole-tensor comparator of the rotated path (tests/bandcheck.c).

TEST INFRASTRUCTURE.  ``build()`` compiles bandcheck.c together with the CPU
oracle's source into tests/libbandcheck.so (gcc, strict IEEE).  ``check_mx``
and ``check_nv`` split the rows over a thread pool (ctypes releases the GIL),
rotate each row once with the oracle and check every GPU result handed in
against the band that tests/_parity.py states; they return the summed
counters and raise on a violation or when more than 0.01% of a result's
elements differ from the oracle.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

import numpy as np

from _parity import THREADS

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRC = [os.path.join(HERE, "bandcheck.c"), os.path.join(ROOT, "oracle", "mxoracle.c")]
LIB = os.path.join(HERE, "libbandcheck.so")


def build(out: str = LIB, extra: list[str] | None = None) -> str:
    tmp = out + ".tmp"
    subprocess.check_call(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-Wall", "-Wextra", "-fno-fast-math",
                           "-ffp-contract=off", "-I", os.path.join(ROOT, "oracle"), *(extra or []),
                           "-o", tmp, *SRC, "-lm"])
    os.replace(tmp, out)
    return out


class Result(ctypes.Structure):
    _fields_ = [("kind", ctypes.c_int32), ("fmt", ctypes.c_int32), ("deq", ctypes.c_void_p),
                ("codes", ctypes.c_void_p), ("scales", ctypes.c_void_p), ("elements", ctypes.c_int64),
                ("differ", ctypes.c_int64), ("ambiguous", ctypes.c_int64), ("violations", ctypes.c_int64),
                ("first_bad", ctypes.c_int64)]


_lib = None


def lib():
    global _lib
    if _lib is None:
        path = os.environ.get("BANDCHECK_LIB", LIB)
        if not os.path.exists(path):
            build()
        L = ctypes.CDLL(path)
        vp, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
        L.bc_mx_rows.argtypes = [vp, i64, i64, i64, vp, i32, vp, i32]
        L.bc_mx_rows.restype = i32
        L.bc_nv_rows.argtypes = [vp, i64, i64, i64, vp, i32, ctypes.c_float, vp, i32]
        L.bc_nv_rows.restype = i32
        _lib = L
    return _lib


def _results(fmt_of, results):
    """results: list of dicts with 'fmt' and either 'deq' (uint16 bits) or
    'codes' + 'scales' (uint8); arrays are kept alive by the caller."""
    out = []
    for r in results:
        kind = 0 if "deq" in r else 1
        arrs = [np.ascontiguousarray(r[k]) for k in (("deq",) if kind == 0 else ("codes", "scales"))]
        if kind == 0:
            assert arrs[0].dtype == np.uint16
        else:
            assert arrs[0].dtype == np.uint8 and arrs[1].dtype == np.uint8
        out.append((kind, fmt_of(r), arrs))
    return out


def _run(fn, M, prepared, threads):
    """Run fn(row0, row1, res_array) over row ranges; sum the counters."""
    threads = max(1, min(threads, M))
    step = max(1, (M + threads * 4 - 1) // (threads * 4))
    ranges = [(r0, min(M, r0 + step)) for r0 in range(0, M, step)]

    def part(rr):
        arr = (Result * len(prepared))()
        for k, (kind, fmt, arrs) in enumerate(prepared):
            arr[k].kind, arr[k].fmt = kind, fmt
            if kind == 0:
                arr[k].deq = arrs[0].ctypes.data
            else:
                arr[k].codes, arr[k].scales = arrs[0].ctypes.data, arrs[1].ctypes.data
            arr[k].first_bad = -1
        rc = fn(rr[0], rr[1], arr)
        assert rc == 0, "band check rejected its arguments"
        return [(a.elements, a.differ, a.ambiguous, a.violations, a.first_bad) for a in arr]

    with ThreadPoolExecutor(max_workers=threads) as ex:
        parts = list(ex.map(part, ranges))
    stats = []
    for k in range(len(prepared)):
        e = sum(p[k][0] for p in parts)
        d = sum(p[k][1] for p in parts)
        a = sum(p[k][2] for p in parts)
        v = sum(p[k][3] for p in parts)
        bad = [p[k][4] for p in parts if p[k][3] > 0]
        stats.append({"elements": e, "differ": d, "ambiguous_scale_groups": a, "violations": v,
                      "first_bad": min(bad) if bad else -1})
    return stats


def _assert(stats, names, what):
    for st, name in zip(stats, names):
        assert st["violations"] == 0, (f"{what} {name}: {st['violations']} groups outside the band, first at "
                                       f"flat element {st['first_bad']}")
        frac = st["differ"] / max(1, st["elements"])
        assert frac <= 1e-4, f"{what} {name}: {st['differ']} elements ({frac:.2e}) differ (limit 1e-4)"


def check_mx(x_bits: np.ndarray, R_bits: np.ndarray, r: int, results: list[dict], threads: int = THREADS,
             what: str = "", check: bool = True) -> list[dict]:
    """x_bits: bf16 source [M, K] (uint16); R_bits: bf16 r x r (uint16).
    results: [{'fmt': 0|1, 'deq': bf16 bits [M, K]} or {'fmt', 'codes', 'scales'}]."""
    x = np.ascontiguousarray(x_bits, dtype=np.uint16)
    R = np.ascontiguousarray(R_bits, dtype=np.uint16)
    M, K = x.shape
    prepared = _results(lambda d: int(d["fmt"]), results)
    L = lib()
    stats = _run(lambda r0, r1, arr: L.bc_mx_rows(x.ctypes.data, r0, r1, K, R.ctypes.data, r, arr, len(arr)),
                 M, prepared, threads)
    if check:
        _assert(stats, [f"fmt{d['fmt']} {'qdq' if 'deq' in d else 'quantize'}" for d in results], what)
    return stats


def check_nv(x_bits: np.ndarray, R_bits: np.ndarray, r: int, g: float, results: list[dict],
             threads: int = THREADS, what: str = "", check: bool = True) -> list[dict]:
    """As check_mx for NVFP4 results ([{'deq': ...}] or [{'codes', 'scales'}])."""
    x = np.ascontiguousarray(x_bits, dtype=np.uint16)
    R = np.ascontiguousarray(R_bits, dtype=np.uint16)
    M, K = x.shape
    prepared = _results(lambda d: 0, results)
    L = lib()
    stats = _run(lambda r0, r1, arr: L.bc_nv_rows(x.ctypes.data, r0, r1, K, R.ctypes.data, r, float(g), arr,
                                                  len(arr)), M, prepared, threads)
    if check:
        _assert(stats, ["qdq" if "deq" in d else "quantize" for d in results], what)
    return stats
