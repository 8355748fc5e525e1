"""Build libmxqdq.so for gfx950 with hipcc (in-tree, next to this file).

Each source is compiled to an object in parallel (under _build/ at the
repository root), then the objects are linked into the shared library.
Packed-fp32 VALU ops are disabled (-packed-fp32-ops): the kernels never need
them and some of their forms are avoided on this hardware.

build_ceiling() compiles the benchmark's streaming ceiling kernels
(bench_ceiling.hip at the repository root) into their own library,
bench_ceiling.so, outside libmxqdq.
"""
from __future__ import annotations

import glob
import hashlib
import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libmxqdq.so")
OBJ = os.path.join(ROOT, "_build")
CEILING_SRC = os.path.join(ROOT, "bench_ceiling.hip")
CEILING_LIB = os.path.join(ROOT, "bench_ceiling.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

CFLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-fvisibility=hidden", "-Wall",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


def sources() -> list[str]:
    return sorted(glob.glob(os.path.join(HERE, "csrc", "*.hip")))


def _compile(src: str, extra: list[str], tag: str) -> str:
    os.makedirs(OBJ, exist_ok=True)
    obj = os.path.join(OBJ, f"{tag}{os.path.splitext(os.path.basename(src))[0]}.o")
    subprocess.check_call([HIPCC, *CFLAGS, *extra, "-c", src, "-o", obj])
    return obj


def build(out: str = LIB, extra: list[str] | None = None) -> str:
    extra = list(extra or [])
    tag = "x" + hashlib.sha1(" ".join(extra).encode()).hexdigest()[:10] + "_" if extra else ""
    srcs = sources()
    with ThreadPoolExecutor(max_workers=min(len(srcs), os.cpu_count() or 1)) as ex:
        objs = list(ex.map(lambda s: _compile(s, extra, tag), srcs))
    tmp = out + ".tmp"
    subprocess.check_call([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp])
    os.replace(tmp, out)
    return out


def build_ceiling(out: str = CEILING_LIB) -> str:
    tmp = out + ".tmp"
    subprocess.check_call([HIPCC, *CFLAGS, "-shared", CEILING_SRC, "-o", tmp])
    os.replace(tmp, out)
    return out


def device_asm(out_dir: str) -> str:
    """Write the gfx950 assembly of every source (for instruction counts)."""
    os.makedirs(out_dir, exist_ok=True)
    for src in sources():
        name = os.path.splitext(os.path.basename(src))[0]
        subprocess.check_call([HIPCC, f"--offload-arch={ARCH}", "-O3", "-std=c++17",
                               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                               "-I", os.path.join(ROOT, "include"),
                               "--cuda-device-only", "-S", src,
                               "-o", os.path.join(out_dir, name + ".s")])
    return out_dir


if __name__ == "__main__":
    print(build())
    print(build_ceiling())
