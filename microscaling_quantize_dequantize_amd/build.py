"""Build libmxqdq.so for gfx950 with hipcc (in-tree, next to this file).

Packed-fp32 VALU ops are disabled (-packed-fp32-ops): the kernels never need
them and some of their forms are avoided on this hardware.
"""
from __future__ import annotations

import glob
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libmxqdq.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-fvisibility=hidden", "-Wall",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


def sources() -> list[str]:
    return sorted(glob.glob(os.path.join(HERE, "csrc", "*.hip")))


def build(out: str = LIB, extra: list[str] | None = None) -> str:
    tmp = out + ".tmp"
    cmd = [HIPCC, *FLAGS, *(extra or []), *sources(), "-o", tmp]
    subprocess.check_call(cmd)
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
