"""The MX GEMM's slice barriers publish LDS written by loads with an LDS
destination, so every wave must have drained its own vector-memory
operations (s_waitcnt vmcnt(0)) before each barrier: a wave waiting after
the barrier only knows that its own loads have landed, not the other
waves'.  __syncthreads() does not imply that wait at workgroup scope, and
the compiler once left it out at one of the two barriers per k-loop
iteration; the kernels now wait explicitly.

CPU check: compile csrc/gemm.hip for gfx950 to assembly with the library's
flags and require, in every k_mx_gemm instance, a vmcnt(0) wait between
each s_barrier and the last vector-memory instruction before it.
"""
import os
import re
import shutil
import subprocess
import tempfile

import pytest

from microscaling_quantize_dequantize_amd import build as B

VMEM = re.compile(r"^\s*(buffer_|global_|flat_|scratch_)")


def test_every_gemm_barrier_waits_for_vector_memory():
    if not shutil.which(B.HIPCC) and not os.path.exists(B.HIPCC):
        pytest.skip("hipcc not available")
    src = os.path.join(os.path.dirname(B.__file__), "csrc", "gemm.hip")
    with tempfile.TemporaryDirectory() as d:
        out = os.path.join(d, "gemm.s")
        subprocess.check_call([B.HIPCC, f"--offload-arch={B.ARCH}", "-O3", "-std=c++17",
                               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                               "-I", os.path.join(B.ROOT, "include"), "--cuda-device-only", "-S", src, "-o", out],
                              stderr=subprocess.DEVNULL)
        lines = open(out).read().split("\n")
    kernels, bad = 0, []
    i = 0
    while i < len(lines):
        m = re.match(r"^(_ZN2mx9k_mx_gemm\S+):", lines[i])
        if not m:
            i += 1
            continue
        kernels += 1
        j = i + 1
        while "s_endpgm" not in lines[j]:
            if re.match(r"^\s*s_barrier\b", lines[j]):
                k = j - 1
                while k > i and not VMEM.match(lines[k]) and not re.search(r"s_waitcnt.*vmcnt\(0\)", lines[k]):
                    k -= 1
                if not re.search(r"s_waitcnt.*vmcnt\(0\)", lines[k]):
                    bad.append((m.group(1)[:60], j))
            j += 1
        i = j
    assert kernels >= 16, kernels
    assert not bad, f"barriers without a preceding vmcnt(0): {bad[:4]}"
