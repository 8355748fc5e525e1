"""The MX GEMM's slice barriers publish LDS written by loads with an LDS
destination, so every wave must have drained the loads being published
before it arrives: a wave waiting after the barrier only knows that its own
loads have landed, not the other waves'.  __syncthreads() does not imply
that wait at workgroup scope, and the compiler once left it out at one of
the two barriers per k-loop iteration; the kernels now wait explicitly.

CPU check: compile csrc/gemm.hip for gfx950 to assembly with the library's
flags and, in every k_mx_gemm instance, look at each barrier after which
LDS is read before the next barrier (a barrier that publishes), and at the
tightest vmcnt wait between it and both the previous barrier and the last
vector-memory instruction:
  - vmcnt(0): everything this wave loaded has landed;
  - vmcnt(k), k > 0: at least k vector-memory instructions were issued
    since the previous barrier, so every load issued before that barrier
    has landed (loads complete in order);
  - anything else (no wait, or k above the loads issued since the previous
    barrier) lets a wave read LDS that another wave's loads may not have
    filled yet.
Barriers with no LDS read after them only free a slot and need no wait.
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
        end = i + 1
        while "s_endpgm" not in lines[end]:
            end += 1
        barriers = [j for j in range(i, end) if re.match(r"^\s*s_barrier\b", lines[j])]
        for n, j in enumerate(barriers):
            prev = barriers[n - 1] if n else i
            nxt = barriers[n + 1] if n + 1 < len(barriers) else end
            if not any(re.match(r"^\s*ds_read", lines[q]) for q in range(j, nxt)):
                continue  # publishes nothing
            # the tightest vmcnt wait since the last vector-memory instruction
            # (and since the previous barrier)
            k, wait = j - 1, None
            while k > prev and not VMEM.match(lines[k]):
                w = re.search(r"s_waitcnt.*vmcnt\((\d+)\)", lines[k])
                if w:
                    wait = int(w.group(1)) if wait is None else min(wait, int(w.group(1)))
                k -= 1
            issued = sum(1 for q in range(prev, j) if VMEM.match(lines[q]))
            if wait is None or (wait > 0 and issued < wait):
                bad.append((m.group(1)[:50], j, f"vmcnt({wait}) with {issued} loads since the last barrier"))
        i = end
    assert kernels >= 16, kernels
    assert not bad, f"barriers that may publish loads before they land: {bad[:4]}"
