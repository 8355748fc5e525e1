"""VALU co-limit of the unrotated step kernels, counted in their own ISA.

At 80% of 8 TB/s the GPU's vector lanes (256 CUs x 64 lanes x 2.4 GHz =
39.3 T lane-operations/s) allow per element about 24.6 operations for QDQ
(4 bytes per element), 15.5 for MXFP4 quantize (2.53125) and 18.6 for
MXFP8 quantize (3.03125).  CPU check: compile csrc/unrot.hip for gfx950 to
assembly with the library's flags and count the VALU instructions of each
step kernel's whole body (prologue and both the full and the partial
paths, so an upper bound on what one pass executes), divided by the
elements a lane takes per pass (8 per piece, one piece for QDQ and two for
quantize).  The bound keeps the kernels memory-bound by a wide margin.
"""
import os
import re
import shutil
import subprocess
import tempfile

import pytest

from microscaling_quantize_dequantize_amd import build as B

LANE_OPS = 256 * 64 * 2.4e9
RATE = 0.8 * 8e12  # bytes per second at 80% of 8 TB/s
BYTES = {(0, 0): 4.0, (1, 0): 4.0, (0, 1): 2.53125, (1, 1): 3.03125}  # (fmt, op) -> bytes per element


def test_unrotated_step_kernels_within_valu_budget():
    if not shutil.which(B.HIPCC) and not os.path.exists(B.HIPCC):
        pytest.skip("hipcc not available")
    src = os.path.join(os.path.dirname(B.__file__), "csrc", "unrot.hip")
    with tempfile.TemporaryDirectory() as d:
        out = os.path.join(d, "unrot.s")
        subprocess.check_call([B.HIPCC, f"--offload-arch={B.ARCH}", "-O3", "-std=c++17",
                               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                               "-I", os.path.join(B.ROOT, "include"), "--cuda-device-only", "-S", src, "-o", out],
                              stderr=subprocess.DEVNULL)
        lines = open(out).read().split("\n")
    seen = {}
    i = 0
    while i < len(lines):
        # k_unrot_bf16<FMT, OP, THREADS, UNROLL, SL>
        m = re.match(r"^_ZN2mx12k_unrot_bf16ILi(\d)ELi(\d)ELi(\d+)ELi(\d)ELi(\d)EEE\S*:", lines[i])
        if not m:
            i += 1
            continue
        end = i + 1
        while "s_endpgm" not in lines[end]:
            end += 1
        fmt, op, unroll, sl = int(m.group(1)), int(m.group(2)), int(m.group(4)), int(m.group(5))
        if sl == 0:
            valu = [ln for ln in lines[i:end] if re.match(r"^\s+v_", ln) and not re.match(r"^\s+v_mfma", ln)]
            per_element = len(valu) / (8 * unroll)
            budget = LANE_OPS / (RATE / BYTES[(fmt, op)])
            seen[(fmt, op)] = (per_element, budget)
        i = end
    assert set(seen) == set(BYTES), f"step kernels found: {sorted(seen)}"
    for key, (per_element, budget) in seen.items():
        assert per_element < 0.5 * budget, f"fmt {key[0]} op {key[1]}: {per_element:.1f} VALU per element, budget {budget:.1f}"
