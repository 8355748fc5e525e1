"""The CPU oracle and the whole-tensor comparator run clean under
AddressSanitizer and UndefinedBehaviorSanitizer: both are rebuilt with
-fsanitize=address,undefined (on the CPU, in a temporary folder), and the
oracle's pins and the comparator tests run against those builds in a child
process with the sanitizer runtimes preloaded; any report aborts the child.
The two exhaustive pins (16.7 M rounding cases, 65 536 scales) are left out
for time: they run unsanitized in the pin suite."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FLAGS = ["-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined", "-fno-sanitize-recover=all"]


def runtime(name):
    p = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True).stdout.strip()
    return p if os.path.isabs(p) and os.path.exists(p) else None


def test_oracle_and_comparator_under_asan_ubsan(tmp_path):
    asan, ubsan = runtime("libasan.so"), runtime("libubsan.so")
    if asan is None or ubsan is None:
        pytest.skip("gcc sanitizer runtimes not installed")
    orc = tmp_path / "libmxoracle_san.so"
    subprocess.check_call(["gcc", "-std=c11", "-fPIC", "-shared", "-Wall", "-Wextra", "-fno-fast-math",
                           "-ffp-contract=off", *FLAGS, "-o", str(orc), os.path.join(ROOT, "oracle", "mxoracle.c"),
                           "-lm"])
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    import _bandcheck
    bc = _bandcheck.build(str(tmp_path / "libbandcheck_san.so"), extra=FLAGS)
    env = dict(os.environ, MXORACLE_LIB=str(orc), BANDCHECK_LIB=bc, LD_PRELOAD=f"{asan}:{ubsan}",
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1", UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        "-k", "not exhaustive",
                        os.path.join(ROOT, "tests", "test_oracle_pins.py"),
                        os.path.join(ROOT, "tests", "test_band_checker.py"),
                        os.path.join(ROOT, "tests", "test_bandcheck_c.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    tail = (r.stdout[-3000:] + "\n" + r.stderr[-3000:])
    assert r.returncode == 0, tail
    assert " passed" in r.stdout and "runtime error" not in r.stderr, tail
