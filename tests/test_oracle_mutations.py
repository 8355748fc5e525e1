"""The pins catch plausible mistakes: each test plants one mistake in a copy
of the oracle's C source (on the CPU), builds it, and checks that the pin
suite fails against it."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "mxoracle.c")

MUTANTS = {
    "ties_away_from_zero": ("return (fmod(fl, 2.0) == 0.0) ? fl : fl + 1.0;", "return fl + 1.0;"),
    "wrong_emax_e2m1": ("{2, 1, 1, 0, 2, 6.0}", "{2, 1, 1, 0, 1, 6.0}"),
    "no_saturation": ("q = f->maxnorm; /* saturate */", "q = q;"),
    "nibbles_swapped": ("if (col % 2 == 0)\n                        *b", "if (col % 2 != 0)\n                        *b"),
    "rotation_transposed": ("x[c + t] * R[t * r + j]", "x[c + t] * R[j * r + t]"),
    "zero_sign_dropped": ("if (v == 0.0)\n        return code;", "if (v == 0.0)\n        return 0;"),
    "scale_clamp_off_by_one": ("if (s < -127)\n        s = -127;", "if (s < -126)\n        s = -126;"),
    "no_subnormal_grid": ("if (e < f->emin)\n        e = f->emin;\n    double ulp", "double ulp"),
    "bf16_subnormal_exponent": ("ldexp((double)man, -133)", "ldexp((double)man, -134)"),
    "scale_from_first_element": ("else if (fabs(y[j]) > amax)", "else if (j == 0)"),
    "blocked_lane_from_group_pair": ("int64_t lane = 32 * (g % 2) + i % 32;",
                                     "int64_t lane = 32 * ((g % 8) / 4) + i % 32;"),
    "blocked_byte_order": ("int64_t byte = (g % 8) / 2;", "int64_t byte = 3 - (g % 8) / 2;"),
    "nvfp4_c6_inverted": ("float c6 = g / 6.0f;", "float c6 = 6.0f / g;"),
    "nvfp4_scale_order": ("float q = amax * c6;", "float q = (amax * g) / 6.0f;"),
    "nvfp4_element_order": ("float v = x * m;", "float v = (sbv == 0.0f) ? 0.0f : (x * g) / sbv;"),
    "nvfp4_dequant_inverted": ("float k = sbv / g;", "float k = g / sbv;"),
    "nvfp4_amax_first_only": ("if (fabsf(x[c + j]) > amax)", "if (j == 0)"),
    "exact_dequant_scale_bias": ("dst[idx] = (b == 0xFF) ? NAN : ldexp(orc_decode(fmt, code), b - 127);",
                                 "dst[idx] = (b == 0xFF) ? NAN : ldexp(orc_decode(fmt, code), b - 128);"),
    "wrong_emax_e4m3": ("{4, 3, 7, -6, 8, 448.0}", "{4, 3, 7, -6, 7, 448.0}"),
    "e4m3_max_480": ("{4, 3, 7, -6, 8, 448.0}", "{4, 3, 7, -6, 8, 480.0}"),
    "bf16_rounded_one_bit_short": ("binary_bits(round_binary(x, 8, -126, 127), 8, 8, 127)",
                                   "binary_bits(round_binary(x, 7, -126, 127), 8, 8, 127)"),
    "f32_rounded_one_bit_short": ("binary_bits(round_binary(x, 24, -126, 127), 24, 8, 127)",
                                  "binary_bits(round_binary(x, 23, -126, 127), 24, 8, 127)"),
    "beta_without_abs": ("sabs += fabs(p);", "sabs += p;"),
    "rotation_drops_last_term": ("for (int t = 0; t < r; ++t) {\n                double p",
                                 "for (int t = 0; t < r - 1; ++t) {\n                double p"),
    "exact_dequant_sign_dropped": ("dst[idx] = (b == 0xFF) ? NAN : ldexp(orc_decode(fmt, code), b - 127);",
                                   "dst[idx] = (b == 0xFF) ? NAN : ldexp(fabs(orc_decode(fmt, code)), b - 127);"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_reject_planted_mistake(name, tmp_path):
    old, new = MUTANTS[name]
    text = open(SRC).read()
    assert text.count(old) == 1, name
    mutant = tmp_path / "mxoracle.c"
    mutant.write_text(text.replace(old, new))
    (tmp_path / "mxoracle.h").write_text(open(os.path.join(ROOT, "oracle", "mxoracle.h")).read())
    lib = tmp_path / "libmut.so"
    subprocess.check_call(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-w",
                           "-o", str(lib), str(mutant), "-lm"])
    env = dict(os.environ, MXORACLE_LIB=str(lib))
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_pins.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode != 0, f"pins did not catch mutant {name}:\n{r.stdout[-2000:]}"


# The GEMM reference's own step (the product of the two exact dequantized
# operands) is Python: the same check on a planted copy of the package.
PY_MUTANTS = {
    "matmul_b_not_transposed": ("return a @ b.T", "return a @ b"),
    "matmul_operands_swapped": ("return a @ b.T", "return b @ a.T"),
}


@pytest.mark.parametrize("name", ["unchanged"] + sorted(PY_MUTANTS))
def test_pins_reject_planted_python_mistake(name, tmp_path):
    """(The unchanged copy is the control: set up the same way, it passes.)"""
    import oracle
    old, new = PY_MUTANTS.get(name, ("return a @ b.T", "return a @ b.T"))
    text = open(os.path.join(ROOT, "oracle", "__init__.py")).read()
    assert text.count(old) == 1, name
    (tmp_path / "oracle").mkdir()
    (tmp_path / "oracle" / "__init__.py").write_text(text.replace(old, new))
    env = dict(os.environ, MXORACLE_LIB=oracle.build(force=False),
               PYTHONPATH=os.pathsep.join([str(tmp_path), ROOT]))
    # run from the planted copy's folder, so that its package is the one imported
    where = subprocess.run([sys.executable, "-c", "import oracle; print(oracle.__file__)"],
                           cwd=str(tmp_path), env=env, capture_output=True, text=True, timeout=60)
    assert where.stdout.strip().startswith(str(tmp_path)), where.stdout + where.stderr
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_pins.py")],
                       cwd=str(tmp_path), env=env, capture_output=True, text=True, timeout=600)
    if name == "unchanged":
        assert r.returncode == 0, r.stdout[-2000:]
    else:
        assert r.returncode != 0, f"pins did not catch mutant {name}:\n{r.stdout[-2000:]}"
