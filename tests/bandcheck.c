/*
 * bandcheck.c -- the comparator of the rotated path, in C, for whole tensors.
 *
 * TEST INFRASTRUCTURE.  It is built together with the CPU oracle
 * (oracle/mxoracle.c, whose public functions it calls) into
 * tests/libbandcheck.so, and is used only by the GPU parity tests.  It is
 * not part of the method: it decides whether a GPU result of a rotated call
 * lies within the stated tolerance of the oracle.
 *
 * The tolerance ("Add QuTLASS support to vLLM", Online rotations: the
 * rotation is fused before the scale; the bar is a reading, stated with the
 * tests): a rotated value may differ from the exact one by at most
 * beta = 1e-5 * sum_t |x[t] R[t][j]|; an element of a result may differ from
 * the oracle's only where some rotated value within beta would give that
 * result, and at most 0.01% of the elements may differ.  Concretely, per
 * 32-group (MX) or 16-group (NVFP4):
 *   - the group's scale may be any scale between those of its smallest and
 *     largest possible abs-max (the scale is monotone in the abs-max);
 *   - under the scale the GPU chose, each element must lie between the
 *     result of y - beta and that of y + beta (rounding is monotone).
 * This file does the same as the numpy checkers band_check / nv_band_check
 * in tests/_parity.py (a CPU test compares the two) in one pass over the
 * rows: each row is rotated once by the oracle and every GPU result handed
 * in is checked against it.  A group whose GPU result equals the oracle's
 * exact result everywhere lies in the band by construction (the exact
 * value is between the bounds for the exact scale), so the band itself is
 * evaluated only for groups that differ.
 */
#include "mxoracle.h"

#include <math.h>
#include <stdint.h>
#include <stdlib.h>

/* One GPU result to check. kind 0: dequantized output (bf16 bits, [M x K]);
 * kind 1: codes (E2M1 packed [M x K/2], even column in bits 3:0, or E4M3
 * [M x K]) with scale bytes ([M x K/32] for MX, [M x K/16] for NVFP4).
 * Counters are accumulated (the caller zeroes them): elements checked,
 * elements that differ from the oracle, groups whose scale is ambiguous,
 * groups outside the band, and the flat index of the first such group's
 * first element (-1 when none). */
typedef struct {
    int32_t kind;
    int32_t fmt;
    const uint16_t *deq;
    const uint8_t *codes;
    const uint8_t *scales;
    int64_t elements, differ, ambiguous, violations, first_bad;
} bc_result;

/* v rounded to bf16 (nearest-even), as a double. */
static double bf16_round_value(double v)
{
    return orc_bf16_value(orc_bf16_from_double(v));
}

/* The same for an MX value (code value times 2^s: at most 4 significant
 * bits), which is returned as it is when it lies in bf16's normal range. */
static double mx_bf16_value(double v)
{
    const double a = fabs(v);
    if (a == 0.0 || (a >= 0x1p-126 && a < 0x1p127))
        return v;
    return bf16_round_value(v);
}

/* The oracle's quantize-dequantize of one value at scale exponent s. */
static double qdq_value(int fmt, double y, int s)
{
    return ldexp(orc_decode(fmt, orc_encode(fmt, y, s)), s);
}

static int code_at(int fmt, const uint8_t *codes, int64_t row, int64_t K,
                   int64_t col)
{
    if (fmt == ORC_E4M3)
        return codes[row * K + col];
    uint8_t b = codes[row * (K / 2) + col / 2];
    return (col % 2 == 0) ? (b & 0xF) : (b >> 4);
}

static void note_bad(bc_result *res, int64_t flat)
{
    if (res->violations == 0 || flat < res->first_bad)
        res->first_bad = flat;
    res->violations++;
}

/* One MX 32-group of row `row` starting at column c. */
static void mx_group(bc_result *res, const double *y, const double *b,
                     int64_t row, int64_t K, int64_t c)
{
    const int fmt = res->fmt;
    double amax = 0.0, alo = 0.0, ahi = 0.0;
    for (int j = 0; j < 32; ++j) {
        double a = fabs(y[j]);
        if (a > amax)
            amax = a;
        if (a - b[j] > alo)
            alo = a - b[j];
        if (a + b[j] > ahi)
            ahi = a + b[j];
    }
    const int s_ex = orc_scale_exponent(fmt, amax);
    const int s_lo = orc_scale_exponent(fmt, alo);
    const int s_hi = orc_scale_exponent(fmt, ahi);
    res->elements += 32;
    if (s_lo != s_hi)
        res->ambiguous++;
    const int64_t flat = row * K + c;
    if (res->kind == 0) {
        double d[32];
        int nd = 0;
        for (int j = 0; j < 32; ++j) {
            d[j] = orc_bf16_value(res->deq[flat + j]);
            if (d[j] != mx_bf16_value(qdq_value(fmt, y[j], s_ex)))
                nd++;
        }
        res->differ += nd;
        if (nd == 0)
            return;
        for (int s = s_lo; s <= s_hi; ++s) {
            int ok = 1;
            for (int j = 0; j < 32 && ok; ++j) {
                double lo = mx_bf16_value(qdq_value(fmt, y[j] - b[j], s));
                double hi = mx_bf16_value(qdq_value(fmt, y[j] + b[j], s));
                ok = (d[j] >= lo) && (d[j] <= hi);
            }
            if (ok)
                return;
        }
        note_bad(res, flat);
    } else {
        const int s_g = (int)res->scales[flat / 32] - 127;
        double v[32];
        int nd = 0;
        for (int j = 0; j < 32; ++j) {
            v[j] = ldexp(orc_decode(fmt, code_at(fmt, res->codes, row, K, c + j)), s_g);
            if (s_g != s_ex || v[j] != qdq_value(fmt, y[j], s_ex))
                nd++;
        }
        res->differ += nd;
        if (nd == 0)
            return;
        if (s_g < s_lo || s_g > s_hi) {
            note_bad(res, flat);
            return;
        }
        for (int j = 0; j < 32; ++j) {
            double lo = qdq_value(fmt, y[j] - b[j], s_g);
            double hi = qdq_value(fmt, y[j] + b[j], s_g);
            if (!(v[j] >= lo && v[j] <= hi)) {
                note_bad(res, flat);
                return;
            }
        }
    }
}

/* Rows [row0, row1) of the bf16 source x [M x K] rotated per r-chunk by R
 * (bf16, r x r, row-major; r in {16, 32, 64, 128}): check every result.
 * Returns 0, or -1 for a bad shape or an allocation failure. */
int bc_mx_rows(const uint16_t *x, int64_t row0, int64_t row1, int64_t K,
               const uint16_t *R, int r, bc_result *res, int nres)
{
    if (K <= 0 || K % 32 != 0 || r <= 0 || K % r != 0)
        return -1;
    double *y = (double *)malloc(sizeof(double) * K);
    double *b = (double *)malloc(sizeof(double) * K);
    if (!y || !b) {
        free(y);
        free(b);
        return -1;
    }
    for (int64_t i = row0; i < row1; ++i) {
        orc_rotate(x + i * K, ORC_BF16, 1, K, R, r, y, b);
        for (int k = 0; k < nres; ++k)
            for (int64_t c = 0; c < K; c += 32)
                mx_group(&res[k], y + c, b + c, i, K, c);
    }
    free(y);
    free(b);
    return 0;
}

/* ---- NVFP4 (16-groups, E4M3 scale bytes, per-tensor multiplier g) ------ */

/* The largest float <= v and the smallest float >= v. */
static float f32_down(double v)
{
    float f = (float)v;
    return ((double)f > v) ? nextafterf(f, -INFINITY) : f;
}

static float f32_up(double v)
{
    float f = (float)v;
    return ((double)f < v) ? nextafterf(f, INFINITY) : f;
}

static void nv_group(bc_result *res, float g, const double *y, const double *b,
                     int64_t row, int64_t K, int64_t c)
{
    double alo = 0.0, ahi = 0.0;
    float y32[16], amax32 = 0.0f;
    for (int j = 0; j < 16; ++j) {
        double a = fabs(y[j]);
        if (a - b[j] > alo)
            alo = a - b[j];
        if (a + b[j] > ahi)
            ahi = a + b[j];
        y32[j] = (float)y[j];
        if (fabsf(y32[j]) > amax32)
            amax32 = fabsf(y32[j]);
    }
    const int sb_lo = orc_nv_scale_byte(g, f32_down(alo));
    const int sb_hi = orc_nv_scale_byte(g, f32_up(ahi));
    const int sb_ex = orc_nv_scale_byte(g, amax32);
    res->elements += 16;
    if (sb_lo != sb_hi)
        res->ambiguous++;
    const int64_t flat = row * K + c;
    int code_ex[16];
    for (int j = 0; j < 16; ++j)
        code_ex[j] = orc_nv_code(g, sb_ex, y32[j]);
    if (res->kind == 0) {
        double d[16];
        int nd = 0;
        for (int j = 0; j < 16; ++j) {
            d[j] = orc_bf16_value(res->deq[flat + j]);
            if (d[j] != bf16_round_value((double)orc_nv_value(g, sb_ex, code_ex[j])))
                nd++;
        }
        res->differ += nd;
        if (nd == 0)
            return;
        for (int s = sb_lo; s <= sb_hi; ++s) {
            int ok = 1;
            for (int j = 0; j < 16 && ok; ++j) {
                double lo = bf16_round_value((double)orc_nv_value(g, s, orc_nv_code(g, s, f32_down(y[j] - b[j]))));
                double hi = bf16_round_value((double)orc_nv_value(g, s, orc_nv_code(g, s, f32_up(y[j] + b[j]))));
                ok = (d[j] >= lo) && (d[j] <= hi);
            }
            if (ok)
                return;
        }
        note_bad(res, flat);
    } else {
        const int sb = res->scales[flat / 16];
        int nd = 0, cg[16];
        for (int j = 0; j < 16; ++j) {
            cg[j] = code_at(ORC_E2M1, res->codes, row, K, c + j);
            if (sb != sb_ex || cg[j] != code_ex[j])
                nd++;
        }
        res->differ += nd;
        if (nd == 0)
            return;
        if (sb < sb_lo || sb > sb_hi) {
            note_bad(res, flat);
            return;
        }
        for (int j = 0; j < 16; ++j) {
            double v = orc_decode(ORC_E2M1, cg[j]);
            double lo = orc_decode(ORC_E2M1, orc_nv_code(g, sb, f32_down(y[j] - b[j])));
            double hi = orc_decode(ORC_E2M1, orc_nv_code(g, sb, f32_up(y[j] + b[j])));
            if (!(v >= lo && v <= hi)) {
                note_bad(res, flat);
                return;
            }
        }
    }
}

/* As bc_mx_rows, for NVFP4 results (fmt is ignored). */
int bc_nv_rows(const uint16_t *x, int64_t row0, int64_t row1, int64_t K,
               const uint16_t *R, int r, float g, bc_result *res, int nres)
{
    if (K <= 0 || K % 32 != 0 || r <= 0 || K % r != 0)
        return -1;
    double *y = (double *)malloc(sizeof(double) * K);
    double *b = (double *)malloc(sizeof(double) * K);
    if (!y || !b) {
        free(y);
        free(b);
        return -1;
    }
    for (int64_t i = row0; i < row1; ++i) {
        orc_rotate(x + i * K, ORC_BF16, 1, K, R, r, y, b);
        for (int k = 0; k < nres; ++k)
            for (int64_t c = 0; c < K; c += 16)
                nv_group(&res[k], g, y + c, b + c, i, K, c);
    }
    free(y);
    free(b);
    return 0;
}
