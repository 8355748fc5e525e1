/*
 * mxoracle.c -- plain, slow, scalar CPU oracle for MX quantize / dequantize.
 *
 * TEST INFRASTRUCTURE ONLY (tests, the smoke check and the benchmark's CPU
 * baseline).  It shares no code with the HIP library.  Every step follows
 * the definitions stated in mxoracle.h, in IEEE double, one element at a
 * time, with no blocking, fusion or reordering.
 */
#include "mxoracle.h"

#include <math.h>
#include <stdlib.h>

/* Element format parameters (OCP MX v1.0 element types; the pages name
 * MXFP4 = E2M1 and MXFP8 = E4M3: "use cute-dsl to speedup mxfp QDQ",
 * Description; "Add QuTLASS support to vLLM", review of the MXFP4 test). */
typedef struct {
    int ebits;      /* exponent field width                         */
    int mbits;      /* mantissa field width                         */
    int bias;       /* exponent bias                                */
    int emin;       /* exponent of the smallest normal (1 - bias)   */
    int emax_elem;  /* exponent of the largest normal               */
    double maxnorm; /* largest finite magnitude                     */
} fmt_t;

static const fmt_t FMTS[2] = {
    {2, 1, 1, 0, 2, 6.0},    /* E2M1: 0 .5 1 1.5 2 3 4 6           */
    {4, 3, 7, -6, 8, 448.0}, /* E4M3: max 0x7E = 448, 0x7F is NaN   */
};

/* Round a non-negative double to the nearest integer, ties to even. */
static double rne_int(double n)
{
    double fl = floor(n);
    double d = n - fl; /* exact: n < 2^53 here */
    if (d > 0.5)
        return fl + 1.0;
    if (d < 0.5)
        return fl;
    return (fmod(fl, 2.0) == 0.0) ? fl : fl + 1.0;
}

/* floor(log2(a)) for finite a > 0, via the exact frexp decomposition. */
static int floor_log2(double a)
{
    int ex;
    frexp(a, &ex); /* a = f * 2^ex, f in [0.5, 1) */
    return ex - 1;
}

/* ---- IEEE binary formats used for the source / destination ----------- */

double orc_bf16_value(uint16_t bits)
{
    int sign = bits >> 15;
    int ex = (bits >> 7) & 0xFF;
    int man = bits & 0x7F;
    double v;
    if (ex == 0xFF)
        v = man ? NAN : INFINITY;
    else if (ex == 0)
        v = ldexp((double)man, -133); /* subnormal: man * 2^(-126-7) */
    else
        v = ldexp((double)(128 + man), ex - 127 - 7);
    return sign ? -v : v;
}

double orc_f32_value(uint32_t bits)
{
    int sign = bits >> 31;
    int ex = (bits >> 23) & 0xFF;
    uint32_t man = bits & 0x7FFFFFu;
    double v;
    if (ex == 0xFF)
        v = man ? NAN : INFINITY;
    else if (ex == 0)
        v = ldexp((double)man, -149);
    else
        v = ldexp((double)(0x800000u + man), ex - 127 - 23);
    return sign ? -v : v;
}

/* Round x to nearest-even into a binary format with p significant bits and
 * normal exponent range [emin, emax]; overflow gives +-inf. */
static double round_binary(double x, int p, int emin, int emax)
{
    if (x == 0.0 || isnan(x) || isinf(x))
        return x;
    double a = fabs(x);
    int e = floor_log2(a);
    if (e < emin)
        e = emin; /* subnormal range: fixed quantum */
    double quantum = ldexp(1.0, e - (p - 1));
    double r = rne_int(a / quantum) * quantum;
    if (r >= ldexp(1.0, emax + 1))
        r = INFINITY;
    return copysign(r, x);
}

/* Bits of an already-representable value in a binary format with p
 * significant bits, exponent field width w and bias. */
static uint32_t binary_bits(double r, int p, int w, int bias)
{
    uint32_t sign = signbit(r) ? 1u : 0u;
    uint32_t out = sign << (p - 1 + w);
    double a = fabs(r);
    int emin = 1 - bias;
    if (isinf(a))
        return out | (((1u << w) - 1u) << (p - 1));
    if (a == 0.0)
        return out;
    int e = floor_log2(a);
    if (e < emin) /* subnormal: exponent field 0 */
        return out | (uint32_t)(a / ldexp(1.0, emin - (p - 1)));
    uint32_t man = (uint32_t)(a / ldexp(1.0, e - (p - 1))) - (1u << (p - 1));
    return out | ((uint32_t)(e + bias) << (p - 1)) | man;
}

uint16_t orc_bf16_from_double(double x)
{
    if (isnan(x))
        return 0x7FC0;
    return (uint16_t)binary_bits(round_binary(x, 8, -126, 127), 8, 8, 127);
}

uint32_t orc_f32_from_double(double x)
{
    if (isnan(x))
        return 0x7FC00000u;
    return binary_bits(round_binary(x, 24, -126, 127), 24, 8, 127);
}

/* ---- MX element steps ------------------------------------------------ */

int orc_scale_exponent(int fmt, double amax)
{
    const fmt_t *f = &FMTS[fmt];
    if (amax == 0.0)
        return -127;
    int s = floor_log2(amax) - f->emax_elem;
    if (s < -127)
        s = -127;
    if (s > 127)
        s = 127;
    return s;
}

static int nan_code(int fmt)
{
    return fmt == ORC_E4M3 ? 0x7F : 0x0;
}

int orc_encode(int fmt, double y, int s)
{
    const fmt_t *f = &FMTS[fmt];
    if (isnan(y) || isinf(y))
        return nan_code(fmt);
    int sign = signbit(y) ? 1 : 0;
    int code = sign << (f->ebits + f->mbits);
    double v = ldexp(fabs(y), -s); /* exact power-of-two scaling */
    if (v == 0.0)
        return code;

    /* Round to the element grid: the quantum at v's binade (or at the
     * smallest normal binade for subnormals) is 2^(e - mbits). */
    int e = floor_log2(v);
    if (e < f->emin)
        e = f->emin;
    double ulp = ldexp(1.0, e - f->mbits);
    double q = rne_int(v / ulp) * ulp;
    if (q > f->maxnorm)
        q = f->maxnorm; /* saturate */
    if (q == 0.0)
        return code;

    /* Encode the grid value q into exponent and mantissa fields. */
    int eq = floor_log2(q);
    int efield, man;
    if (eq < f->emin) {
        efield = 0;
        man = (int)(q / ldexp(1.0, f->emin - f->mbits));
    } else {
        efield = eq + f->bias;
        man = (int)(q / ldexp(1.0, eq - f->mbits)) - (1 << f->mbits);
    }
    return code | (efield << f->mbits) | man;
}

double orc_decode(int fmt, int code)
{
    const fmt_t *f = &FMTS[fmt];
    int sign = (code >> (f->ebits + f->mbits)) & 1;
    int efield = (code >> f->mbits) & ((1 << f->ebits) - 1);
    int man = code & ((1 << f->mbits) - 1);
    if (fmt == ORC_E4M3 && efield == 15 && man == 7)
        return NAN;
    double v;
    if (efield == 0)
        v = ldexp((double)man, f->emin - f->mbits);
    else
        v = ldexp((double)((1 << f->mbits) + man), efield - f->bias - f->mbits);
    return sign ? -v : v;
}

void orc_scale_exponent_n(int fmt, const double *amax, int64_t n, int32_t *s)
{
    for (int64_t i = 0; i < n; ++i)
        s[i] = orc_scale_exponent(fmt, amax[i]);
}

void orc_encode_n(int fmt, const double *y, const int32_t *s, int64_t n,
                  uint8_t *codes)
{
    for (int64_t i = 0; i < n; ++i)
        codes[i] = (uint8_t)orc_encode(fmt, y[i], s[i]);
}

void orc_qdq_value_n(int fmt, const double *y, const int32_t *s, int64_t n,
                     double *q)
{
    for (int64_t i = 0; i < n; ++i)
        q[i] = ldexp(orc_decode(fmt, orc_encode(fmt, y[i], s[i])), s[i]);
}

/* ---- whole-matrix operations ----------------------------------------- */

static int valid_fmt(int fmt) { return fmt == ORC_E2M1 || fmt == ORC_E4M3; }
static int valid_dtype(int d) { return d == ORC_BF16 || d == ORC_F32; }

static int valid_shape(int64_t M, int64_t K, int rot_size, const void *rot)
{
    if (M < 0 || K < 0 || K % 32 != 0)
        return 0;
    if (rot_size == 0)
        return 1;
    if (rot_size != 16 && rot_size != 32 && rot_size != 64 && rot_size != 128)
        return 0;
    return rot != NULL && K % rot_size == 0;
}

static double src_value(const void *src, int dtype, int64_t idx)
{
    if (dtype == ORC_BF16)
        return orc_bf16_value(((const uint16_t *)src)[idx]);
    return orc_f32_value(((const uint32_t *)src)[idx]);
}

/* One row: x -> y (rotated per r-chunk, or copied) and beta. */
static void rotate_row(const void *src, int dtype, int64_t row, int64_t K,
                       const double *R, int r, double *x, double *y,
                       double *beta)
{
    for (int64_t k = 0; k < K; ++k)
        x[k] = src_value(src, dtype, row * K + k);
    if (r == 0) {
        for (int64_t k = 0; k < K; ++k) {
            y[k] = x[k];
            beta[k] = 0.0;
        }
        return;
    }
    for (int64_t c = 0; c < K; c += r) {
        for (int j = 0; j < r; ++j) {
            double sum = 0.0, sabs = 0.0;
            for (int t = 0; t < r; ++t) {
                double p = x[c + t] * R[t * r + j];
                sum += p;
                sabs += fabs(p);
            }
            y[c + j] = sum;
            beta[c + j] = 1e-5 * sabs;
        }
    }
}

static double *load_rot(const void *rot, int dtype, int r)
{
    if (r == 0)
        return NULL;
    double *R = (double *)malloc(sizeof(double) * r * r);
    for (int i = 0; i < r * r; ++i)
        R[i] = src_value(rot, dtype, i);
    return R;
}

int orc_rotate(const void *src, int src_dtype, int64_t M, int64_t K,
               const void *rot, int rot_size, double *y, double *beta)
{
    if (!valid_dtype(src_dtype) || !valid_shape(M, K, rot_size, rot))
        return -1;
    double *R = load_rot(rot, src_dtype, rot_size);
    double *x = (double *)malloc(sizeof(double) * (K ? K : 1));
    for (int64_t i = 0; i < M; ++i)
        rotate_row(src, src_dtype, i, K, R, rot_size, x, y + i * K,
                   beta + i * K);
    free(x);
    free(R);
    return 0;
}

/* One 32-group: scale byte, codes and dequantized values. */
static void group_step(int fmt, const double *y, uint8_t *scale_byte,
                       int *codes, double *deq)
{
    double amax = 0.0;
    int finite = 1;
    for (int j = 0; j < 32; ++j) {
        if (isnan(y[j]) || isinf(y[j]))
            finite = 0;
        else if (fabs(y[j]) > amax)
            amax = fabs(y[j]);
    }
    if (!finite) {
        *scale_byte = 0xFF;
        for (int j = 0; j < 32; ++j) {
            codes[j] = nan_code(fmt);
            deq[j] = NAN;
        }
        return;
    }
    int s = orc_scale_exponent(fmt, amax);
    *scale_byte = (uint8_t)(s + 127);
    for (int j = 0; j < 32; ++j) {
        codes[j] = orc_encode(fmt, y[j], s);
        deq[j] = ldexp(orc_decode(fmt, codes[j]), s);
    }
}

static void store_dst(void *dst, int dtype, int64_t idx, double v)
{
    if (dtype == ORC_BF16)
        ((uint16_t *)dst)[idx] = orc_bf16_from_double(v);
    else
        ((uint32_t *)dst)[idx] = orc_f32_from_double(v);
}

int orc_qdq(int fmt, const void *src, int src_dtype, int64_t M, int64_t K,
            const void *rot, int rot_size, void *dst)
{
    if (!valid_fmt(fmt) || !valid_dtype(src_dtype) ||
        !valid_shape(M, K, rot_size, rot))
        return -1;
    double *R = load_rot(rot, src_dtype, rot_size);
    size_t kk = (size_t)(K ? K : 1);
    double *x = (double *)malloc(sizeof(double) * kk);
    double *y = (double *)malloc(sizeof(double) * kk);
    double *beta = (double *)malloc(sizeof(double) * kk);
    int codes[32];
    double deq[32];
    uint8_t sb;
    for (int64_t i = 0; i < M; ++i) {
        rotate_row(src, src_dtype, i, K, R, rot_size, x, y, beta);
        for (int64_t g = 0; g < K; g += 32) {
            group_step(fmt, y + g, &sb, codes, deq);
            for (int j = 0; j < 32; ++j)
                store_dst(dst, src_dtype, i * K + g + j, deq[j]);
        }
    }
    free(x);
    free(y);
    free(beta);
    free(R);
    return 0;
}

int orc_quantize(int fmt, const void *src, int64_t M, int64_t K,
                 const void *rot, int rot_size, uint8_t *codes,
                 uint8_t *scales)
{
    if (!valid_fmt(fmt) || !valid_shape(M, K, rot_size, rot))
        return -1;
    double *R = load_rot(rot, ORC_BF16, rot_size);
    size_t kk = (size_t)(K ? K : 1);
    double *x = (double *)malloc(sizeof(double) * kk);
    double *y = (double *)malloc(sizeof(double) * kk);
    double *beta = (double *)malloc(sizeof(double) * kk);
    int gc[32];
    double deq[32];
    for (int64_t i = 0; i < M; ++i) {
        rotate_row(src, ORC_BF16, i, K, R, rot_size, x, y, beta);
        for (int64_t g = 0; g < K; g += 32) {
            group_step(fmt, y + g, &scales[(i * K + g) / 32], gc, deq);
            for (int j = 0; j < 32; ++j) {
                int64_t col = g + j;
                if (fmt == ORC_E4M3) {
                    codes[i * K + col] = (uint8_t)gc[j];
                } else {
                    /* column 2k -> bits 3:0, column 2k+1 -> bits 7:4 */
                    uint8_t *b = &codes[(i * K + col) / 2];
                    if (col % 2 == 0)
                        *b = (uint8_t)(gc[j] & 0xF);
                    else
                        *b = (uint8_t)(*b | ((gc[j] & 0xF) << 4));
                }
            }
        }
    }
    free(x);
    free(y);
    free(beta);
    free(R);
    return 0;
}

int orc_dequantize(int fmt, const uint8_t *codes, const uint8_t *scales,
                   int64_t M, int64_t K, int dst_dtype, void *dst)
{
    if (!valid_fmt(fmt) || !valid_dtype(dst_dtype) ||
        !valid_shape(M, K, 0, NULL))
        return -1;
    for (int64_t i = 0; i < M; ++i) {
        for (int64_t col = 0; col < K; ++col) {
            int64_t idx = i * K + col;
            int b = scales[idx / 32];
            int code;
            if (fmt == ORC_E4M3)
                code = codes[idx];
            else
                code = (col % 2 == 0) ? (codes[idx / 2] & 0xF)
                                      : (codes[idx / 2] >> 4);
            double v = (b == 0xFF) ? NAN : ldexp(orc_decode(fmt, code), b - 127);
            store_dst(dst, dst_dtype, idx, v);
        }
    }
    return 0;
}

int orc_dequantize_f64(int fmt, const uint8_t *codes, const uint8_t *scales,
                       int64_t M, int64_t K, double *dst)
{
    if (!valid_fmt(fmt) || !valid_shape(M, K, 0, NULL))
        return -1;
    for (int64_t i = 0; i < M; ++i) {
        for (int64_t col = 0; col < K; ++col) {
            int64_t idx = i * K + col;
            int b = scales[idx / 32];
            int code;
            if (fmt == ORC_E4M3)
                code = codes[idx];
            else
                code = (col % 2 == 0) ? (codes[idx / 2] & 0xF)
                                      : (codes[idx / 2] >> 4);
            dst[idx] = (b == 0xFF) ? NAN : ldexp(orc_decode(fmt, code), b - 127);
        }
    }
    return 0;
}

int64_t orc_blocked_size(int64_t M, int64_t K)
{
    if (M < 0 || K < 0 || K % 32 != 0)
        return -1;
    int64_t row_blocks = (M + 31) / 32;
    int64_t group_blocks = (K / 32 + 7) / 8;
    return row_blocks * group_blocks * 256;
}

int orc_scales_to_blocked(const uint8_t *scales, int64_t M, int64_t K,
                          uint8_t *out)
{
    int64_t size = orc_blocked_size(M, K);
    if (size < 0)
        return -1;
    int64_t G = K / 32;
    int64_t group_blocks = (G + 7) / 8;
    for (int64_t b = 0; b < size; ++b)
        out[b] = 127; /* padding: the scale 2^0 */
    for (int64_t i = 0; i < M; ++i) {
        for (int64_t g = 0; g < G; ++g) {
            int64_t block = (i / 32) * group_blocks + g / 8;
            int64_t lane = 32 * (g % 2) + i % 32;
            int64_t byte = (g % 8) / 2;
            out[block * 256 + 4 * lane + byte] = scales[i * G + g];
        }
    }
    return 0;
}

/* ---- NVFP4 (a reading; the steps are listed in mxoracle.h) ------------- */

int orc_nv_scale_byte(float g, float amax)
{
    float c6 = g / 6.0f;
    float q = amax * c6;
    return orc_encode(ORC_E4M3, (double)q, 0); /* q >= 0; saturates at 448 */
}

int orc_nv_code(float g, int sb, float x)
{
    float sbv = (float)orc_decode(ORC_E4M3, sb);
    float m = (sbv == 0.0f) ? 0.0f : g / sbv;
    float v = x * m;
    return orc_encode(ORC_E2M1, (double)v, 0);
}

float orc_nv_value(float g, int sb, int code)
{
    float sbv = (float)orc_decode(ORC_E4M3, sb);
    float k = sbv / g;
    float cv = (float)orc_decode(ORC_E2M1, code);
    return cv * k;
}

void orc_nv_scale_byte_n(float g, const float *amax, int64_t n, uint8_t *sb)
{
    for (int64_t i = 0; i < n; ++i)
        sb[i] = (uint8_t)orc_nv_scale_byte(g, amax[i]);
}

void orc_nv_code_n(float g, const uint8_t *sb, const float *x, int64_t n,
                   uint8_t *codes)
{
    for (int64_t i = 0; i < n; ++i)
        codes[i] = (uint8_t)orc_nv_code(g, sb[i], x[i]);
}

void orc_nv_value_n(float g, const uint8_t *sb, const uint8_t *codes,
                    int64_t n, float *out)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = orc_nv_value(g, sb[i], codes[i]);
}

static int nv_valid_shape(int64_t M, int64_t K, int rot_size, const void *rot)
{
    if (M < 0 || K < 0 || K % 16 != 0)
        return 0;
    if (rot_size == 0)
        return 1;
    if (rot_size != 16 && rot_size != 32 && rot_size != 64 && rot_size != 128)
        return 0;
    return rot != NULL && K % rot_size == 0 && K % 32 == 0;
}

/* One row of NVFP4: codes (one per element) and scale bytes (one per
 * 16-group) of the fp32 values x (the source, or its rotation rounded once
 * to fp32). */
static void nv_row(float g, const float *x, int64_t K, int *codes,
                   uint8_t *scales)
{
    for (int64_t c = 0; c < K; c += 16) {
        float amax = 0.0f;
        for (int j = 0; j < 16; ++j)
            if (fabsf(x[c + j]) > amax)
                amax = fabsf(x[c + j]);
        int sb = orc_nv_scale_byte(g, amax);
        scales[c / 16] = (uint8_t)sb;
        for (int j = 0; j < 16; ++j)
            codes[c + j] = orc_nv_code(g, sb, x[c + j]);
    }
}

static void nv_row_values(const void *src, int64_t i, int64_t K,
                          const double *R, int r, double *x, double *y,
                          double *beta, float *xf)
{
    rotate_row(src, ORC_BF16, i, K, R, r, x, y, beta);
    for (int64_t k = 0; k < K; ++k)
        xf[k] = (float)y[k]; /* exact without rotation; one rounding with */
}

int orc_nv_quantize(const void *src, int64_t M, int64_t K, const void *rot,
                    int rot_size, float g, uint8_t *codes, uint8_t *scales)
{
    if (!nv_valid_shape(M, K, rot_size, rot))
        return -1;
    double *R = load_rot(rot, ORC_BF16, rot_size);
    size_t kk = (size_t)(K ? K : 1);
    double *x = (double *)malloc(sizeof(double) * kk);
    double *y = (double *)malloc(sizeof(double) * kk);
    double *beta = (double *)malloc(sizeof(double) * kk);
    float *xf = (float *)malloc(sizeof(float) * kk);
    int *rc = (int *)malloc(sizeof(int) * kk);
    for (int64_t i = 0; i < M; ++i) {
        nv_row_values(src, i, K, R, rot_size, x, y, beta, xf);
        nv_row(g, xf, K, rc, scales + i * (K / 16));
        for (int64_t col = 0; col < K; col += 2)
            codes[(i * K + col) / 2] =
                (uint8_t)((rc[col] & 0xF) | ((rc[col + 1] & 0xF) << 4));
    }
    free(x);
    free(y);
    free(beta);
    free(xf);
    free(rc);
    free(R);
    return 0;
}

int orc_nv_qdq(const void *src, int64_t M, int64_t K, const void *rot,
               int rot_size, float g, uint16_t *dst)
{
    if (!nv_valid_shape(M, K, rot_size, rot))
        return -1;
    double *R = load_rot(rot, ORC_BF16, rot_size);
    size_t kk = (size_t)(K ? K : 1);
    double *x = (double *)malloc(sizeof(double) * kk);
    double *y = (double *)malloc(sizeof(double) * kk);
    double *beta = (double *)malloc(sizeof(double) * kk);
    float *xf = (float *)malloc(sizeof(float) * kk);
    int *rc = (int *)malloc(sizeof(int) * kk);
    uint8_t *sc = (uint8_t *)malloc(kk / 16 + 1);
    for (int64_t i = 0; i < M; ++i) {
        nv_row_values(src, i, K, R, rot_size, x, y, beta, xf);
        nv_row(g, xf, K, rc, sc);
        for (int64_t col = 0; col < K; ++col)
            dst[i * K + col] = orc_bf16_from_double(
                (double)orc_nv_value(g, sc[col / 16], rc[col]));
    }
    free(x);
    free(y);
    free(beta);
    free(xf);
    free(rc);
    free(sc);
    free(R);
    return 0;
}

int orc_nv_dequantize(const uint8_t *codes, const uint8_t *scales, int64_t M,
                      int64_t K, float g, int dst_dtype, void *dst)
{
    if (!valid_dtype(dst_dtype) || !nv_valid_shape(M, K, 0, NULL))
        return -1;
    for (int64_t i = 0; i < M; ++i) {
        for (int64_t col = 0; col < K; ++col) {
            int64_t idx = i * K + col;
            int code = (col % 2 == 0) ? (codes[idx / 2] & 0xF)
                                      : (codes[idx / 2] >> 4);
            float v = orc_nv_value(g, scales[idx / 16], code);
            store_dst(dst, dst_dtype, idx, (double)v);
        }
    }
    return 0;
}
