/*
 * mxoracle.h -- plain, slow, scalar CPU oracle for microscaling (MX)
 * quantize / dequantize.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may include, link,
 * load or call this code: only the test-suite, the smoke check and the
 * benchmark's CPU-baseline leg use it.  It shares no code, header, table or
 * constant with the HIP library.
 *
 * What it computes (all arithmetic in IEEE double; frexp/ldexp are exact):
 *   - MX block format: contiguous groups of 32 elements along the row share
 *     one scale ("use cute-dsl to speedup mxfp QDQ", Description: group size
 *     32, K divisible by 32).
 *   - The shared scale is an abs-max one ("Add QuTLASS support to vLLM",
 *     Purpose / Multiple quantization schemes: Abs-Max), stored as an E8M0
 *     byte (same page, review of vllm/_custom_ops.py: float8_e8m0fnu scales).
 *     The pages give no exponent rule; the OCP MX v1.0 rule is used:
 *     s = floor(log2(amax)) - emax_elem, emax_elem = 2 (E2M1) / 8 (E4M3),
 *     clamped to the E8M0 range [-127, 127]; an all-zero group gets -127.
 *   - Elements: v = y * 2^-s rounded to nearest, ties to even, onto the
 *     E2M1 or E4M3 grid, saturating at the largest finite magnitude.
 *   - Optional rotation before the scale ("Add QuTLASS support to vLLM",
 *     Online rotations: transform, quantization and scale computation fused,
 *     runtime-loaded matrices of size 16/32/64/128): each r-chunk x of a row
 *     becomes y = x . R, i.e. y[j] = sum_t x[t] * R[t][j], R row-major r x r.
 *   - QDQ: dequantized value code_value * 2^s, rounded to nearest-even into
 *     the source dtype (the value of the rotated data; no inverse rotation).
 *
 * Conventions the pages leave open (readings, not facts of the pages):
 *   - FP4 packing: column 2k in bits 3:0, column 2k+1 in bits 7:4.
 *   - Scales: unpadded row-major [M x K/32] bytes, value 2^(byte-127).
 *   - The sign of a result that rounds to zero is kept (code 0x8 / 0x80).
 *   - A group holding NaN or Inf: scale byte 0xFF, E4M3 codes 0x7F, E2M1
 *     codes 0x0, dequantized values NaN.  Not part of any parity bar.
 *
 * Parity pins: every function here is pinned by the CPU tests (hand-worked
 * groups, closed forms, exhaustive enumerations against a brute-force
 * nearest-grid search, round trips, invariants, library matmul for the
 * rotation).  None is "parity unpinned".
 */
#ifndef MXORACLE_H
#define MXORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element formats. */
#define ORC_E2M1 0
#define ORC_E4M3 1
/* Source / destination dtypes. */
#define ORC_BF16 0
#define ORC_F32 1

/* ---- scalar helpers (exposed so that tests can pin each step) ---------- */

/* Exact value of a bf16 / binary32 bit pattern (subnormals kept). */
double orc_bf16_value(uint16_t bits);
double orc_f32_value(uint32_t bits);

/* Round a double to nearest-even into bf16 / binary32 and return its bits. */
uint16_t orc_bf16_from_double(double x);
uint32_t orc_f32_from_double(double x);

/* Shared-scale exponent s of a group with abs-max `amax` (finite, >= 0). */
int orc_scale_exponent(int fmt, double amax);

/* Code (sign bit included) of element y under scale exponent s. */
int orc_encode(int fmt, double y, int s);

/* Element value of a code, without the scale (NaN for E4M3 0x7F/0xFF). */
double orc_decode(int fmt, int code);

/* Batch forms of the element steps, for exhaustive pins and band checks:
 * s[i]     = orc_scale_exponent(fmt, amax[i]);
 * codes[i] = orc_encode(fmt, y[i], s[i]);
 * q[i]     = orc_decode(fmt, orc_encode(fmt, y[i], s[i])) * 2^s[i]. */
void orc_scale_exponent_n(int fmt, const double *amax, int64_t n, int32_t *s);
void orc_encode_n(int fmt, const double *y, const int32_t *s, int64_t n,
                  uint8_t *codes);
void orc_qdq_value_n(int fmt, const double *y, const int32_t *s, int64_t n,
                     double *q);

/* ---- whole-matrix operations (rows [0, M) of a row-major M x K matrix) -- */

/* Rotated values y and tolerance weights beta = 1e-5 * sum_t |x[t] R[t][j]|
 * (y = x, beta = 0 when rot_size == 0).  rot is r x r in src_dtype. */
int orc_rotate(const void *src, int src_dtype, int64_t M, int64_t K,
               const void *rot, int rot_size, double *y, double *beta);

/* Fused quantize-dequantize; dst has the source dtype. */
int orc_qdq(int fmt, const void *src, int src_dtype, int64_t M, int64_t K,
            const void *rot, int rot_size, void *dst);

/* Quantize bf16 source to codes ([M x K/2] packed E2M1 or [M x K] E4M3)
 * and E8M0 scale bytes [M x K/32]. */
int orc_quantize(int fmt, const void *src, int64_t M, int64_t K,
                 const void *rot, int rot_size, uint8_t *codes,
                 uint8_t *scales);

/* Dequantize codes + scales into dst_dtype. */
int orc_dequantize(int fmt, const uint8_t *codes, const uint8_t *scales,
                   int64_t M, int64_t K, int dst_dtype, void *dst);

/* The same dequantized values kept in double, with no rounding into a
 * storage type: the exact operands of an MX GEMM (the MXFP4 GEMM test on
 * "Add QuTLASS support to vLLM" multiplies dequantized operands in high
 * precision).  Every MX value (at most 8 significant bits times a power of
 * two in [2^-127, 2^127]) is exact in double. */
int orc_dequantize_f64(int fmt, const uint8_t *codes, const uint8_t *scales,
                       int64_t M, int64_t K, double *dst);

/* Blocked scale layout (a reading: the pages name a padded, blocked scale
 * tensor -- "Add QuTLASS support to vLLM", review of vllm/_custom_ops.py
 * and vllm/qutlass_utils/utils.py: padded_rows x padded_cols, to_blocked;
 * FlashInfer cute-dsl digest page: is_sf_swizzled_layout -- but define it
 * only for another GPU's matrix cores).  Here the blocks are the operand
 * order of the gfx950 scaled MFMA with 32x32 tiles and 64-deep k-steps:
 *   rows are padded to a multiple of 32 and the K/32 groups of a row to a
 *   multiple of 8; the scales form 256-byte blocks of 32 rows x 8 groups,
 *   blocks in row-major order over (row block, group block);
 *   in a block, the 32-bit word l (l = 0..63) holds, for row l%32 of the
 *   block and h = l/32, the scales of groups h, 2+h, 4+h and 6+h of the
 *   block in bytes 0..3: the word a lane of the MFMA supplies over four
 *   consecutive k-steps.
 *   Padding bytes are 127 (the scale 2^0).
 * orc_blocked_size: bytes of the blocked tensor (-1 for a bad shape). */
int64_t orc_blocked_size(int64_t M, int64_t K);
int orc_scales_to_blocked(const uint8_t *scales, int64_t M, int64_t K,
                          uint8_t *out);

/* NVFP4 (a reading).  The pages name NVFP4 beside MXFP4 with the same fused
 * rotations and show its call shape -- fusedQuantizeNv(a, rotation,
 * global_scale), scales viewed as [-1, K/16] ("Add QuTLASS support to
 * vLLM", Purpose: NVFP4 and MXFP4; review of
 * benchmarks/kernels/bench_nvfp4_qutlass.py) -- but no rule.  Reading, the
 * published two-level NVFP4 format: groups of 16 elements along K, an E4M3
 * block scale per group, E2M1 elements, and a per-tensor fp32 multiplier g
 * (global_scale, g > 0, finite) applied before the block scale.  Because
 * floating point decides the codes, the steps are fixed as IEEE fp32
 * operations, each rounded to nearest-even:
 *   c6   = g / 6                      (per tensor)
 *   q    = amax * c6                  (amax = max |x| over the group)
 *   sb   = E4M3(q)                    (nearest-even, saturating at 448;
 *                                      the scale byte; q <= 2^-10 gives 0)
 *   m    = g / value(sb)              (0 when value(sb) = 0)
 *   code = E2M1(x * m)                (nearest-even, saturating at 6, sign
 *                                      kept)
 *   deq  = value(code) * (value(sb) / g), then nearest-even to bf16.
 * x is the bf16 source, or (with a rotation) the rotated value rounded once
 * to fp32.  Non-finite input is outside the contract. */
int orc_nv_scale_byte(float g, float amax);
int orc_nv_code(float g, int sb, float x);
float orc_nv_value(float g, int sb, int code);
void orc_nv_scale_byte_n(float g, const float *amax, int64_t n, uint8_t *sb);
void orc_nv_code_n(float g, const uint8_t *sb, const float *x, int64_t n,
                   uint8_t *codes);
void orc_nv_value_n(float g, const uint8_t *sb, const uint8_t *codes,
                    int64_t n, float *out);
/* Whole matrices: bf16 source [M x K], K % 16 == 0 (with a rotation also
 * K % r == 0 and K % 32 == 0); codes [M x K/2] (even column in bits 3:0),
 * E4M3 scale bytes [M x K/16] row-major; QDQ output bf16. */
int orc_nv_quantize(const void *src, int64_t M, int64_t K, const void *rot,
                    int rot_size, float g, uint8_t *codes, uint8_t *scales);
int orc_nv_qdq(const void *src, int64_t M, int64_t K, const void *rot,
               int rot_size, float g, uint16_t *dst);
int orc_nv_dequantize(const uint8_t *codes, const uint8_t *scales, int64_t M,
                      int64_t K, float g, int dst_dtype, void *dst);

#ifdef __cplusplus
}
#endif
#endif
