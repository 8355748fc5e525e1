/*
 * libmxqdq -- microscaling (MX) quantize / dequantize on AMD Instinct MI355X
 * (gfx950, CDNA4).  C ABI: plain pointers and sizes, no framework types.
 *
 * The operation (what each call computes):
 *   - A row-major [M x K] matrix is split along each row into contiguous
 *     groups of 32 elements; K must be a multiple of 32 ("use cute-dsl to
 *     speedup mxfp QDQ", Description: group size 32, K divisible by 32,
 *     contiguous input).
 *   - Each group gets one shared power-of-two scale from its abs-max
 *     ("[Transform] [Quantization] Add QuTLASS support to vLLM", Purpose:
 *     Abs-Max scheme), stored as an E8M0 byte b meaning 2^(b-127) (same page,
 *     review of vllm/_custom_ops.py: float8_e8m0fnu scale tensor).  Exponent
 *     rule (OCP MX v1.0; the pages do not print one): s = floor(log2 amax)
 *     - emax_elem, emax_elem = 2 for E2M1 and 8 for E4M3, clamped to
 *     [-127, 127]; an all-zero group gets s = -127 (byte 0).
 *   - Each element y becomes y * 2^-s rounded to nearest, ties to even, onto
 *     the FP4 E2M1 (MXFP4) or FP8 E4M3 (MXFP8) grid, saturating at 6 / 448.
 *     The sign of a result that rounds to zero is kept.
 *   - Optional rotation before the scale ("Add QuTLASS support to vLLM",
 *     Online rotations: transform + quantization + scale computation fused,
 *     matrix loaded at runtime, sizes 16/32/64/128): every r-element chunk x
 *     of a row (chunks start at column 0) is replaced by y = x . R, i.e.
 *     y[j] = sum_t x[t] * R[t][j], with R an r x r row-major matrix in the
 *     source dtype, accumulated in fp32.  bf16 sources multiply exactly (bf16
 *     matrix cores); fp32 sources run on the fp32 matrix cores, whose
 *     products are rounded once to fp32.  For a symmetric
 *     matrix such as the normalised Hadamard H * r^-0.5 the side does not
 *     matter.  QDQ then returns the dequantized rotated values (no inverse).
 *
 * Layouts:
 *   src, dst     [M x K] row-major, contiguous, 16-byte aligned.
 *   codes        E2M1: [M x K/2] bytes, column 2k in bits 3:0 and column
 *                2k+1 in bits 7:4; E4M3: [M x K] bytes.  16-byte aligned.
 *   scales       [M x K/32] bytes, row-major, unpadded (the non-swizzled
 *                [M, K/32] layout of the MXFP8 quantize on the FlashInfer
 *                cute-dsl digest page, key source excerpt).  4-byte aligned.
 *   rot          [r x r] row-major in the source dtype, 16-byte aligned.
 *
 * Ownership and execution: every pointer is device memory owned by the
 * caller.  The library allocates nothing, frees nothing and never
 * synchronizes; every call validates its arguments on the host, enqueues one
 * kernel on the calling thread's stream (mx_set_stream) and returns.  Calls
 * are therefore safe to capture in a HIP graph.  dst == src (an exact alias)
 * is allowed for mx_qdq; any other overlap between inputs and outputs is
 * undefined.  Faults inside a kernel surface at the caller's next
 * synchronization, as for any HIP kernel.
 *
 * Errors: 0 on success, a negative MX_E* code otherwise; argument errors are
 * returned before anything is enqueued.  M == 0 or K == 0 is a successful
 * no-op.  There is no fallback path: unsupported arguments are errors.
 *
 * Non-finite input (outside every accuracy contract): a group holding NaN or
 * Inf gets scale byte 0xFF, E4M3 codes 0x7F (E2M1 codes 0x0), and
 * dequantized values NaN.  With a rotation the group is the rotated one, and
 * a NaN or Inf input reaches every output of the block the kernel rotates it
 * in (products with Inf and sums of opposite infinities give NaN, and so do
 * the zeros of a block-diagonal matrix): bf16 sources rotate blocks of
 * max(r, 64) elements when M*K is a multiple of 64 (for blocked scales:
 * when K is) and max(r, 32) otherwise, fp32 sources blocks of max(r, 32);
 * each group of such a block is non-finite.
 */
#ifndef LIBMXQDQ_H
#define LIBMXQDQ_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MX_API __attribute__((visibility("default")))

/* Element formats. */
#define MX_FMT_E2M1 0 /* MXFP4 */
#define MX_FMT_E4M3 1 /* MXFP8 */

/* Source / destination dtypes. */
#define MX_DTYPE_BF16 0
#define MX_DTYPE_F32 1

/* Status codes. */
#define MX_OK 0
#define MX_EFMT (-1)    /* fmt is not MX_FMT_E2M1 / MX_FMT_E4M3            */
#define MX_EDTYPE (-2)  /* dtype is not MX_DTYPE_BF16 / MX_DTYPE_F32        */
#define MX_ESHAPE (-3)  /* M < 0, K < 0, K % 32 != 0 (NVFP4: K % 16), or
                           M*K too large                                    */
#define MX_EROT (-4)    /* rot_size not in {0,16,32,64,128}, K % rot_size,
                           rot == NULL with rot_size > 0, or (NVFP4)
                           a rotation with K % 32 != 0                       */
#define MX_ENULL (-5)   /* a required pointer is NULL                       */
#define MX_EALIGN (-6)  /* a pointer breaks the alignment stated above      */
#define MX_ELAUNCH (-7) /* the kernel launch failed (hipGetLastError)       */
#define MX_ELAYOUT (-8) /* scale_layout is not one of MX_SCALES_*           */

/* Scale layouts. */
#define MX_SCALES_ROWMAJOR 0 /* [M x K/32] bytes, row-major, unpadded      */
#define MX_SCALES_BLOCKED 1  /* the blocked layout described below         */

/*
 * Fused quantize-dequantize ("use cute-dsl to speedup mxfp QDQ",
 * Description: mxfp4_qdq / mxfp8_qdq).
 *   fmt        MX_FMT_E2M1 or MX_FMT_E4M3.
 *   src        [M x K] in src_dtype (MX_DTYPE_BF16 or MX_DTYPE_F32).
 *   rot        NULL, or the r x r rotation in src_dtype; rot_size = r or 0.
 *   dst        [M x K] in src_dtype: code_value * 2^s, rounded to
 *              nearest-even into src_dtype (exact whenever representable).
 */
MX_API int mx_qdq(int fmt, const void *src, int src_dtype, int64_t M,
                  int64_t K, const void *rot, int rot_size, void *dst);

/*
 * Quantize a bf16 matrix to MX codes and E8M0 scales ("Add QuTLASS support
 * to vLLM", review of vllm/_custom_ops.py: fusedQuantizeMx returning the
 * E2M1 codes and E8M0 scales; FlashInfer cute-dsl digest page, key source
 * excerpt: MXFP8 quantize returning (x_q, x_scales)).
 *   src        [M x K] bf16.
 *   rot        NULL, or the r x r bf16 rotation; rot_size = r or 0.
 *   codes      [M x K/2] (E2M1, packed) or [M x K] (E4M3) bytes.
 *   scales     [M x K/32] E8M0 bytes.
 */
MX_API int mx_quantize(int fmt, const void *src, int64_t M, int64_t K,
                       const void *rot, int rot_size, uint8_t *codes,
                       uint8_t *scales);

/*
 * Dequantize codes + scales (the inverse used by the MXFP4 GEMM test on
 * "Add QuTLASS support to vLLM", review of the test file: a_dq / b_dq built
 * by a dequantize helper).  dst[i][k] = code_value * 2^(scale-127) rounded
 * to nearest-even into dst_dtype; a scale byte of 0xFF or an E4M3 NaN code
 * gives NaN.
 */
MX_API int mx_dequantize(int fmt, const uint8_t *codes, const uint8_t *scales,
                         int64_t M, int64_t K, int dst_dtype, void *dst);

/*
 * The rotation step alone: dst[M x K] (fp32) = per-chunk x . R with fp32
 * accumulation, exactly as the fused calls compute it before the scale.
 * Exposed so that the rotation's accuracy can be checked directly.
 */
MX_API int mx_rotate(const void *src, int src_dtype, int64_t M, int64_t K,
                     const void *rot, int rot_size, float *dst);

/*
 * Blocked scale layout: the E8M0 scales in the order the gfx950 scaled
 * matrix cores read them (32x32 tiles, 64-deep k-steps), so that a GEMM
 * fetches each lane's scales with one coalesced 32-bit load per 256-deep
 * k-span.  The pages pad and re-block the scale tensor for their GEMM
 * ("Add QuTLASS support to vLLM", review of vllm/_custom_ops.py and
 * vllm/qutlass_utils/utils.py: padded_rows x padded_cols, to_blocked;
 * FlashInfer cute-dsl digest page: is_sf_swizzled_layout) but define it
 * only for another GPU's matrix cores; this is the same idea for CDNA4.
 *   - Rows are padded to a multiple of 32 and the K/32 groups of a row to a
 *     multiple of 8.
 *   - The scales form 256-byte blocks of 32 rows x 8 groups, stored in
 *     row-major order over (row block, group block).
 *   - In a block, 32-bit word l (l = 0..63) holds row l%32 of the block
 *     and, in bytes 0..3, its groups h, 2+h, 4+h, 6+h (h = l/32).
 *   - Padding bytes are 127 (the scale 2^0).
 * mx_blocked_scales_bytes returns the size in bytes (MX_ESHAPE for a bad
 * shape); blocked buffers must be 4-byte aligned.
 */
MX_API int64_t mx_blocked_scales_bytes(int64_t M, int64_t K);

/* Re-blocks row-major [M x K/32] scales into the blocked layout (every byte
 * of the blocked buffer is written, padding included). */
MX_API int mx_scales_to_blocked(const uint8_t *scales, int64_t M, int64_t K,
                                uint8_t *blocked);

/* mx_quantize with the scales written directly in the blocked layout
 * (padding included); codes as for mx_quantize. */
MX_API int mx_quantize_blocked(int fmt, const void *src, int64_t M, int64_t K,
                               const void *rot, int rot_size, uint8_t *codes,
                               uint8_t *blocked_scales);

/*
 * MX GEMM: c[M x N] (row-major) = alpha * A_dq . B_dq^T, where A is [M x K]
 * and B is [N x K], both with codes in the layout mx_quantize writes
 * (K-contiguous: the "TN" operand order) and scales in scale_layout
 * (MX_SCALES_ROWMAJOR or MX_SCALES_BLOCKED, both operands alike), on the
 * CDNA4 scaled matrix cores.  Products of codes are exact, each product
 * carries the two scales of its groups, and accumulation is fp32; the
 * result is multiplied by alpha in fp32 and stored as out_dtype (bf16 by
 * nearest-even rounding, or fp32).  This is the consumer of the quantized
 * layout, with the call shape and check of the pages' MXFP4 GEMM ("Add
 * QuTLASS support to vLLM", Purpose: MXFP4 matmul kernel with alpha and
 * bf16 output; review of the MXFP4 test: compared with a_dq @ b_dq^T).
 *   codes      16-byte aligned; c 16-byte aligned; row-major scales any
 *              alignment, blocked scales 4-byte aligned.  Row-major
 *              scales load fastest when K/32 is a multiple of 16 and
 *              they are 16-byte aligned (MXFP4), next when K/32 is a
 *              multiple of 8 (MXFP4) or 4 (MXFP8) and they are 4-byte
 *              aligned; other shapes read them byte by byte (same
 *              results, slower).  Blocked scales are faster still: for a
 *              large product, re-blocking row-major scales first
 *              (mx_scales_to_blocked, or mx_quantize_blocked in place of
 *              mx_quantize) and passing MX_SCALES_BLOCKED costs less than
 *              the row-major read (on MI355X, 8192 x 8192 x 28672 MXFP4:
 *              about 6 us of re-blocking against 130 us saved).
 *   K == 0 stores zeros.  M <= 65535 * 128; K <= 2^24 (MXFP4) or 2^23
 *   (MXFP8), else MX_ESHAPE.
 *   A scale byte of 0xFF (NaN) or an E4M3 NaN code gives NaN in the
 *   affected outputs.
 */
MX_API int mx_matmul(int fmt, const uint8_t *a_codes, const uint8_t *a_scales,
                     const uint8_t *b_codes, const uint8_t *b_scales,
                     int scale_layout, int64_t M, int64_t N, int64_t K,
                     float alpha, int out_dtype, void *c);

/*
 * NVFP4: the second 4-bit format the pages name beside MXFP4, with the same
 * fused rotations ("Add QuTLASS support to vLLM", Purpose: NVFP4 and MXFP4;
 * review of benchmarks/kernels/bench_nvfp4_qutlass.py: fusedQuantizeNv(a,
 * rotation, global_scale), scales viewed as [-1, K/16]).  The pages give no
 * rule; the reading is the published two-level NVFP4 format: groups of 16
 * elements along K, one E4M3 block scale per group, E2M1 elements, and a
 * per-tensor fp32 multiplier g = *global_scale (positive and finite; e.g.
 * 448 * 6 / amax of the tensor).  The steps are fp32 operations, each
 * rounded to nearest-even, so that the codes are defined exactly:
 *   c6 = g / 6;  q = amax * c6 (amax: the group's abs-max);
 *   scale byte = E4M3(q), nearest-even, saturating at 448 (0x7E); q <= 2^-10
 *   gives 0;  m = g / value(scale), or 0 for a zero scale;
 *   code = E2M1(x * m), nearest-even, saturating at 6, sign kept;
 *   dequantized value = value(code) * (value(scale) / g), then nearest-even
 *   into the destination type.
 * With a rotation, x is the rotated value (fp32 accumulation), as for MX.
 *   src          [M x K] bf16, K % 16 == 0 (with a rotation also K % r == 0
 *                and K % 32 == 0), 16-byte aligned.
 *   codes        [M x K/2] bytes, column 2k in bits 3:0; 16-byte aligned.
 *   scales       [M x K/16] E4M3 bytes, row-major; 4-byte aligned.
 *   global_scale device pointer to one fp32, 4-byte aligned; read by the
 *                kernel (so it may be computed on the device).
 * Non-finite input, or g not positive and finite, is outside the contract.
 * mx_nvfp4_qdq writes dst [M x K] bf16 (16-byte aligned); dst == src (an
 * exact alias) is allowed there, as for mx_qdq.
 */
MX_API int mx_nvfp4_quantize(const void *src, int64_t M, int64_t K,
                             const void *rot, int rot_size,
                             const float *global_scale, uint8_t *codes,
                             uint8_t *scales);
MX_API int mx_nvfp4_qdq(const void *src, int64_t M, int64_t K,
                        const void *rot, int rot_size,
                        const float *global_scale, void *dst);
MX_API int mx_nvfp4_dequantize(const uint8_t *codes, const uint8_t *scales,
                               int64_t M, int64_t K,
                               const float *global_scale, int dst_dtype,
                               void *dst);

/* Stream used by the calling thread's subsequent calls (a hipStream_t;
 * NULL = the default stream).  The setting is thread-local. */
MX_API void mx_set_stream(void *stream);
MX_API void *mx_get_stream(void);

/* Static, human-readable text for a status code. */
MX_API const char *mx_status_string(int status);

#ifdef __cplusplus
}
#endif
#endif
