// MX GEMM consumer: C = alpha * A . B^T from MX codes and E8M0 scales, on the
// CDNA4 scaled matrix cores (v_mfma_scale_f32_32x32x64_f8f6f4).
//
// This is the consumer check of the quantized layout: the pages test their
// MXFP4 GEMM (matmul_mxf4_bf16_tn, "TN": both operands K-contiguous) against
// the dequantized operands multiplied in high precision ("[Transform]
// [Quantization] Add QuTLASS support to vLLM", Purpose: MXFP4 matmul kernel;
// review of the MXFP4 test).  A is [M x K] and B is [N x K], both in the
// layout mx_quantize writes (row-major codes, unpadded [rows x K/32] scales).
//
// Operand layout of the scaled MFMA (characterised on gfx950): in a 64-deep
// k-step, lane l supplies row (or column) l%32 and
//   FP4: the 32 consecutive k of MX group l/32 (16 bytes, low nibble first)
//        plus that group's scale byte;
//   FP8: bytes [16h, 16h+16) of both groups of the step (h = l/32), k-block
//        order 32*chunk + 16h + byte, plus the scale of group h.
// So the row-major code layout feeds the matrix cores directly: no
// reordering of codes or scales is needed.
//
// Tiling: a 256-thread workgroup owns a 128 x 128 tile of C; each wave a
// 64 x 64 quarter (2 x 2 MFMA tiles).  128-deep k-slices of A and B are
// staged in LDS (rows padded by 16 bytes, conflict-free 16-byte reads).
#include "launch.h"
#include "mx_device.h"

namespace mx {

typedef int i32x8 __attribute__((ext_vector_type(8)));

constexpr int GT = 256, BM = 128, BN = 128, BK = 128;

// SL 0: row-major [rows x K/32] scales, staged through LDS per k-slice;
// SL 1: the blocked layout, where a lane's word for its row block and
// 256-deep k-span is one coalesced 32-bit load.
template <int FMT, int OUT, int SL>
__global__ __launch_bounds__(GT) void k_mx_gemm(const uint8_t *__restrict__ A, const uint8_t *__restrict__ As,
                                                 const uint8_t *__restrict__ B, const uint8_t *__restrict__ Bs,
                                                 int64_t M, int64_t N, int64_t K, float alpha,
                                                 void *__restrict__ C) {
  constexpr int RB = FMT == 0 ? BK / 2 : BK;  // code bytes per row per k-slice
  constexpr int LDR = RB + 16;                // padded LDS row stride
  constexpr int CH = RB / 16;                 // 16-byte chunks per row
  constexpr int GS = BK / 32;                 // scale groups per row per k-slice
  constexpr int CBSZ = FMT == 0 ? 4 : 0;      // FP4 E2M1 : FP8 E4M3
  __shared__ __attribute__((aligned(16))) uint8_t sA[BM * LDR];
  __shared__ __attribute__((aligned(16))) uint8_t sB[BN * LDR];
  __shared__ uint8_t sSA[BM * GS], sSB[BN * GS];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r = lane & 31, h = lane >> 5;
  const int64_t m0 = (int64_t)blockIdx.y * BM, n0 = (int64_t)blockIdx.x * BN;
  const int wm = (wave >> 1) * 64, wn = (wave & 1) * 64;
  const int64_t rowbytes = FMT == 0 ? K / 2 : K;
  const int64_t groups = K / 32;
  const int64_t gblocks = (groups + 7) / 8;

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x16{};

  for (int64_t k0 = 0; k0 < K; k0 += BK) {
    const int64_t kb0 = FMT == 0 ? k0 / 2 : k0;  // byte offset of the slice in a row
#pragma unroll
    for (int it = 0; it < BM * CH / GT; ++it) {
      const int idx = tid + it * GT, row = idx / CH, c = idx % CH;
      const int64_t kb = kb0 + 16 * c;
      u32x4 va = {0u, 0u, 0u, 0u}, vb = {0u, 0u, 0u, 0u};
      if (m0 + row < M && kb < rowbytes) va = *(const u32x4 *)(A + (m0 + row) * rowbytes + kb);
      if (n0 + row < N && kb < rowbytes) vb = *(const u32x4 *)(B + (n0 + row) * rowbytes + kb);
      *(u32x4 *)(sA + row * LDR + 16 * c) = va;
      *(u32x4 *)(sB + row * LDR + 16 * c) = vb;
    }
    // rows past the end and groups past K hold zero codes; any finite scale will do
    unsigned wa[2] = {0x7F7F7F7Fu, 0x7F7F7F7Fu}, wb[2] = {0x7F7F7F7Fu, 0x7F7F7F7Fu};
    if (SL == 0) {
#pragma unroll
      for (int it = 0; it < BM * GS / GT; ++it) {
        const int idx = tid + it * GT, row = idx / GS, gg = idx % GS;
        const int64_t g = k0 / 32 + gg;
        sSA[idx] = (m0 + row < M && g < groups) ? As[(m0 + row) * groups + g] : (uint8_t)127;
        sSB[idx] = (n0 + row < N && g < groups) ? Bs[(n0 + row) * groups + g] : (uint8_t)127;
      }
    } else {
      // row blocks exist up to the one holding the last row; padding groups hold 127
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int64_t ra = m0 + wm + 32 * i, rb = n0 + wn + 32 * i;
        if (ra < M) wa[i] = ((const unsigned *)As)[((ra >> 5) * gblocks + (k0 >> 8)) * 64 + lane];
        if (rb < N) wb[i] = ((const unsigned *)Bs)[((rb >> 5) * gblocks + (k0 >> 8)) * 64 + lane];
      }
    }
    __syncthreads();
#pragma unroll
    for (int s = 0; s < BK / 64; ++s) {
      i32x8 fa[2], fb[2];
      int sa[2], sb[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int ra = wm + 32 * i + r, rb = wn + 32 * i + r;
        u32x4 a0, a1 = {0u, 0u, 0u, 0u}, b0, b1 = {0u, 0u, 0u, 0u};
        if (FMT == 0) {
          a0 = *(const u32x4 *)(sA + ra * LDR + 32 * s + 16 * h);
          b0 = *(const u32x4 *)(sB + rb * LDR + 32 * s + 16 * h);
        } else {
          a0 = *(const u32x4 *)(sA + ra * LDR + 64 * s + 16 * h);
          a1 = *(const u32x4 *)(sA + ra * LDR + 64 * s + 32 + 16 * h);
          b0 = *(const u32x4 *)(sB + rb * LDR + 64 * s + 16 * h);
          b1 = *(const u32x4 *)(sB + rb * LDR + 64 * s + 32 + 16 * h);
        }
        fa[i] = i32x8{(int)a0.x, (int)a0.y, (int)a0.z, (int)a0.w, (int)a1.x, (int)a1.y, (int)a1.z, (int)a1.w};
        fb[i] = i32x8{(int)b0.x, (int)b0.y, (int)b0.z, (int)b0.w, (int)b1.x, (int)b1.y, (int)b1.z, (int)b1.w};
        if (SL == 0) {
          sa[i] = sSA[ra * GS + 2 * s + h];  // this lane's group of the 64-deep step
          sb[i] = sSB[rb * GS + 2 * s + h];
        } else {
          const int sh = 8 * ((int)((k0 >> 6) & 3) + s);  // k-step within the 256-deep span
          sa[i] = (int)((wa[i] >> sh) & 0xFFu);
          sb[i] = (int)((wb[i] >> sh) & 0xFFu);
        }
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fa[i], fb[j], acc[i][j], CBSZ, CBSZ, 0,
                                                                      sa[i], 0, sb[j]);
    }
    __syncthreads();
  }
  // accumulator: lane l, register a holds C[8(a/4) + 4(l/32) + a%4][l%32]
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int64_t col = n0 + wn + 32 * j + r;
#pragma unroll
      for (int a = 0; a < 16; ++a) {
        const int64_t row = m0 + wm + 32 * i + 8 * (a / 4) + 4 * h + a % 4;
        if (row < M && col < N) {
          const float v = alpha * acc[i][j][a];
          if (OUT == 0) ((uint16_t *)C)[row * N + col] = (uint16_t)(v != v ? 0x7FC0u : bf16_rne(v));
          else ((float *)C)[row * N + col] = v;
        }
      }
    }
}

template <int SL>
static void run_gemm(int fmt, int out_dtype, dim3 grid, const uint8_t *a, const uint8_t *as, const uint8_t *b,
                     const uint8_t *bs, int64_t M, int64_t N, int64_t K, float alpha, void *c, hipStream_t st) {
  if (fmt == 0 && out_dtype == 0) k_mx_gemm<0, 0, SL><<<grid, GT, 0, st>>>(a, as, b, bs, M, N, K, alpha, c);
  else if (fmt == 0) k_mx_gemm<0, 1, SL><<<grid, GT, 0, st>>>(a, as, b, bs, M, N, K, alpha, c);
  else if (out_dtype == 0) k_mx_gemm<1, 0, SL><<<grid, GT, 0, st>>>(a, as, b, bs, M, N, K, alpha, c);
  else k_mx_gemm<1, 1, SL><<<grid, GT, 0, st>>>(a, as, b, bs, M, N, K, alpha, c);
}

hipError_t launch_gemm(int fmt, const uint8_t *a, const uint8_t *as, const uint8_t *b, const uint8_t *bs,
                       int scale_layout, int64_t M, int64_t N, int64_t K, float alpha, int out_dtype, void *c,
                       hipStream_t st) {
  const dim3 grid((unsigned)((N + BN - 1) / BN), (unsigned)((M + BM - 1) / BM));
  if (scale_layout == 0) run_gemm<0>(fmt, out_dtype, grid, a, as, b, bs, M, N, K, alpha, c, st);
  else run_gemm<1>(fmt, out_dtype, grid, a, as, b, bs, M, N, K, alpha, c, st);
  return hipGetLastError();
}

}  // namespace mx
