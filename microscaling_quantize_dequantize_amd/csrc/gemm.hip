// MX GEMM consumer: C = alpha * A . B^T from MX codes and E8M0 scales, on the
// CDNA4 scaled matrix cores (v_mfma_scale_f32_32x32x64_f8f6f4).
//
// This is the consumer check of the quantized layout: the pages test their
// MXFP4 GEMM (matmul_mxf4_bf16_tn, "TN": both operands K-contiguous) against
// the dequantized operands multiplied in high precision ("[Transform]
// [Quantization] Add QuTLASS support to vLLM", Purpose: MXFP4 matmul kernel;
// review of the MXFP4 test).  A is [M x K] and B is [N x K], both in the
// layout mx_quantize writes (row-major codes; scales row-major [rows x K/32]
// or in the blocked layout).
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
// Tiling: a 256-thread workgroup (one wave per SIMD) owns a 256 x 256 tile
// of C; each wave a 128 x 128 quarter as 4 x 4 MFMA tiles, so that a k-step
// reads 8 fragments from LDS for 16 MFMAs.  K-slices of 64 code bytes per row
// are double-buffered in LDS (rows padded by 16 bytes): while the matrix
// cores work on slice k, slice k+1 is written to the other buffer from
// registers and slice k+2 is loaded from memory into those registers; the
// fragments of each k-step are read from LDS while the MFMAs of the previous
// step run (two register sets, one barrier per slice).
#include <type_traits>

#include "launch.h"
#include "mx_device.h"

namespace mx {

typedef int i32x8 __attribute__((ext_vector_type(8)));

constexpr int GT = 256, TI = 4, TJ = 4;               // threads; MFMA tiles per wave (rows, columns)
constexpr int BM = 64 * TI, BN = 64 * TJ;             // workgroup tile

// A k-slice is 64 code bytes of every row: 128 k of E2M1 (two MFMA k-steps)
// or 64 k of E4M3 (one k-step, twice as long on the matrix cores).
template <int FMT>
struct GemmShape {
  static constexpr int BK = FMT == 0 ? 128 : 64;      // k per slice
  static constexpr int RB = 64;                       // code bytes per row per k-slice
  static constexpr int LDR = RB + 16;                 // padded LDS row stride
  static constexpr int CH = RB / 16;                  // 16-byte chunks per row
  static constexpr int NCA = BM * CH / GT;            // chunks per thread, A
  static constexpr int NCB = BN * CH / GT;            // chunks per thread, B
  static constexpr int BUF = (BM + BN) * LDR;         // bytes per LDS buffer
};

// SL 0: row-major [rows x K/32] scales, staged through LDS with the codes;
// SL 1: the blocked layout, where a lane's word for its row block and
// 256-deep k-span is one coalesced 32-bit load.
template <int FMT, int OUT, int SL>
__global__ __launch_bounds__(GT) void k_mx_gemm(const uint8_t *__restrict__ A, const uint8_t *__restrict__ As,
                                                 const uint8_t *__restrict__ B, const uint8_t *__restrict__ Bs,
                                                 int64_t M, int64_t N, int64_t K, float alpha,
                                                 void *__restrict__ C) {
  using S = GemmShape<FMT>;
  constexpr int BK = S::BK;
  constexpr int CBSZ = FMT == 0 ? 4 : 0;  // FP4 E2M1 : FP8 E4M3
  __shared__ __attribute__((aligned(16))) uint8_t sm[2 * S::BUF];
  __shared__ __attribute__((aligned(4))) uint8_t ss[2][BM + BN][4];  // row-major scales of a slice (SL 0)
  __shared__ unsigned sw[2][4][TI + TJ][64];                         // each wave's blocked words (SL 1)

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r = lane & 31, h = lane >> 5;
  const int64_t m0 = (int64_t)blockIdx.y * BM, n0 = (int64_t)blockIdx.x * BN;
  const int wm = (wave >> 1) * (32 * TI), wn = (wave & 1) * (32 * TJ);
  const int64_t rowbytes = FMT == 0 ? K / 2 : K;
  const int64_t groups = K / 32;
  const int64_t gblocks = (groups + 7) / 8;
  const int nslices = (int)((K + BK - 1) / BK);

  // ---- registers in flight: the codes (and scales) of one k-slice --------
  u32x4 pa[S::NCA], pb[S::NCB];
  unsigned psa = 0x7F7F7F7Fu, psb = 0x7F7F7F7Fu;  // SL 0: this thread's row's 4 scale bytes
  unsigned pwa[TI], pwb[TJ];                      // SL 1: this lane's blocked words

  const bool interior = m0 + BM <= M && n0 + BN <= N;  // wave-uniform
  auto load_slice = [&](int ks) {
    const int64_t k0 = (int64_t)ks * BK, kb0 = FMT == 0 ? k0 / 2 : k0;
    if (kb0 >= rowbytes) return;  // past the end: nothing to load
    if (interior && kb0 + S::RB <= rowbytes) {
      // a whole slice inside the operands: no per-chunk bounds
#pragma unroll
      for (int it = 0; it < S::NCA; ++it) {
        const int idx = tid + it * GT, row = idx / S::CH, c = idx % S::CH;
        pa[it] = *(const u32x4 *)(A + (m0 + row) * rowbytes + kb0 + 16 * c);
      }
#pragma unroll
      for (int it = 0; it < S::NCB; ++it) {
        const int idx = tid + it * GT, row = idx / S::CH, c = idx % S::CH;
        pb[it] = *(const u32x4 *)(B + (n0 + row) * rowbytes + kb0 + 16 * c);
      }
    } else {
#pragma unroll
      for (int it = 0; it < S::NCA; ++it) {
        const int idx = tid + it * GT, row = idx / S::CH, c = idx % S::CH;
        const int64_t kb = kb0 + 16 * c;
        pa[it] = (m0 + row < M && kb < rowbytes) ? *(const u32x4 *)(A + (m0 + row) * rowbytes + kb)
                                                 : u32x4{0u, 0u, 0u, 0u};
      }
#pragma unroll
      for (int it = 0; it < S::NCB; ++it) {
        const int idx = tid + it * GT, row = idx / S::CH, c = idx % S::CH;
        const int64_t kb = kb0 + 16 * c;
        pb[it] = (n0 + row < N && kb < rowbytes) ? *(const u32x4 *)(B + (n0 + row) * rowbytes + kb)
                                                 : u32x4{0u, 0u, 0u, 0u};
      }
    }
    // rows past the end and groups past K hold zero codes; any finite scale will do
    if (SL == 0) {
      unsigned wa = 0x7F7F7F7Fu, wb = 0x7F7F7F7Fu;
#pragma unroll
      for (int j = 0; j < BK / 32; ++j) {
        const int64_t g = k0 / 32 + j;
        const unsigned va = (m0 + tid < M && g < groups) ? As[(m0 + tid) * groups + g] : 127u;
        const unsigned vb = (n0 + tid < N && g < groups) ? Bs[(n0 + tid) * groups + g] : 127u;
        wa = (wa & ~(0xFFu << (8 * j))) | (va << (8 * j));
        wb = (wb & ~(0xFFu << (8 * j))) | (vb << (8 * j));
      }
      psa = wa;
      psb = wb;
    } else {
#pragma unroll
      for (int i = 0; i < TI; ++i) {
        const int64_t ra = m0 + wm + 32 * i;
        pwa[i] = ra < M ? ((const unsigned *)As)[((ra >> 5) * gblocks + (k0 >> 8)) * 64 + lane] : 0x7F7F7F7Fu;
      }
#pragma unroll
      for (int j = 0; j < TJ; ++j) {
        const int64_t rb = n0 + wn + 32 * j;
        pwb[j] = rb < N ? ((const unsigned *)Bs)[((rb >> 5) * gblocks + (k0 >> 8)) * 64 + lane] : 0x7F7F7F7Fu;
      }
    }
  };
  auto store_slice = [&](int buf) {
    uint8_t *sA = sm + buf * S::BUF, *sB = sA + BM * S::LDR;
#pragma unroll
    for (int it = 0; it < S::NCA; ++it) {
      const int idx = tid + it * GT, row = idx / S::CH, c = idx % S::CH;
      *(u32x4 *)(sA + row * S::LDR + 16 * c) = pa[it];
    }
#pragma unroll
    for (int it = 0; it < S::NCB; ++it) {
      const int idx = tid + it * GT, row = idx / S::CH, c = idx % S::CH;
      *(u32x4 *)(sB + row * S::LDR + 16 * c) = pb[it];
    }
    if (SL == 0) {
      *(unsigned *)ss[buf][tid] = psa;  // one thread per row (GT == BM == BN)
      *(unsigned *)ss[buf][BM + tid] = psb;
    } else {
#pragma unroll
      for (int i = 0; i < TI; ++i) sw[buf][wave][i][lane] = pwa[i];
#pragma unroll
      for (int j = 0; j < TJ; ++j) sw[buf][wave][TI + j][lane] = pwb[j];
    }
  };
  static_assert(GT == BM && GT == BN, "one thread per row stages the row-major scales");

  f32x16 acc[TI][TJ];
#pragma unroll
  for (int i = 0; i < TI; ++i)
#pragma unroll
    for (int j = 0; j < TJ; ++j) acc[i][j] = f32x16{};

  // ---- fragments of one 64-deep k-step, two sets (steps alternate) -------
  constexpr int NS = BK / 64;           // k-steps per slice
  // E2M1 fragments are 16 bytes (the MFMA reads 4 registers); E4M3
  // fragments 32 bytes, kept as one 8-register tuple
  using Frag = typename std::conditional<FMT == 0, u32x4, i32x8>::type;
  Frag fr[NS][TI + TJ];
  int sc[NS][TI + TJ];
  // fragments and scale bytes of k-step s of slice ks (LDS buffer buf)
  auto read_frags = [&](auto P, int buf, int ks, int s) {
    constexpr int p = decltype(P)::value;
    const uint8_t *sA = sm + buf * S::BUF, *sB = sA + BM * S::LDR;
    const int sh = 8 * ((int)(((int64_t)ks * BK >> 6) & 3) + s);  // k-step within the 256-deep span
#pragma unroll
    for (int f = 0; f < TI + TJ; ++f) {
      const int row = (f < TI ? wm + 32 * f : wn + 32 * (f - TI)) + r;
      const uint8_t *base = (f < TI ? sA : sB) + row * S::LDR + (FMT == 0 ? 32 : 64) * s + 16 * h;
      if constexpr (FMT == 0) {
        fr[p][f] = *(const u32x4 *)base;
      } else {
        const u32x4 lo = *(const u32x4 *)base, hi = *(const u32x4 *)(base + 32);
        fr[p][f] = i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
      }
      if (SL == 0) sc[p][f] = (int)ss[buf][(f < TI ? 0 : BM) + row][2 * s + h];
      else sc[p][f] = (int)((sw[buf][wave][f][lane] >> sh) & 0xFFu);
    }
  };
  auto mfma_step = [&](auto P) {
    constexpr int p = decltype(P)::value;
#pragma unroll
    for (int i = 0; i < TI; ++i)
#pragma unroll
      for (int j = 0; j < TJ; ++j) {
        i32x8 fa, fb;
        if constexpr (FMT == 0) {
          const u32x4 a = fr[p][i], b = fr[p][TI + j];  // upper halves unused for E2M1
          fa = i32x8{(int)a.x, (int)a.y, (int)a.z, (int)a.w, 0, 0, 0, 0};
          fb = i32x8{(int)b.x, (int)b.y, (int)b.z, (int)b.w, 0, 0, 0, 0};
        } else {
          fa = fr[p][i];
          fb = fr[p][TI + j];
        }
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fa, fb, acc[i][j], CBSZ, CBSZ, 0, sc[p][i], 0,
                                                                    sc[p][TI + j]);
      }
  };
  // interleave the 16 MFMAs of a step with the LDS reads of the next one
  auto interleave = [&]() {
#pragma unroll
    for (int k = 0; k < TI * TJ; ++k) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // two LDS reads
    }
  };
  // the last k-step of slice ks: stage slice ks+1 into the other buffer and
  // slice ks+2 into registers, synchronise, then read step 0 of slice ks+1
  // while the matrix cores run step P.  Past the end the stores and reads
  // touch only unused LDS and the loads are bounds-checked away.
  auto last_step = [&](auto P, auto Q, int ks) {
    const int buf = ks & 1;
    store_slice(buf ^ 1);
    load_slice(ks + 2);
    __syncthreads();
    read_frags(Q, buf ^ 1, ks + 1, 0);
    mfma_step(P);
    interleave();
  };
  using P0 = std::integral_constant<int, 0>;
  using P1 = std::integral_constant<int, 1>;

  load_slice(0);
  store_slice(0);
  load_slice(1);
  __syncthreads();

  if constexpr (NS == 2) {
    // E2M1: two k-steps per slice, fragment sets 0 and 1 within each slice
    read_frags(P0{}, 0, 0, 0);
    for (int ks = 0; ks < nslices; ++ks) {
      read_frags(P1{}, ks & 1, ks, 1);
      mfma_step(P0{});
      interleave();
      last_step(P1{}, P0{}, ks);
    }
  } else {
    // E4M3: one k-step per slice and one fragment set (two sets of 32-byte
    // fragments do not fit beside the accumulators)
    for (int ks = 0; ks < nslices; ++ks) {
      read_frags(P0{}, ks & 1, ks, 0);
      mfma_step(P0{});
      store_slice((ks & 1) ^ 1);
      load_slice(ks + 2);
      __syncthreads();
    }
  }

  // accumulator: lane l, register a holds C[8(a/4) + 4(l/32) + a%4][l%32]
#pragma unroll
  for (int i = 0; i < TI; ++i)
#pragma unroll
    for (int j = 0; j < TJ; ++j) {
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
