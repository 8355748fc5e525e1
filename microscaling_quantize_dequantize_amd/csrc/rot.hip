// Rotated MX kernels: per-chunk rotation on MFMA, then the MX step.
//
// "[Transform] [Quantization] Add QuTLASS support to vLLM", Online
// rotations: the transform, the quantization and the scale computation are
// fused, and the rotation matrix (size 16/32/64/128) is loaded at runtime.
// Every r-chunk x of a row becomes y = x . R (y[j] = sum_t x[t] R[t][j]).
//
// Since K is a multiple of r and of 32, chunks never straddle rows and the
// matrix is one flat array of r-chunks.  The kernel works on blocks of
// RB = max(r, 32) elements with the block-diagonal matrix diag(R, ..., R) of
// size RB (r = 16 gives diag(R, R)), so that every 32-group lies inside one
// block.
//
// The contraction Y^T = Reff^T . X^T runs on v_mfma_f32_32x32x16_bf16 (bf16
// products are exact in fp32; accumulation in fp32):
//   A (32 x 16) = a 32-column slice jt of Reff^T, staged once per workgroup in
//                 LDS in the exact order the MFMAs read it;
//   B (16 x 32) = 32 consecutive blocks ("a tile"), lane l holding block l%32.
// The k index of an MFMA is free to permute as long as A and B agree, so lane
// l reads the half (l/32) of its block as RB/16 contiguous 16-byte loads:
// k-step kb covers t = (l/32)*RB/2 + 8*kb + i, i = 0..7.
// In the 32x32 accumulator, lane l holds, for its block, the 16 values
// j = 32*jt + 8q + 4*(l/32) + e (q, e = 0..3): one 32-group (jt) is split
// between lanes l and l+32, so its abs-max takes one v_permlane32_swap.  The
// same swap then trades 4-element runs so that each lane stores 16-byte runs.
#include "launch.h"
#include "mx_device.h"

namespace mx {

constexpr int RTHREADS = 256;

// Entry (t, j) of the block-diagonal RB x RB matrix built from the r x r R.
template <typename T>
__device__ __forceinline__ T reff(const T *__restrict__ rot, int r, int t, int j) {
  if (t / r != j / r) return T(0);
  return rot[(t % r) * r + (j % r)];
}

// Store a lane's share of one rotated, quantized 32-group.
//   acc[4q + e] = y[32*jt + 8q + 4h + e] of block `blk` (h = lane / 32).
template <int FMT, int OP, int RB, bool SRC_BF16>
__device__ __forceinline__ void group_epilogue(const f32x16 &acc, int64_t blk, int jt, int h,
                                               bool valid, void *__restrict__ dst,
                                               uint8_t *__restrict__ codes, unsigned &sbw) {
  const int64_t e0 = blk * RB + jt * 32;  // first element of the group
  if (OP == OP_ROTATE) {
    if (valid) {
      float *d = (float *)dst + e0 + 4 * h;
#pragma unroll
      for (int q = 0; q < 4; ++q)
        __builtin_nontemporal_store(f32x4{acc[4 * q], acc[4 * q + 1], acc[4 * q + 2], acc[4 * q + 3]},
                                    (f32x4 *)(d + 8 * q));
    }
    return;
  }
  unsigned m = 0;
#pragma unroll
  for (int a = 0; a < 16; ++a) m = umax(m, __float_as_uint(acc[a]) & 0x7FFFFFFFu);
  m = max_across_halves(m);
  const unsigned sb = scale_byte<FMT>(m);
  const float sc = scale_operand(sb);
  sbw |= sb << (8 * jt);
  float y[16];
#pragma unroll
  for (int a = 0; a < 16; ++a) y[a] = acc[a];
  if (FMT == 1) {
    const float cl = __uint_as_float(((sb + 8u) << 23) | 0x600000u);  // 448 * 2^s
#pragma unroll
    for (int a = 0; a < 16; ++a) y[a] = clamp_f32(y[a], cl);
  }
  // c[q]: the run's 4 codes (E2M1: 16 bits, E4M3: 32 bits)
  unsigned c[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    if (FMT == 0) {
      unsigned v = fp4_from_f32x2<0>(0u, y[4 * q], y[4 * q + 1], sc);
      c[q] = fp4_from_f32x2<1>(v, y[4 * q + 2], y[4 * q + 3], sc);
    } else {
      unsigned v = fp8_from_f32x2<false>(0u, y[4 * q], y[4 * q + 1], sc);
      c[q] = fp8_from_f32x2<true>(v, y[4 * q + 2], y[4 * q + 3], sc);
    }
  }
  if (OP == OP_QDQ && SRC_BF16) {
    unsigned o[8];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      if (FMT == 0) {
        o[2 * q] = __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(c[q], sc, 0));
        o[2 * q + 1] = __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(c[q], sc, 1));
      } else {
        o[2 * q] = __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c[q], sc, false));
        o[2 * q + 1] = __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c[q], sc, true));
      }
    }
    if (sb == 255u) {
#pragma unroll
      for (int k = 0; k < 8; ++k) o[k] = BF16_NAN | (BF16_NAN << 16);
    }
    // runs (0,1) and (2,3): lower half ends with j 0-7 / 16-23, upper 8-15 / 24-31
    swap_halves(o[0], o[2]);
    swap_halves(o[1], o[3]);
    swap_halves(o[4], o[6]);
    swap_halves(o[5], o[7]);
    if (valid) {
      u32x4 *d = (u32x4 *)((uint16_t *)dst + e0 + 8 * h);
      __builtin_nontemporal_store(u32x4{o[0], o[1], o[2], o[3]}, d);
      __builtin_nontemporal_store(u32x4{o[4], o[5], o[6], o[7]}, d + 2);
    }
  } else if (OP == OP_QDQ) {  // fp32 destination: exact software decode
    const int s = (int)sb - 127;
    constexpr int CB = FMT == 0 ? 4 : 8;
    constexpr unsigned CM = (1u << CB) - 1u;
    if (valid) {
      float *d = (float *)dst + e0 + 4 * h;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        f32x4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e)
          v[e] = sb == 255u ? __uint_as_float(F32_NAN) : decode_code<FMT>((c[q] >> (CB * e)) & CM, s);
        __builtin_nontemporal_store(v, (f32x4 *)(d + 8 * q));
      }
    }
  } else {  // quantize: codes
    if (FMT == 0) {
      // byte pairs: lower lane holds codes of j 0-3|8-11 (ca) and 16-19|24-27
      // (cb); the upper lane the runs 4 elements later.
      unsigned ca = c[0] | (c[1] << 16), cb = c[2] | (c[3] << 16);
      if (sb == 255u) ca = cb = 0u;
      swap_halves(ca, cb);
      // lower: ca = bytes {0-1, 4-5}, cb = {2-3, 6-7}; upper: {8-9,12-13}, {10-11,14-15}
      const unsigned w0 = (ca & 0xFFFFu) | (cb << 16);
      const unsigned w1 = (ca >> 16) | (cb & 0xFFFF0000u);
      if (valid) __builtin_nontemporal_store(u32x2{w0, w1}, (u32x2 *)(codes + e0 / 2 + 8 * h));
    } else {
      unsigned r0 = c[0], r1 = c[1], r2 = c[2], r3 = c[3];
      if (sb == 255u) r0 = r1 = r2 = r3 = 0x7F7F7F7Fu;
      swap_halves(r0, r1);  // lower: bytes 0-7,  upper: 8-15
      swap_halves(r2, r3);  // lower: bytes 16-23, upper: 24-31
      swap_halves(r0, r2);  // lower: 0-3, 8-11 -> with r1/r3 below: 0-15
      swap_halves(r1, r3);
      // lower now holds bytes 0-3 (r0), 4-7 (r1), 8-11 (r2), 12-15 (r3);
      // upper holds 16-19, 20-23, 24-27, 28-31.
      if (valid) __builtin_nontemporal_store(u32x4{r0, r1, r2, r3}, (u32x4 *)(codes + e0 + 16 * h));
    }
  }
}

template <int FMT, int OP, int RB>
__global__ __launch_bounds__(RTHREADS) void k_rot_bf16(const uint16_t *__restrict__ src,
                                                       const uint16_t *__restrict__ rot, int r,
                                                       void *__restrict__ dst,
                                                       uint8_t *__restrict__ codes,
                                                       uint8_t *__restrict__ scales,
                                                       int64_t n_blk) {
  constexpr int NJT = RB / 32, NKB = RB / 16, HALF = RB / 2;
  __shared__ u32x4 sA[NJT * NKB * 64];
  for (int idx = threadIdx.x; idx < NJT * NKB * 64; idx += RTHREADS) {
    const int ln = idx & 63, f = idx >> 6, jt = f / NKB, kb = f % NKB;
    const int j = jt * 32 + (ln & 31), t0 = (ln >> 5) * HALF + 8 * kb;
    unsigned w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      w[i] = (unsigned)reff(rot, r, t0 + 2 * i, j) | ((unsigned)reff(rot, r, t0 + 2 * i + 1, j) << 16);
    sA[idx] = u32x4{w[0], w[1], w[2], w[3]};
  }
  __syncthreads();

  const int lane = threadIdx.x & 63, h = lane >> 5;
  const int waves = RTHREADS / 64;
  const int64_t n_tiles = (n_blk + 31) / 32;
  for (int64_t tile = (int64_t)blockIdx.x * waves + (threadIdx.x >> 6); tile < n_tiles;
       tile += (int64_t)gridDim.x * waves) {
    const int64_t blk = tile * 32 + (lane & 31);
    const bool valid = blk < n_blk;
    const u32x4 *p = (const u32x4 *)(src + blk * RB + h * HALF);
    u32x4 b[NKB];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) b[kb] = valid ? __builtin_nontemporal_load(p + kb) : u32x4{0u, 0u, 0u, 0u};
    unsigned sbw = 0;
#pragma unroll
    for (int jt = 0; jt < NJT; ++jt) {
      f32x16 acc = {};
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, sA[(jt * NKB + kb) * 64 + lane]),
                                                      __builtin_bit_cast(bf16x8, b[kb]), acc, 0, 0, 0);
      group_epilogue<FMT, OP, RB, true>(acc, blk, jt, h, valid, dst, codes, sbw);
    }
    if (OP == OP_QUANT && h == 0 && valid) {
      if (NJT == 4) *(unsigned *)(scales + blk * 4) = sbw;
      else if (NJT == 2) *(uint16_t *)(scales + blk * 2) = (uint16_t)sbw;
      else scales[blk] = (uint8_t)sbw;
    }
  }
}

// fp32 source: v_mfma_f32_32x32x2_f32, lane l supplying B[k = l/32][n = l%32]
// and A[m = l%32][k = l/32]; k-step kb covers t = (l/32)*RB/2 + kb.
template <int FMT, int OP, int RB>
__global__ __launch_bounds__(RTHREADS) void k_rot_f32(const float *__restrict__ src,
                                                      const float *__restrict__ rot, int r,
                                                      void *__restrict__ dst, int64_t n_blk) {
  constexpr int NJT = RB / 32, HALF = RB / 2;
  __shared__ float sA[NJT * HALF * 64];
  for (int idx = threadIdx.x; idx < NJT * HALF * 64; idx += RTHREADS) {
    const int ln = idx & 63, f = idx >> 6, jt = f / HALF, kb = f % HALF;
    sA[idx] = reff(rot, r, (ln >> 5) * HALF + kb, jt * 32 + (ln & 31));
  }
  __syncthreads();

  const int lane = threadIdx.x & 63, h = lane >> 5;
  const int waves = RTHREADS / 64;
  const int64_t n_tiles = (n_blk + 31) / 32;
  for (int64_t tile = (int64_t)blockIdx.x * waves + (threadIdx.x >> 6); tile < n_tiles;
       tile += (int64_t)gridDim.x * waves) {
    const int64_t blk = tile * 32 + (lane & 31);
    const bool valid = blk < n_blk;
    const f32x4 *p = (const f32x4 *)(src + blk * RB + h * HALF);
    float xv[HALF];
#pragma unroll
    for (int k4 = 0; k4 < HALF / 4; ++k4) {
      const f32x4 v = valid ? __builtin_nontemporal_load(p + k4) : f32x4{0.f, 0.f, 0.f, 0.f};
      xv[4 * k4] = v[0];
      xv[4 * k4 + 1] = v[1];
      xv[4 * k4 + 2] = v[2];
      xv[4 * k4 + 3] = v[3];
    }
    unsigned sbw = 0;
#pragma unroll
    for (int jt = 0; jt < NJT; ++jt) {
      f32x16 acc = {};
#pragma unroll
      for (int kb = 0; kb < HALF; ++kb)
        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(sA[(jt * HALF + kb) * 64 + lane], xv[kb], acc, 0, 0, 0);
      group_epilogue<FMT, OP, RB, false>(acc, blk, jt, h, valid, dst, nullptr, sbw);
    }
  }
}

template <int FMT, int OP, int RB>
static void run_bf16(const void *src, const void *rot, int r, void *dst, uint8_t *codes,
                     uint8_t *scales, int64_t n, unsigned grid_cap, hipStream_t st) {
  const int64_t n_blk = n / RB;
  const int64_t tiles = (n_blk + 31) / 32;
  int64_t g = (tiles + 3) / 4;
  if (g > grid_cap) g = grid_cap;
  k_rot_bf16<FMT, OP, RB><<<(unsigned)g, RTHREADS, 0, st>>>((const uint16_t *)src, (const uint16_t *)rot, r,
                                                           dst, codes, scales, n_blk);
}

template <int FMT, int OP, int RB>
static void run_f32(const void *src, const void *rot, int r, void *dst, int64_t n, unsigned grid_cap,
                    hipStream_t st) {
  const int64_t n_blk = n / RB;
  const int64_t tiles = (n_blk + 31) / 32;
  int64_t g = (tiles + 3) / 4;
  if (g > grid_cap) g = grid_cap;
  k_rot_f32<FMT, OP, RB><<<(unsigned)g, RTHREADS, 0, st>>>((const float *)src, (const float *)rot, r, dst, n_blk);
}

template <int FMT, int OP>
static void dispatch_rb(int dtype, const void *src, const void *rot, int r, void *dst, uint8_t *codes,
                        uint8_t *scales, int64_t n, unsigned cap, hipStream_t st) {
  const int rb = r < 32 ? 32 : r;
  if (dtype == 0) {
    if (rb == 32) run_bf16<FMT, OP, 32>(src, rot, r, dst, codes, scales, n, cap, st);
    else if (rb == 64) run_bf16<FMT, OP, 64>(src, rot, r, dst, codes, scales, n, cap, st);
    else run_bf16<FMT, OP, 128>(src, rot, r, dst, codes, scales, n, cap, st);
  } else if (OP != OP_QUANT) {
    if (rb == 32) run_f32<FMT, OP, 32>(src, rot, r, dst, n, cap, st);
    else if (rb == 64) run_f32<FMT, OP, 64>(src, rot, r, dst, n, cap, st);
    else run_f32<FMT, OP, 128>(src, rot, r, dst, n, cap, st);
  }
}

hipError_t launch_rot(int fmt, int op, int dtype, const void *src, const void *rot, int r, void *dst,
                      uint8_t *codes, uint8_t *scales, int64_t n, hipStream_t st) {
  const unsigned cap = (unsigned)device_cu_count() * 8u;
  if (op == OP_ROTATE) {
    dispatch_rb<0, OP_ROTATE>(dtype, src, rot, r, dst, codes, scales, n, cap, st);
  } else if (fmt == 0) {
    if (op == OP_QDQ) dispatch_rb<0, OP_QDQ>(dtype, src, rot, r, dst, codes, scales, n, cap, st);
    else dispatch_rb<0, OP_QUANT>(dtype, src, rot, r, dst, codes, scales, n, cap, st);
  } else {
    if (op == OP_QDQ) dispatch_rb<1, OP_QDQ>(dtype, src, rot, r, dst, codes, scales, n, cap, st);
    else dispatch_rb<1, OP_QUANT>(dtype, src, rot, r, dst, codes, scales, n, cap, st);
  }
  return hipGetLastError();
}

}  // namespace mx
