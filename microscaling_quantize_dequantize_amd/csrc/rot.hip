// Rotated MX kernels: per-chunk rotation on MFMA, then the MX step.
//
// "[Transform] [Quantization] Add QuTLASS support to vLLM", Online
// rotations: the transform, the quantization and the scale computation are
// fused, and the rotation matrix (size 16/32/64/128) is loaded at runtime.
// Every r-chunk x of a row becomes y = x . R (y[j] = sum_t x[t] R[t][j]).
//
// Since K is a multiple of r and of 32, chunks never straddle rows and the
// matrix is one flat array of r-chunks.  The kernels work on blocks of
// RB >= max(r, 32) elements with the block-diagonal matrix diag(R, ..., R)
// of size RB, so that every 32-group lies inside one block (RB = max(r, 32),
// or 64 for r = 16 and 32 where the shape allows; see staged_rb).
//
// The contraction Y^T = Reff^T . X^T runs on v_mfma_f32_32x32x16_bf16 (bf16
// products are exact in fp32; accumulation in fp32):
//   A (32 x 16) = a 32-column slice jt of Reff^T, staged once per workgroup in
//                 LDS in the exact order the MFMAs read it;
//   B (16 x 32) = 32 consecutive blocks ("a tile"), lane l holding block l%32.
// The k index of an MFMA is free to permute as long as A and B agree: k-step
// kb covers t = 16*kb + 8*(l/32) + i (i = 0..7).
// In the 32x32 accumulator, lane l holds, for its block, the 16 values
// j = 32*jt + 8q + 4*(l/32) + e (q, e = 0..3): one 32-group (jt) is split
// between lanes l and l+32, so its abs-max takes one v_permlane32_swap, and
// the same swap then trades 4-element runs so that each lane owns whole
// 16-byte pieces of output.
//
// Memory traffic: a lane of the MFMA layout touches one block, so reading or
// writing HBM in that layout scatters every instruction over 32 blocks.
// Instead each wave stages its tile through a private LDS buffer: the input
// is read from HBM fully coalesced (lane l, instruction q: 16-byte piece
// 64q + l of the tile), written to LDS, and read back in the MFMA layout; the
// outputs go the opposite way.  Pieces are placed with an XOR swizzle of
// their column so that both the linear and the per-block accesses are free
// of bank conflicts.
#include "launch.h"
#include "mx_device.h"

namespace mx {

// Entry (t, j) of the block-diagonal RB x RB matrix built from the r x r R.
template <typename T>
__device__ __forceinline__ T reff(const T *__restrict__ rot, int r, int t, int j) {
  if (t / r != j / r) return T(0);
  return rot[(t % r) * r + (j % r)];
}

constexpr int ilog2(int v) { return v <= 1 ? 0 : 1 + ilog2(v / 2); }

// LDS slot of 16-byte piece p of a tile whose blocks hold C pieces each: the
// low 3 bits of the piece index are XORed with bits of the block index so
// that eight consecutive blocks at the same column land in eight different
// 16-byte bank groups, and eight consecutive pieces stay a permutation of
// one aligned group of eight.
template <int C>
__device__ __forceinline__ int swz(int p) {
  constexpr int SH = C >= 8 ? ilog2(C) : 3;
  constexpr int MK = (C < 8 ? C : 8) - 1;
  return p ^ ((p >> SH) & MK);
}

// Orders a wave's LDS accesses around an exchange between its lanes.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  __builtin_amdgcn_wave_barrier();
}

// The MX step of one rotated 32-group held as acc[4q + e] =
// y[32*jt + 8q + 4h + e] by lanes l and l+32: scale byte, scale operand and
// the 4-element runs' codes c[q] (E2M1: 16 bits, E4M3: 32 bits).
template <int FMT>
__device__ __forceinline__ void group_codes(const f32x16 &acc, unsigned &sb, float &sc, unsigned c[4]) {
  float y[16];
#pragma unroll
  for (int a = 0; a < 16; ++a) y[a] = acc[a];
  const unsigned m = max_across_halves(abs_max_bits<16>(y));
  sb = scale_byte<FMT>(m);
  sc = scale_operand(sb);
  if (FMT == 1) {
    const float cl = __uint_as_float(((sb + 8u) << 23) | 0x600000u);  // 448 * 2^s
#pragma unroll
    for (int a = 0; a < 16; ++a) y[a] = clamp_f32(y[a], cl);
  }
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
}

// Dequantized bf16 of one group, rearranged across the lane pair: on return
// the lower lane holds elements 0-7 (o[0..3]) and 16-23 (o[4..7]) of the
// group, the upper lane 8-15 and 24-31.
template <int FMT>
__device__ __forceinline__ void group_bf16(const unsigned c[4], unsigned sb, float sc, unsigned o[8]) {
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
  swap_halves(o[0], o[2]);
  swap_halves(o[1], o[3]);
  swap_halves(o[4], o[6]);
  swap_halves(o[5], o[7]);
}

// NVFP4 on the same 32-wide tile: the tile's outputs j = 0-15 (acc[0..7] of
// lanes l and l+32) and j = 16-31 (acc[8..15]) are two 16-groups, each with
// its own E4M3 scale byte (sb[0], sb[1]); the codes come out as for E2M1
// (c[q]: 4 nibbles of elements 4q..4q+3 of this lane's run).
template <bool FAST>
__device__ __forceinline__ void nv_group_codes(const f32x16 &acc, const NvTensor &t, unsigned sb[2],
                                               float sbv[2], unsigned c[4]) {
#pragma unroll
  for (int hg = 0; hg < 2; ++hg) {
    float y[8];
#pragma unroll
    for (int a = 0; a < 8; ++a) y[a] = acc[8 * hg + a];
    const unsigned m = max_across_halves(abs_max_bits<8>(y));
    sb[hg] = nv_scale_byte(__uint_as_float(m) * t.c6);
    sbv[hg] = nv_scale_value(sb[hg]);
  }
  const float mul[2] = {nv_mul<FAST>(t, sbv[0]), nv_mul<FAST>(t, sbv[1])};
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const float mq = mul[q >> 1];
    unsigned v = fp4_from_f32x2<0>(0u, acc[4 * q] * mq, acc[4 * q + 1] * mq, 1.0f);
    c[q] = fp4_from_f32x2<1>(v, acc[4 * q + 2] * mq, acc[4 * q + 3] * mq, 1.0f);
  }
}

// Dequantized bf16 of the two 16-groups of a tile, arranged as group_bf16.
template <bool FAST>
__device__ __forceinline__ void nv_group_bf16(const unsigned c[4], const float sbv[2], const NvTensor &t,
                                              unsigned o[8]) {
  const float kf[2] = {nv_kf<FAST>(t, sbv[0]), nv_kf<FAST>(t, sbv[1])};
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    o[2 * q] = nv_bf16_pair<0>(c[q], kf[q >> 1]);
    o[2 * q + 1] = nv_bf16_pair<1>(c[q], kf[q >> 1]);
  }
  swap_halves(o[0], o[2]);
  swap_halves(o[1], o[3]);
  swap_halves(o[4], o[6]);
  swap_halves(o[5], o[7]);
}

// E2M1 codes of one group: on return the lower lane holds bytes 0-7 of the
// group's 16 code bytes (w[0], w[1]), the upper lane bytes 8-15.
__device__ __forceinline__ void group_fp4_bytes(const unsigned c[4], unsigned sb, unsigned w[2]) {
  // before the swap the lower lane holds the codes of j 0-3|8-11 (ca) and
  // 16-19|24-27 (cb), the upper lane those 4 elements later
  unsigned ca = c[0] | (c[1] << 16), cb = c[2] | (c[3] << 16);
  if (sb == 255u) ca = cb = 0u;
  swap_halves(ca, cb);
  // lower: ca = bytes {0-1, 4-5}, cb = {2-3, 6-7}; upper: {8-9, 12-13}, {10-11, 14-15}
  w[0] = (ca & 0xFFFFu) | (cb << 16);
  w[1] = (ca >> 16) | (cb & 0xFFFF0000u);
}

// E4M3 codes of one group: on return the lower lane holds bytes 0-15 of the
// group's 32 code bytes, the upper lane bytes 16-31.
__device__ __forceinline__ void group_fp8_bytes(const unsigned c[4], unsigned sb, unsigned r[4]) {
  r[0] = c[0];
  r[1] = c[1];
  r[2] = c[2];
  r[3] = c[3];
  if (sb == 255u) r[0] = r[1] = r[2] = r[3] = 0x7F7F7F7Fu;
  swap_halves(r[0], r[1]);  // lower: bytes 0-7,  upper: 8-15
  swap_halves(r[2], r[3]);  // lower: bytes 16-23, upper: 24-31
  swap_halves(r[0], r[2]);  // lower: 0-3 | 8-11, upper: 16-19 | 24-27
  swap_halves(r[1], r[3]);  // lower: 4-7 | 12-15, upper: 20-23 | 28-31
}

// bf16 source, OP_QDQ (bf16 out) or OP_QUANT, staged through LDS.
// FMT: 0 = MXFP4, 1 = MXFP8, 2 = NVFP4 (16-groups, E4M3 scales and the
// per-tensor multiplier *gp).
// SL (OP_QUANT only): 0 = row-major scales, 1 = the blocked layout `bl`.
// Launch shape of the 32-block staged kernels (k_rot_bf16): workgroup size,
// workgroups per CU in the grid (per_cu; per_cu_qdq for QDQ) and workgroups resident on a CU at
// once (resident).  LDS per workgroup is RB*RB*2 bytes of A fragments plus a
// 64*RB-byte tile buffer per wave; the launch pads it so that no more than
// `resident` fit in a CU's LDS, and the kernel's register budget lets that
// many fit (left to the register allocator, the residency changed from one
// build to the next).  Chosen by measurement on MI355X (8192 x 57344 bf16,
// QDQ and quantize): one resident workgroup (16 waves) for RB = 32 and two
// (16 waves) for RB = 64 run 2-3% faster than the 32 and 24 waves that fit
// otherwise.  For RB = 64 a grid of 32 per CU (about 3.5 tiles per wave) is
// fastest for quantize and 48 (about 2.3) for QDQ (per_cu_qdq; 1-2% faster
// than 32 for QDQ, 3-4% slower for blocked-scale quantize).  (RB = 128
// runs on k_rot_t16 and the lane-owned kernels.)
template <int RB> struct StagedCfg;
template <> struct StagedCfg<32> { static constexpr int threads = 1024, per_cu = 8, per_cu_qdq = 8, resident = 1; };
template <> struct StagedCfg<64> { static constexpr int threads = 512, per_cu = 32, per_cu_qdq = 48, resident = 2; };

constexpr int LDS_PER_CU = 160 * 1024;

// Static LDS of k_rot_bf16 at block size RB, and the dynamic LDS that the
// launch adds so that at most StagedCfg<RB>::resident workgroups fit a CU.
template <int RB> constexpr int staged_lds() {
  return (RB / 32) * (RB / 16) * 64 * 16 + (StagedCfg<RB>::threads / 64) * (32 * RB / 8) * 16;
}
template <int RB> constexpr int staged_lds_pad() {
  constexpr int need = LDS_PER_CU / (StagedCfg<RB>::resident + 1) + 1;
  static_assert(StagedCfg<RB>::resident * (need > staged_lds<RB>() ? need : staged_lds<RB>()) + 1024 <= LDS_PER_CU,
                "the resident workgroups fit");
  return need > staged_lds<RB>() ? need - staged_lds<RB>() : 0;
}

// Coalesced loads of one 32-block tile: piece 64q + lane.  Full tiles (all
// but possibly the last one) skip the per-piece bound (a wave-uniform test).
template <int RB>
__device__ __forceinline__ void rot_load_tile(const uint16_t *__restrict__ src, int64_t n_elem, int64_t tile,
                                              int lane, u32x4 (&v)[RB / 16]) {
  constexpr int NKB = RB / 16, TP = 32 * RB / 8;
  const int64_t e_tile = tile * 32 * RB;
  const u32x4 *g = (const u32x4 *)(src + e_tile) + lane;
  if (e_tile + (int64_t)TP * 8 <= n_elem) {
#pragma unroll
    for (int q = 0; q < NKB; ++q) v[q] = __builtin_nontemporal_load(g + q * 64);
  } else {
#pragma unroll
    for (int q = 0; q < NKB; ++q)
      v[q] = e_tile + (int64_t)(q * 64 + lane) * 8 < n_elem ? __builtin_nontemporal_load(g + q * 64)
                                                           : u32x4{0u, 0u, 0u, 0u};
  }
}

// The tile loop of k_rot_bf16, once R's fragments are in sA: each wave
// takes 32-block tiles (grid-stride), staging each through its LDS tile
// buffer T.  v holds the wave's first tile, loaded before R was staged.
// NVFAST selects the division-free NVFP4 quotients (nv_mul).
template <int FMT, int OP, int RB, int THREADS, int SL, bool NVFAST>
__device__ __forceinline__ void rot_tiles(const uint16_t *__restrict__ src, void *__restrict__ dst,
                                          uint8_t *__restrict__ codes, uint8_t *__restrict__ scales,
                                          int64_t n_blk, const BlockedScales &bl, float nv_g,
                                          const u32x4 *sA, u32x4 *T, u32x4 (&v)[RB / 16]) {
  constexpr int NJT = RB / 32, NKB = RB / 16;
  constexpr bool FP4 = FMT != 1;      // E2M1 codes (MXFP4 and NVFP4)
  constexpr int C = RB / 8;           // 16-byte input pieces per block
  constexpr int TP = 32 * C;          // input pieces per tile (= 64 * NKB)
  constexpr int WAVES = THREADS / 64;
  constexpr int C4 = RB / 32;         // E2M1 code pieces per block
  constexpr int C8 = RB / 16;         // E4M3 code pieces per block
  const int lane = threadIdx.x & 63, h = lane >> 5, n = lane & 31;
  const int64_t n_elem = n_blk * RB;
  const int64_t n_tiles = (n_blk + 31) / 32;
  const int64_t stride = (int64_t)gridDim.x * WAVES;

  NvTensor nvt{};
  if constexpr (FMT == 2) nvt = nv_tensor<NVFAST>(nv_g);
  int64_t tile = (int64_t)blockIdx.x * WAVES + (threadIdx.x >> 6);
  for (; tile < n_tiles; tile += stride) {
    const int64_t e_tile = tile * 32 * RB;  // first element of the tile
    const bool full = e_tile + (int64_t)TP * 8 <= n_elem;
    // 1. the tile into LDS
#pragma unroll
    for (int q = 0; q < NKB; ++q) T[swz<C>(q * 64 + lane)] = v[q];
    wave_lds_sync();
    // 2. B fragments in the MFMA layout
    u32x4 b[NKB];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) b[kb] = T[swz<C>(n * C + 2 * kb + h)];
    wave_lds_sync();
    // 3. rotate, quantize, and place the outputs in LDS
    const int64_t blk = tile * 32 + n;
    uint64_t sbw = 0;  // the block's scale bytes, in order
#pragma unroll
    for (int jt = 0; jt < NJT; ++jt) {
      f32x16 acc = {};
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, sA[(jt * NKB + kb) * 64 + lane]),
                                                      __builtin_bit_cast(bf16x8, b[kb]), acc, 0, 0, 0);
      {
        unsigned sb, c[4];
        float sc;
        unsigned o[8];
        if constexpr (FMT == 2) {
          unsigned sb2[2];
          float sbv[2];
          nv_group_codes<NVFAST>(acc, nvt, sb2, sbv, c);
          sb = 0u;  // never the NaN marker
          sbw |= (uint64_t)(sb2[0] | (sb2[1] << 8)) << (16 * jt);
          if (OP == OP_QDQ) nv_group_bf16<NVFAST>(c, sbv, nvt, o);
        } else {
          group_codes<FMT>(acc, sb, sc, c);
          sbw |= (uint64_t)sb << (8 * jt);
          if (OP == OP_QDQ) group_bf16<FMT>(c, sb, sc, o);
        }
        if (OP == OP_QDQ) {
          T[swz<C>(n * C + 4 * jt + h)] = u32x4{o[0], o[1], o[2], o[3]};
          T[swz<C>(n * C + 4 * jt + 2 + h)] = u32x4{o[4], o[5], o[6], o[7]};
        } else if (FP4) {
          unsigned w[2];
          group_fp4_bytes(c, sb, w);
          ((u32x2 *)T)[2 * swz<C4>(n * C4 + jt) + h] = u32x2{w[0], w[1]};
        } else {
          unsigned w[4];
          group_fp8_bytes(c, sb, w);
          T[swz<C8>(n * C8 + 2 * jt + h)] = u32x4{w[0], w[1], w[2], w[3]};
        }
      }
    }
    if (OP == OP_QUANT && SL == 1 && h == 0 && blk < n_blk) {
      // a block lies in one row: its groups are g0 .. g0 + NJT - 1
      const int64_t gf0 = blk * NJT, i = gf0 / bl.groups, g0 = gf0 - i * bl.groups;
#pragma unroll
      for (int jt = 0; jt < NJT; ++jt) scales[blocked_offset(i, g0 + jt, bl.gblocks)] = (uint8_t)(sbw >> (8 * jt));
    } else if (OP == OP_QUANT && FMT == 2 && h == 0 && blk < n_blk) {
      // RB/16 bytes per block
      if (NJT == 4) {
        *(unsigned *)(scales + blk * 8) = (unsigned)sbw;  // scales are 4-byte aligned
        *(unsigned *)(scales + blk * 8 + 4) = (unsigned)(sbw >> 32);
      }
      else if (NJT == 2) *(unsigned *)(scales + blk * 4) = (unsigned)sbw;
      else *(uint16_t *)(scales + blk * 2) = (uint16_t)sbw;
    } else if (OP == OP_QUANT && h == 0 && blk < n_blk) {
      if (NJT == 4) *(unsigned *)(scales + blk * 4) = (unsigned)sbw;
      else if (NJT == 2) *(uint16_t *)(scales + blk * 2) = (uint16_t)sbw;
      else scales[blk] = (uint8_t)sbw;
    }
    wave_lds_sync();
    // 4. coalesced stores of the tile's outputs
    if (OP == OP_QDQ) {
      u32x4 *g = (u32x4 *)((uint16_t *)dst + e_tile) + lane;
      u32x4 o[NKB];
#pragma unroll
      for (int q = 0; q < NKB; ++q) o[q] = T[swz<C>(q * 64 + lane)];
      if (full) {
#pragma unroll
        for (int q = 0; q < NKB; ++q) __builtin_nontemporal_store(o[q], g + q * 64);
      } else {
#pragma unroll
        for (int q = 0; q < NKB; ++q)
          if (e_tile + (int64_t)(q * 64 + lane) * 8 < n_elem) __builtin_nontemporal_store(o[q], g + q * 64);
      }
    } else {
      constexpr int CP = FP4 ? C4 : C8;           // code pieces per block
      constexpr int EPP = FP4 ? 32 : 16;          // elements per code piece
      constexpr int NQ = (32 * CP + 63) / 64;
      u32x4 *g = (u32x4 *)(codes + e_tile / EPP * 16) + lane;
      u32x4 o[NQ];
#pragma unroll
      for (int q = 0; q < NQ; ++q) o[q] = (q * 64 + lane < 32 * CP) ? T[swz<CP>(q * 64 + lane)] : u32x4{};
#pragma unroll
      for (int q = 0; q < NQ; ++q) {
        const int p = q * 64 + lane;
        if (p < 32 * CP && (full || e_tile + (int64_t)p * EPP < n_elem)) __builtin_nontemporal_store(o[q], g + q * 64);
      }
    }
    wave_lds_sync();
    if (tile + stride < n_tiles) rot_load_tile<RB>(src, n_elem, tile + stride, lane, v);
  }
}

template <int FMT, int OP, int RB, int THREADS, int SL>
__global__ __launch_bounds__(THREADS)
__attribute__((amdgpu_waves_per_eu(StagedCfg<RB>::resident * THREADS / 256))) void k_rot_bf16(const uint16_t *__restrict__ src,
                                                      const uint16_t *__restrict__ rot, int r,
                                                      void *__restrict__ dst, uint8_t *__restrict__ codes,
                                                      uint8_t *__restrict__ scales, int64_t n_blk,
                                                      BlockedScales bl, const float *__restrict__ gp) {
  constexpr int NJT = RB / 32, NKB = RB / 16;
  constexpr int TP = 32 * RB / 8;     // 16-byte input pieces per tile
  constexpr int WAVES = THREADS / 64;
  __shared__ u32x4 sA[NJT * NKB * 64];
  __shared__ u32x4 sT[WAVES][TP];
  static_assert(THREADS != StagedCfg<RB>::threads || sizeof(sA) + sizeof(sT) == staged_lds<RB>(), "LDS size");

  // R (r*r <= RB*RB bf16) is first copied into the tile buffers with
  // coalesced 16-byte loads, all in flight at once; the fragments are then
  // gathered from LDS.
  static_assert(sizeof(sT) >= RB * RB * 2, "R is staged in the tile buffers");
  // The wave's first tile is loaded right behind R, so that its latency
  // overlaps R's staging: with the grid covering the tensor once (the
  // smaller layers), a wave has one or two tiles in all.
  u32x4 v[NKB];
  {
    constexpr int RP = (RB * RB / 8 + THREADS - 1) / THREADS;  // 16-byte pieces per thread
    const int pieces = r * r / 8;
    u32x4 rv[RP];
#pragma unroll
    for (int k = 0; k < RP; ++k) {
      const int i = threadIdx.x + k * THREADS;
      if (i < pieces) rv[k] = ((const u32x4 *)rot)[i];
    }
    const int64_t tile0 = (int64_t)blockIdx.x * WAVES + (threadIdx.x >> 6);
    if (tile0 < (n_blk + 31) / 32) rot_load_tile<RB>(src, n_blk * RB, tile0, threadIdx.x & 63, v);
#pragma unroll
    for (int k = 0; k < RP; ++k) {
      const int i = threadIdx.x + k * THREADS;
      if (i < pieces) (&sT[0][0])[i] = rv[k];
    }
  }
  __syncthreads();
  if (SL == 1)
    write_blocked_pads(scales, bl, (int64_t)blockIdx.x * THREADS + threadIdx.x, (int64_t)gridDim.x * THREADS);
  const uint16_t *Rs = (const uint16_t *)&sT[0][0];
  // A fragment (jt, kb) of lane ln: Reff[t][j] for j = 32*jt + ln%32 and
  // t = 16*kb + 8*(ln/32) + i, i = 0..7.
  for (int idx = threadIdx.x; idx < NJT * NKB * 64; idx += THREADS) {
    const int ln = idx & 63, f = idx >> 6, jt = f / NKB, kb = f % NKB;
    const int j = jt * 32 + (ln & 31), t0 = 16 * kb + 8 * (ln >> 5);
    unsigned w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      w[i] = (unsigned)reff(Rs, r, t0 + 2 * i, j) | ((unsigned)reff(Rs, r, t0 + 2 * i + 1, j) << 16);
    sA[idx] = u32x4{w[0], w[1], w[2], w[3]};
  }
  __syncthreads();

  u32x4 *T = sT[threadIdx.x >> 6];
  if constexpr (FMT == 2) {
    // one instance of the tile loop per range of g (see nv_mul)
    const float g = *gp;
    if (nv_fast(g)) rot_tiles<FMT, OP, RB, THREADS, SL, true>(src, dst, codes, scales, n_blk, bl, g, sA, T, v);
    else rot_tiles<FMT, OP, RB, THREADS, SL, false>(src, dst, codes, scales, n_blk, bl, g, sA, T, v);
  } else {
    rot_tiles<FMT, OP, RB, THREADS, SL, true>(src, dst, codes, scales, n_blk, bl, 0.0f, sA, T, v);
  }
}

// ---------------------------------------------------------------------------
// RB = 64 and 128 on 16-block tiles (2 or 4 KiB per wave) with
// v_mfma_f32_16x16x32_bf16.
//
// Streaming whole 8 KiB tiles per wave (32 blocks, the 32x32 layout above)
// is slower on this GPU than 4 KiB ones: a persistent copy with the same
// sweep runs at 5.8 TB/s with 8 KiB per wave and 6.1 TB/s with 4 KiB.  The
// 16x16x32 MFMA needs only 16 blocks per tile.  Y^T = Reff^T . X^T with
// m = output j (16 per jt, RB/16 jt), k = t (32 per kb, RB/32 kb),
// n = block:
//   lane l = 16p + n;  B fragment kb: x[block n][t = 32kb + 8p + i];
//   A fragment (jt, kb): Reff[32kb + 8p + i][16jt + n], i = 0..7;
//   accumulator jt: y[block n][j = 16jt + 4p + i], i = 0..3.
// The 32-group g is jt 2g and 2g+1: lane l holds its elements 4p..4p+3
// ("run a") and 16+4p..16+4p+3 ("run b"), and the group spans lanes n,
// n+16, n+32, n+48 (two lane swaps reduce the abs-max).  MX formats only.
// LDS: a tile is 16 blocks x RB/8 pieces of 16 bytes, XOR-swizzled (tslot)
// so that the fragment reads (16 lanes, one block each, same piece) and the
// coalesced accesses (a block's pieces in consecutive lanes) are both free
// of bank conflicts.

// Max of v over lanes l, l^16, l^32 and l^48.
__device__ __forceinline__ unsigned max_across_quarters(unsigned v) {
  auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  return max_across_halves(umax(r[0], r[1]));
}

// The MX step of one 32-group in the 16x16 layout: scale byte, scale
// operand and the codes of run a and run b (E2M1: 16 bits, E4M3: 32 bits).
template <int FMT>
__device__ __forceinline__ void group16_codes(const f32x4 &a, const f32x4 &b, unsigned &sb, float &sc,
                                              unsigned &ca, unsigned &cb) {
  const float ab[8] = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  const unsigned m = max_across_quarters(abs_max_bits<8>(ab));
  sb = scale_byte<FMT>(m);
  sc = scale_operand(sb);
  float ya[4], yb[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    ya[i] = a[i];
    yb[i] = b[i];
  }
  if (FMT == 1) {
    const float cl = __uint_as_float(((sb + 8u) << 23) | 0x600000u);  // 448 * 2^s
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      ya[i] = clamp_f32(ya[i], cl);
      yb[i] = clamp_f32(yb[i], cl);
    }
  }
  if (FMT == 0) {
    ca = fp4_from_f32x2<1>(fp4_from_f32x2<0>(0u, ya[0], ya[1], sc), ya[2], ya[3], sc);
    cb = fp4_from_f32x2<1>(fp4_from_f32x2<0>(0u, yb[0], yb[1], sc), yb[2], yb[3], sc);
  } else {
    ca = fp8_from_f32x2<true>(fp8_from_f32x2<false>(0u, ya[0], ya[1], sc), ya[2], ya[3], sc);
    cb = fp8_from_f32x2<true>(fp8_from_f32x2<false>(0u, yb[0], yb[1], sc), yb[2], yb[3], sc);
  }
}

// bf16 of a run's 4 codes (8 bytes): E2M1 16 bits or E4M3 32 bits.
template <int FMT>
__device__ __forceinline__ u32x2 run_bf16(unsigned c, float sc) {
  if (FMT == 0)
    return u32x2{__builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(c, sc, 0)),
                 __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(c, sc, 1))};
  return u32x2{__builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c, sc, false)),
               __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c, sc, true))};
}

// Launch shape of the 16-block kernel: threads per workgroup, the waves per
// SIMD the register budget is compiled for, tiles per wave and tiles kept in
// registers ahead of the one a wave works on.  RB = 128: three workgroups
// fit a CU's LDS (32 KiB of A fragments plus a 4 KiB tile per wave each).
// RB = 128: four tiles per wave, three of them in registers ahead (bench-
// style blocks on the 8192 x 57344 layer: 303-306 us against 309-313 with
// 8 and 4, 313-327 with 2, 3, 5, 6 or 12 tiles per wave).
// RB = 64 (2 KiB tiles): one tile per wave, the shortest-lived workgroups,
// measured fastest on the 8192 x 57344 layer (MXFP4 QDQ at r = 16, 32:
// 295 and 293 us, against 299-300 with two tiles per wave, 305-321 with
// four, 313-356 with 8 to 32).
template <int RB> struct T16Cfg;
template <> struct T16Cfg<128> {
  static constexpr int threads = 256, waves_per_simd = 3, tpw = 4, nr = 3;
};
template <> struct T16Cfg<64> {
  static constexpr int threads = 256, waves_per_simd = 4, tpw = 1, nr = 1;
};

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

// Slot of piece c of block n in a tile buffer of PPB (16 or 8) pieces per
// block: the XOR key n / (16 / PPB) makes the 16 blocks of a fragment read
// (same c) and a block's PPB pieces in consecutive lanes fall on distinct
// 16-byte bank groups of a 256-byte LDS row.
template <int PPB>
__device__ __forceinline__ int tslot(int n, int c) { return PPB * n + (c ^ ((n / (16 / PPB)) & (PPB - 1))); }

// Slot of piece c of row t of Reff staged in LDS (PPB pieces per row): the
// key 2 (t % 4) puts the two pieces that a transposed fragment read takes
// from each of four consecutive rows into eight different 16-byte bank
// groups (unswizzled, rows 256 or 128 bytes apart share their banks).
template <int PPB>
__device__ __forceinline__ int rslot(int t, int c) { return PPB * t + (c ^ (2 * (t & 3))); }

// MX QDQ (bf16 in and out) with a rotation block of RB = 64 or 128 on
// 16-block tiles.  A short-lived workgroup: Reff (row-major RB x RB bf16;
// for r < RB the block-diagonal diag(R, ..., R)) is formed in LDS, the A
// fragments are formed from it with transposed reads (ds_read_b64_tr_b16:
// within each 16-lane group, lane i receives element i%4 of the 8 bytes
// that lanes 4r + i/4 address, r = 0..3, so when lane j addresses row
// t0 + j/4 at column j0 + 4(j%4), lane i receives column j0 + i of rows
// t0 .. t0+3), and the waves then stream their tiles.  The grid covers the
// tensor once (up to a cap beyond which workgroups loop), so the hardware
// dispatcher balances the work across CUs.
template <int FMT, int RB>
__global__ __launch_bounds__(T16Cfg<RB>::threads) __attribute__((amdgpu_waves_per_eu(T16Cfg<RB>::waves_per_simd)))
void k_rot_t16(const uint16_t *__restrict__ src, const uint16_t *__restrict__ rot, int r,
               uint16_t *__restrict__ dst, int64_t n_blk) {
  static_assert(FMT == 0 || FMT == 1, "MX formats");
  using Cfg = T16Cfg<RB>;
  constexpr int THREADS = Cfg::threads, TPW = Cfg::tpw, NR = Cfg::nr;
  constexpr int NJT = RB / 16, NKB = RB / 32, TB = 16;  // 16-wide j tiles, 32-deep k steps, blocks per tile
  constexpr int PPB = RB / 8;                       // 16-byte pieces per block
  constexpr int TP = TB * PPB;                      // 16-byte input pieces per tile
  constexpr int NL = TP / 64;                       // coalesced pieces per lane
  constexpr int WAVES = THREADS / 64;
  constexpr int RP = RB * RB / 8 / THREADS;         // 16-byte pieces of Reff per thread
  constexpr int JPW = NJT * NKB / WAVES;            // A fragments (j tiles) a wave forms
  static_assert(WAVES % NKB == 0 && JPW * WAVES == NJT * NKB && RP * THREADS * 8 == RB * RB && NR <= TPW,
                "each wave forms the fragments of one k step and a whole share of the j tiles");
  __shared__ u32x4 sA[NJT * NKB * 64];
  __shared__ u32x4 sT[WAVES][TP];
  static_assert(sizeof(sA) == RB * RB * 2, "Reff is staged in the fragment buffer");

  const int lane = threadIdx.x & 63, p = lane >> 4, n = lane & 15, wave = threadIdx.x >> 6;
  const int64_t n_elem = n_blk * RB;
  const int64_t n_tiles = (n_blk + TB - 1) / TB;
  const int64_t n_units = (n_tiles + WAVES * TPW - 1) / (WAVES * TPW);

  // coalesced loads of one tile: lane piece 64q + lane (block (64q+lane)/PPB)
  auto load_tile = [&](int64_t tile, u32x4 *v) {
    const int64_t e_tile = tile * TB * RB;
    const u32x4 *gs = (const u32x4 *)(src + e_tile) + lane;
    if (e_tile + (int64_t)TP * 8 <= n_elem) {
#pragma unroll
      for (int q = 0; q < NL; ++q) v[q] = __builtin_nontemporal_load(gs + q * 64);
    } else {
#pragma unroll
      for (int q = 0; q < NL; ++q)
        v[q] = e_tile + (int64_t)(q * 64 + lane) * 8 < n_elem ? __builtin_nontemporal_load(gs + q * 64)
                                                             : u32x4{0u, 0u, 0u, 0u};
    }
  };

  // Reff and the first NR tiles of this wave, all loads in flight at once.
  // Piece x of Reff is row x / PPB, columns 8 (x % PPB) .. +7: inside the
  // diagonal block of its row it is piece (t % r) r/8 + (j % r)/8 of R,
  // elsewhere zero (r is a multiple of 16, so no piece straddles a block).
  int64_t unit = blockIdx.x;
  u32x4 v[NR][NL];
  {
    u32x4 rv[RP];
    const int rs = __builtin_ctz(r);  // r is a power of two
#pragma unroll
    for (int k = 0; k < RP; ++k) {
      const int x = threadIdx.x + k * THREADS, t = x / PPB, j = 8 * (x % PPB);
      if (RB == 128 || r == RB)
        rv[k] = ((const u32x4 *)rot)[x];
      else
        rv[k] = (t >> rs) == (j >> rs) ? ((const u32x4 *)rot)[((t & (r - 1)) << (rs - 3)) + ((j & (r - 1)) >> 3)]
                                       : u32x4{0u, 0u, 0u, 0u};
    }
    const int64_t t0 = (unit * WAVES + wave) * TPW;
#pragma unroll
    for (int t = 0; t < NR; ++t)
      if (t0 + t < n_tiles) load_tile(t0 + t, v[t]);
#pragma unroll
    for (int k = 0; k < RP; ++k) {
      const int x = threadIdx.x + k * THREADS;
      sA[rslot<PPB>(x / PPB, x % PPB)] = rv[k];
    }
  }
  __syncthreads();
  {
    // A fragment (jt, kb) of lane 16p + n: Reff[32kb + 8p + i][16jt + n],
    // i = 0..7.  Wave w forms those of kb = w % NKB, jt = j0 .. j0+JPW-1.
    // Lane n reads 8 bytes at column 16jt + 4 (n % 4): piece 2jt + (n % 4) / 2,
    // half n % 2, of rows `row` and `row` + 4 (the same key).
    const uint16_t *Rs = (const uint16_t *)sA;
    const int kbw = wave % NKB, j0 = (wave / NKB) * JPW;
    const int row = 32 * kbw + 8 * p + (n >> 2);
    u32x4 fa[JPW];
#pragma unroll
    for (int j = 0; j < JPW; ++j) {
      const int c0 = 8 * (rslot<PPB>(row, 2 * (j0 + j) + ((n & 3) >> 1)) - PPB * row) + 4 * (n & 1);
      const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(Rs + row * RB + c0));
      const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(Rs + (row + 4) * RB + c0));
      const u32x2 a = __builtin_bit_cast(u32x2, lo), b = __builtin_bit_cast(u32x2, hi);
      fa[j] = u32x4{a[0], a[1], b[0], b[1]};
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < JPW; ++j) sA[((j0 + j) * NKB + kbw) * 64 + lane] = fa[j];
  }
  __syncthreads();

  u32x4 *T = sT[wave];
  for (;;) {
    const int64_t t0 = (unit * WAVES + wave) * TPW;
#pragma unroll
    for (int t = 0; t < TPW; ++t) {
      const int64_t tile = t0 + t;
      if (tile >= n_tiles) break;
      const int64_t e_tile = tile * TB * RB;
      const bool full = e_tile + (int64_t)TP * 8 <= n_elem;
      // 1. the tile into LDS (piece P = 64q + lane is block P/PPB, piece P%PPB)
#pragma unroll
      for (int q = 0; q < NL; ++q) T[tslot<PPB>((64 * q + lane) / PPB, lane % PPB)] = v[t % NR][q];
      wave_lds_sync();
      // 2. B fragments: block n, pieces 4kb + p
      u32x4 b[NKB];
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) b[kb] = T[tslot<PPB>(n, 4 * kb + p)];
      wave_lds_sync();
      // 3. rotate and QDQ, one 32-group (jt 2g, 2g+1) at a time
#pragma unroll
      for (int gq = 0; gq < NJT / 2; ++gq) {
        f32x4 acc[2] = {f32x4{}, f32x4{}};
#pragma unroll
        for (int hh = 0; hh < 2; ++hh)
#pragma unroll
          for (int kb = 0; kb < NKB; ++kb)
            acc[hh] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                __builtin_bit_cast(bf16x8, sA[((2 * gq + hh) * NKB + kb) * 64 + lane]),
                __builtin_bit_cast(bf16x8, b[kb]), acc[hh], 0, 0, 0);
        unsigned sb, ca, cb;
        float sc;
        group16_codes<FMT>(acc[0], acc[1], sb, sc, ca, cb);
        u32x2 oa = run_bf16<FMT>(ca, sc), ob = run_bf16<FMT>(cb, sc);
        if (sb == 255u) oa = ob = u32x2{BF16_NAN | (BF16_NAN << 16), BF16_NAN | (BF16_NAN << 16)};
        // run a: elements 32gq + 4p.. = piece 4gq + p/2, half p%2; run b: 2 pieces on
        ((u32x2 *)T)[2 * tslot<PPB>(n, 4 * gq + (p >> 1)) + (p & 1)] = oa;
        ((u32x2 *)T)[2 * tslot<PPB>(n, 4 * gq + 2 + (p >> 1)) + (p & 1)] = ob;
      }
      wave_lds_sync();
      // 4. coalesced stores of the tile's outputs
      u32x4 *gd = (u32x4 *)(dst + e_tile) + lane;
      u32x4 o[NL];
#pragma unroll
      for (int q = 0; q < NL; ++q) o[q] = T[tslot<PPB>((64 * q + lane) / PPB, lane % PPB)];
      if (full) {
#pragma unroll
        for (int q = 0; q < NL; ++q) __builtin_nontemporal_store(o[q], gd + q * 64);
      } else {
#pragma unroll
        for (int q = 0; q < NL; ++q)
          if (e_tile + (int64_t)(q * 64 + lane) * 8 < n_elem) __builtin_nontemporal_store(o[q], gd + q * 64);
      }
      wave_lds_sync();
      // the tile NR ahead into the registers just freed (issued after this
      // tile's stores, so waiting for it never waits for them)
      if (t + NR < TPW && tile + NR < n_tiles) load_tile(tile + NR, v[t % NR]);
    }
    unit += gridDim.x;
    if (unit >= n_units) break;
    const int64_t t1 = (unit * WAVES + wave) * TPW;
    for (int t = 0; t < NR; ++t)
      if (t1 + t < n_tiles) load_tile(t1 + t, v[t]);
  }
}

// The rotation alone (fp32 out) or fp32 sources: direct stores.
// For bf16 sources the B layout is the one above; for fp32 sources
// v_mfma_f32_32x32x2_f32 takes one value per lane: lane l supplies
// B[k = l/32][n = l%32] and A[m = l%32][k = l/32], and k-step kb covers
// t = (l/32)*RB/2 + kb.
// The fp32 outputs of one accumulator: o[q] = elements 8q + 4h .. +3 of the
// block's 32 columns (the rotated values, or their QDQ by exact software
// decode of the hardware codes).
template <int FMT, int OP>
__device__ __forceinline__ void direct_values(const f32x16 &acc, f32x4 (&o)[4]) {
  if (OP == OP_ROTATE) {
#pragma unroll
    for (int q = 0; q < 4; ++q) o[q] = f32x4{acc[4 * q], acc[4 * q + 1], acc[4 * q + 2], acc[4 * q + 3]};
    return;
  }
  unsigned sb, c[4];
  float sc;
  group_codes<FMT>(acc, sb, sc, c);
  const int s = (int)sb - 127;
  constexpr int CB = FMT == 0 ? 4 : 8;
  constexpr unsigned CM = (1u << CB) - 1u;
#pragma unroll
  for (int q = 0; q < 4; ++q)
#pragma unroll
    for (int e = 0; e < 4; ++e)
      o[q][e] = sb == 255u ? __uint_as_float(F32_NAN) : decode_code<FMT>((c[q] >> (CB * e)) & CM, s);
}

template <int FMT, int OP, int RB>
__device__ __forceinline__ void store_direct(const f32x16 &acc, int64_t blk, int jt, int h, bool valid,
                                             void *__restrict__ dst) {
  const int64_t e0 = blk * RB + jt * 32;
  float *d = (float *)dst + e0 + 4 * h;
  if (OP == OP_ROTATE) {
    if (valid) {
#pragma unroll
      for (int q = 0; q < 4; ++q)
        *(f32x4 *)(d + 8 * q) = f32x4{acc[4 * q], acc[4 * q + 1], acc[4 * q + 2], acc[4 * q + 3]};
    }
    return;
  }
  // fp32 QDQ: exact software decode of the hardware codes
  unsigned sb, c[4];
  float sc;
  group_codes<FMT>(acc, sb, sc, c);
  const int s = (int)sb - 127;
  constexpr int CB = FMT == 0 ? 4 : 8;
  constexpr unsigned CM = (1u << CB) - 1u;
  if (valid) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      f32x4 v;
#pragma unroll
      for (int e = 0; e < 4; ++e)
        v[e] = sb == 255u ? __uint_as_float(F32_NAN) : decode_code<FMT>((c[q] >> (CB * e)) & CM, s);
      *(f32x4 *)(d + 8 * q) = v;
    }
  }
}

constexpr int DTHREADS = 256;

// fp32 sources: the rotation on v_mfma_f32_32x32x2_f32, whose A and B
// operands are one value per lane (layout above).  A workgroup's four waves
// share steps of 16 KiB of input (TPS tiles of 32 blocks): wave w takes
// output columns 32 (w % NCG) .. +31 of tile w / NCG, so it holds only those
// columns of Reff, in registers (RB/2 values per lane), and one wave owns
// each 32-group.  The input is loaded fully coalesced (1 KiB per
// instruction) into one of two LDS step buffers, the next step's loads in
// flight while the current one is rotated; lanes read their block's run
// back 16 bytes at a time (four k-steps).  Pieces are XOR-swizzled so that
// both the coalesced writes and the per-block reads are free of bank
// conflicts.  Outputs go out from the MFMA layout (store_direct).
template <int PPB>
__device__ __forceinline__ int fslot(int b, int c) {
  constexpr int BPR = PPB >= 16 ? 1 : 16 / PPB;  // blocks per 256-byte LDS row
  constexpr int KM = PPB >= 16 ? 15 : PPB - 1;
  return PPB * b + (c ^ ((b / BPR) & KM));
}

template <int FMT, int OP, int RB>
__global__ __launch_bounds__(DTHREADS) void k_rot_f32(const float *__restrict__ src,
                                                      const float *__restrict__ rot, int r,
                                                      void *__restrict__ dst, int64_t n_blk) {
  constexpr int NCG = RB / 32, TPS = (DTHREADS / 64) / NCG, HALF = RB / 2;
  constexpr int PPB = RB / 4;                 // 16-byte pieces per block
  constexpr int SP = TPS * 32 * PPB;          // pieces per step (1024: 16 KiB)
  constexpr int NLD = SP / DTHREADS;          // pieces each thread loads per step
  static_assert(NLD * DTHREADS == SP && TPS * NCG * 64 == DTHREADS, "whole steps");
  __shared__ f32x4 buf[2][SP];
  // RB <= 64: each wave's outputs go out through LDS in whole 128-byte
  // column runs (3% faster there; at RB = 128 the extra registers cost more)
  constexpr bool OSTAGE = RB <= 64;
  __shared__ f32x4 obuf[OSTAGE ? DTHREADS / 64 : 1][OSTAGE ? 256 : 1];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, h = lane >> 5, n = lane & 31;
  const int cg = wave % NCG, tw = wave / NCG;
  const int64_t n_steps = (n_blk + 32 * TPS - 1) / (32 * TPS);
  const int64_t n_pieces = n_blk * PPB;
  int64_t step = blockIdx.x;
  if (step >= n_steps) return;  // (the whole workgroup)

  auto load_step = [&](int64_t st, f32x4 *v) {
    const f32x4 *g = (const f32x4 *)src + st * SP + threadIdx.x;
#pragma unroll
    for (int q = 0; q < NLD; ++q)
      v[q] = st * SP + q * DTHREADS + threadIdx.x < n_pieces ? __builtin_nontemporal_load(g + q * DTHREADS)
                                                             : f32x4{0.f, 0.f, 0.f, 0.f};
  };
  auto stage = [&](f32x4 *b, const f32x4 *v) {
#pragma unroll
    for (int q = 0; q < NLD; ++q) {
      const int P = q * DTHREADS + threadIdx.x;
      b[fslot<PPB>(P / PPB, P % PPB)] = v[q];
    }
  };

  f32x4 v[NLD];
  load_step(step, v);
  // this wave's columns of Reff: ra[kb] = Reff[h HALF + kb][32 cg + n]
  float ra[HALF];
#pragma unroll
  for (int kb = 0; kb < HALF; ++kb) ra[kb] = reff(rot, r, h * HALF + kb, 32 * cg + n);
  stage(buf[0], v);
  __syncthreads();
  for (int cur = 0;; cur ^= 1) {
    const int64_t next = step + gridDim.x;
    if (next < n_steps) load_step(next, v);
    const f32x4 *b = buf[cur];
    f32x16 acc = {};
#pragma unroll
    for (int k4 = 0; k4 < HALF / 4; ++k4) {
      const f32x4 x4 = b[fslot<PPB>(32 * tw + n, h * (HALF / 4) + k4)];
#pragma unroll
      for (int k = 0; k < 4; ++k) acc = __builtin_amdgcn_mfma_f32_32x32x2f32(ra[4 * k4 + k], x4[k], acc, 0, 0, 0);
    }
    if constexpr (OSTAGE) {
      // piece 2q + h of block n in the wave's buffer (keyed like tslot),
      // then 8 blocks' column runs per store instruction
      f32x4 o[4];
      direct_values<FMT, OP>(acc, o);
      f32x4 *ob = obuf[wave];
#pragma unroll
      for (int q = 0; q < 4; ++q) ob[8 * n + ((2 * q + h) ^ ((n >> 1) & 7))] = o[q];
      wave_lds_sync();
      const int64_t blk0 = step * 32 * TPS + 32 * tw;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int P = 64 * i + lane, bn = P >> 3, c = P & 7;
        const f32x4 w = ob[8 * bn + (c ^ ((bn >> 1) & 7))];
        if (blk0 + bn < n_blk) *((f32x4 *)((float *)dst + (blk0 + bn) * RB + 32 * cg) + c) = w;
      }
      wave_lds_sync();
    } else {
      const int64_t blk = step * 32 * TPS + 32 * tw + n;
      store_direct<FMT, OP, RB>(acc, blk, cg, h, blk < n_blk, dst);
    }
    if (next >= n_steps) break;
    stage(buf[cur ^ 1], v);  // buf[cur ^ 1] was last read before the previous barrier
    __syncthreads();
    step = next;
  }
}


// The rotation alone of bf16 sources (fp32 out), on the same plan as the
// fp32-source kernel above: a workgroup's four waves share steps of 8 KiB
// of input (TPS tiles of 32 blocks), loaded coalesced into one of two
// swizzled LDS buffers with the next step's loads in flight; wave w keeps
// the MFMA fragments of its 32 output columns of Reff in registers and reads
// its block's 16 bytes per k-step back (32x32x16 layout: k-step kb covers
// t = 16 kb + 8 (l/32) + i).
template <int RB>
__global__ __launch_bounds__(DTHREADS) void k_rotate_bf16(const uint16_t *__restrict__ src,
                                                          const uint16_t *__restrict__ rot, int r,
                                                          float *__restrict__ dst, int64_t n_blk) {
  constexpr int NCG = RB / 32, TPS = (DTHREADS / 64) / NCG, NKB = RB / 16;
  constexpr int PPB = RB / 8;                 // 16-byte pieces per block
  constexpr int SP = TPS * 32 * PPB;          // pieces per step (512: 8 KiB)
  constexpr int NLD = SP / DTHREADS;
  static_assert(NLD * DTHREADS == SP && TPS * NCG * 64 == DTHREADS, "whole steps");
  __shared__ u32x4 buf[2][SP];
  __shared__ f32x4 obuf[DTHREADS / 64][256];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, h = lane >> 5, n = lane & 31;
  const int cg = wave % NCG, tw = wave / NCG;
  const int64_t n_steps = (n_blk + 32 * TPS - 1) / (32 * TPS);
  const int64_t n_pieces = n_blk * PPB;
  int64_t step = blockIdx.x;
  if (step >= n_steps) return;  // (the whole workgroup)

  auto load_step = [&](int64_t st, u32x4 *v) {
    const u32x4 *g = (const u32x4 *)src + st * SP + threadIdx.x;
#pragma unroll
    for (int q = 0; q < NLD; ++q)
      v[q] = st * SP + q * DTHREADS + threadIdx.x < n_pieces ? __builtin_nontemporal_load(g + q * DTHREADS)
                                                             : u32x4{0u, 0u, 0u, 0u};
  };
  auto stage = [&](u32x4 *b, const u32x4 *v) {
#pragma unroll
    for (int q = 0; q < NLD; ++q) {
      const int P = q * DTHREADS + threadIdx.x;
      b[fslot<PPB>(P / PPB, P % PPB)] = v[q];
    }
  };

  u32x4 v[NLD];
  load_step(step, v);
  // A fragments of this wave's columns: Reff[16 kb + 8h + i][32 cg + n]
  u32x4 ra[NKB];
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb) {
    const int t0 = 16 * kb + 8 * h, j = 32 * cg + n;
    unsigned w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      w[i] = (unsigned)reff(rot, r, t0 + 2 * i, j) | ((unsigned)reff(rot, r, t0 + 2 * i + 1, j) << 16);
    ra[kb] = u32x4{w[0], w[1], w[2], w[3]};
  }
  stage(buf[0], v);
  __syncthreads();
  for (int cur = 0;; cur ^= 1) {
    const int64_t next = step + gridDim.x;
    if (next < n_steps) load_step(next, v);
    const u32x4 *b = buf[cur];
    f32x16 acc = {};
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, ra[kb]),
                                                    __builtin_bit_cast(bf16x8, b[fslot<PPB>(32 * tw + n, 2 * kb + h)]),
                                                    acc, 0, 0, 0);
    {
      // outputs through the wave's LDS buffer, then 8 blocks' whole 128-byte
      // column runs per store instruction
      f32x4 *ob = obuf[wave];
#pragma unroll
      for (int q = 0; q < 4; ++q)
        ob[8 * n + ((2 * q + h) ^ ((n >> 1) & 7))] = f32x4{acc[4 * q], acc[4 * q + 1], acc[4 * q + 2], acc[4 * q + 3]};
      wave_lds_sync();
      const int64_t blk0 = step * 32 * TPS + 32 * tw;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int P = 64 * i + lane, bn = P >> 3, c = P & 7;
        const f32x4 w = ob[8 * bn + (c ^ ((bn >> 1) & 7))];
        if (blk0 + bn < n_blk) *((f32x4 *)(dst + (blk0 + bn) * RB + 32 * cg) + c) = w;
      }
      wave_lds_sync();
    }
    if (next >= n_steps) break;
    stage(buf[cur ^ 1], v);  // buf[cur ^ 1] was last read before the previous barrier
    __syncthreads();
    step = next;
  }
}

static unsigned persistent_grid(int64_t tiles, int waves, int per_cu) {
  int64_t g = (tiles + waves - 1) / waves;
  const int64_t cap = (int64_t)device_cu_count() * per_cu;
  return (unsigned)(g < cap ? g : cap);
}

// MX QDQ runs on 16-block tiles (k_rot_t16, one workgroup per tpw tiles of
// each of its waves) at RB = 128, and at RB = 64 when r < 64: there each
// workgroup forms Reff from a half or a quarter of R's bytes (the rest are
// the block-diagonal's zeros).  Measured on the 8192 x 57344 layer, bench-
// style blocks of 20 launches: r = 16 307 -> 295 us, r = 32 303 -> 293 us
// against the 32-block tiles here, but r = 64, whose workgroups each read
// all of R, 300 -> 302-304 us, so r = 64 stays on the 32-block tiles.
// Quantize (whose outputs are a quarter of QDQ's) and NVFP4 at RB = 128 run
// on the lane-owned kernel, and at RB = 32 and 64 on the 32-block tiles.

template <int FMT, int OP, int RB>
static void run_staged(const void *src, const void *rot, int r, void *dst, uint8_t *codes, uint8_t *scales,
                       int64_t n, hipStream_t st, const BlockedScales *bl, const float *gp = nullptr) {
  const int64_t n_blk = n / RB;
  if constexpr ((RB == 128 || RB == 64) && FMT != 2 && OP == OP_QDQ) {
    if (RB == 128 || r < 64) {
      using Cfg = T16Cfg<RB>;
      constexpr int64_t per_unit = (Cfg::threads / 64) * Cfg::tpw;  // tiles per workgroup
      const int64_t units = ((n_blk + 15) / 16 + per_unit - 1) / per_unit;
      const unsigned g = (unsigned)(units < ((int64_t)1 << 30) ? units : ((int64_t)1 << 30));
      k_rot_t16<FMT, RB><<<g, Cfg::threads, 0, st>>>((const uint16_t *)src, (const uint16_t *)rot, r,
                                                    (uint16_t *)dst, n_blk);
      return;
    }
  }
  if constexpr (!(RB == 128 && FMT != 2 && OP == OP_QDQ)) {
    using Cfg = StagedCfg<RB>;
    const int64_t tiles = (n_blk + 31) / 32;
    int per_cu = OP == OP_QDQ ? Cfg::per_cu_qdq : Cfg::per_cu;
    if (RB == 64 && OP == OP_QDQ) {
      // A grid that covers a smaller tensor once gives each wave one tile,
      // behind its workgroup's staging of R: at least two tiles per wave
      // (at least 4 workgroups per CU) measured 5-7% faster on 4096 x 8192
      // and 8192 x 8192, while the larger layers keep 48 per CU
      const int64_t waves_per_cu = (int64_t)device_cu_count() * (Cfg::threads / 64);
      const int64_t want = (tiles + 2 * waves_per_cu - 1) / (2 * waves_per_cu);
      per_cu = (int)(want < 4 ? 4 : (want < per_cu ? want : per_cu));
    }
    const unsigned g = persistent_grid(tiles, Cfg::threads / 64, per_cu);
    if constexpr (OP == OP_QUANT && FMT != 2) {
      if (bl != nullptr) {
        k_rot_bf16<FMT, OP, RB, Cfg::threads, 1><<<g, Cfg::threads, staged_lds_pad<RB>(), st>>>(
            (const uint16_t *)src, (const uint16_t *)rot, r, dst, codes, scales, n_blk, *bl, nullptr);
        return;
      }
    }
    k_rot_bf16<FMT, OP, RB, Cfg::threads, 0><<<g, Cfg::threads, staged_lds_pad<RB>(), st>>>(
        (const uint16_t *)src, (const uint16_t *)rot, r, dst, codes, scales, n_blk, BlockedScales{0, 0, 0}, gp);
  }
}

template <int RB> constexpr int f32_per_cu() { return RB == 128 ? 8 : 3; }

template <int FMT, int OP, int RB>
static void run_direct(int dtype, const void *src, const void *rot, int r, void *dst, int64_t n, hipStream_t st) {
  const int64_t n_blk = n / RB;
  if (dtype == 0) {
    const int64_t tps = (DTHREADS / 64) / (RB / 32);
    const unsigned g = persistent_grid((n_blk + 32 * tps - 1) / (32 * tps), 1, RB == 128 ? 4 : f32_per_cu<RB>());
    k_rotate_bf16<RB><<<g, DTHREADS, 0, st>>>((const uint16_t *)src, (const uint16_t *)rot, r, (float *)dst, n_blk);
  } else {
    // one workgroup per 16 KiB step, persistent beyond f32_per_cu per CU
    const int64_t tps = (DTHREADS / 64) / (RB / 32);
    const unsigned g = persistent_grid((n_blk + 32 * tps - 1) / (32 * tps), 1, f32_per_cu<RB>());
    k_rot_f32<FMT, OP, RB><<<g, DTHREADS, 0, st>>>((const float *)src, (const float *)rot, r, dst, n_blk);
  }
}

// Block size of the staged (bf16) kernels: RB = max(r, 32), except that
// r = 16 and r = 32 run as RB = 64 (four or two copies of R on the
// diagonal) whenever the tensor is a whole number of 64-blocks and, for
// blocked scales, a row holds a whole number of them: the RB = 64 kernel
// streams its 4 KiB tiles faster than the RB = 32 kernel its 2 KiB ones.
static int staged_rb(int r, int64_t n, const BlockedScales *bl) {
  if (r <= 32 && n % 64 == 0 && (bl == nullptr || bl->groups % 2 == 0)) return 64;
  return r < 32 ? 32 : r;
}

template <int FMT, int OP>
static void dispatch_rb(int dtype, const void *src, const void *rot, int r, void *dst, uint8_t *codes,
                        uint8_t *scales, int64_t n, hipStream_t st, const BlockedScales *bl) {
  const int rb = dtype == 0 && OP != OP_ROTATE ? staged_rb(r, n, bl) : (r < 32 ? 32 : r);
  if (dtype == 0 && OP != OP_ROTATE) {
    if (rb == 32) run_staged<FMT, OP, 32>(src, rot, r, dst, codes, scales, n, st, bl);
    else if (rb == 64) run_staged<FMT, OP, 64>(src, rot, r, dst, codes, scales, n, st, bl);
    else if constexpr (OP == OP_QDQ) run_staged<FMT, OP, 128>(src, rot, r, dst, codes, scales, n, st, bl);
    else (void)launch_rot_lanes(FMT, OP, src, rot, r, dst, codes, scales, n, st, bl);  // (launch_rot sends it there)
  } else if (OP != OP_QUANT) {
    if (rb == 32) run_direct<FMT, OP, 32>(dtype, src, rot, r, dst, n, st);
    else if (rb == 64) run_direct<FMT, OP, 64>(dtype, src, rot, r, dst, n, st);
    else run_direct<FMT, OP, 128>(dtype, src, rot, r, dst, n, st);
  }
}

// Which bf16 rotations run on the lane-owned kernels of rotl.hip: r = 128
// for MX quantize (row-major scales, or blocked scales written by whole
// units) and for NVFP4 (QDQ and quantize).  Measured on MI355X against the
// kernels here, on the 8192 x 57344 layer, same box and run: MX quantize
// MXFP4 / MXFP8 3% / 2% faster, NVFP4 quantize 5% faster.  NVFP4 QDQ on
// the 16-block kernel measured 3-4% faster in interleaved A/B, but as
// bench.py times it (launches back to back, after the unrotated NVFP4 QDQ)
// 391-400 us against 333 us here.  MX QDQ at r = 128 runs on the 16-block
// kernel (310 against 349-358 us here); at r <= 64 the lane-owned kernel is
// slower (the full 128-wide contraction where the 64-element blocks here do
// a half or less).
static bool lanes_for(int fmt, int op, int r) { return r == 128 && (op == OP_QUANT || fmt == 2); }

hipError_t launch_nv_rot(int op, const void *src, const void *rot, int r, void *dst, uint8_t *codes,
                         uint8_t *scales, const float *gp, int64_t n, hipStream_t st) {
  if (lanes_for(2, op, r)) return launch_rot_lanes(2, op, src, rot, r, dst, codes, scales, n, st, nullptr, gp);
  const int rb = staged_rb(r, n, nullptr);  // 32 or 64: r = 128 runs on the lane-owned kernel
  if (op == OP_QDQ) {
    if (rb == 32) run_staged<2, OP_QDQ, 32>(src, rot, r, dst, codes, scales, n, st, nullptr, gp);
    else run_staged<2, OP_QDQ, 64>(src, rot, r, dst, codes, scales, n, st, nullptr, gp);
  } else {
    if (rb == 32) run_staged<2, OP_QUANT, 32>(src, rot, r, dst, codes, scales, n, st, nullptr, gp);
    else run_staged<2, OP_QUANT, 64>(src, rot, r, dst, codes, scales, n, st, nullptr, gp);
  }
  return hipGetLastError();
}

hipError_t launch_rot(int fmt, int op, int dtype, const void *src, const void *rot, int r, void *dst,
                      uint8_t *codes, uint8_t *scales, int64_t n, hipStream_t st, const BlockedScales *bl) {
  if (dtype == 0 && op != OP_ROTATE && lanes_for(fmt, op, r))
    return launch_rot_lanes(fmt, op, src, rot, r, dst, codes, scales, n, st, bl);
  if (op == OP_ROTATE) {
    dispatch_rb<0, OP_ROTATE>(dtype, src, rot, r, dst, codes, scales, n, st, nullptr);
  } else if (fmt == 0) {
    if (op == OP_QDQ) dispatch_rb<0, OP_QDQ>(dtype, src, rot, r, dst, codes, scales, n, st, nullptr);
    else dispatch_rb<0, OP_QUANT>(dtype, src, rot, r, dst, codes, scales, n, st, bl);
  } else {
    if (op == OP_QDQ) dispatch_rb<1, OP_QDQ>(dtype, src, rot, r, dst, codes, scales, n, st, nullptr);
    else dispatch_rb<1, OP_QUANT>(dtype, src, rot, r, dst, codes, scales, n, st, bl);
  }
  return hipGetLastError();
}

}  // namespace mx
