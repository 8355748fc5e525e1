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
// reads 8 fragments from LDS for 16 MFMAs.  A k-slice is 64 code bytes of
// every row (two E2M1 k-steps or one E4M3 k-step: 1024 matrix-core cycles
// per wave either way).
//
// Pipeline, per k-slice j:
//   global -> registers   buffer loads issued two slices ahead (two register
//                         sets), out-of-range rows and the K tail read as
//                         zero by the buffer unit, so the loop has no
//                         branches;
//   registers -> LDS      written into a ring of three buffers two slices
//                         ahead of use;
//   LDS -> registers      each k-step's fragments read while the matrix
//                         cores run the previous k-step, including the first
//                         k-step of slice j+1 during the last of slice j.
// With three buffers one barrier per slice suffices, and it comes after the
// slice's last MFMA: no matrix-core idle time waits on LDS reads.
// LDS rows are 64 bytes with the 16-byte chunks XOR-swizzled by row
// ((row/4)%4), which keeps both the chunk writes and the fragment reads free
// of bank conflicts without padding.
#include <type_traits>

#include "launch.h"
#include "mx_device.h"

namespace mx {

typedef int i32x8 __attribute__((ext_vector_type(8)));

constexpr int GT = 256, TI = 4, TJ = 4;               // threads; MFMA tiles per wave (rows, columns)
constexpr int BM = 64 * TI, BN = 64 * TJ;             // workgroup tile
constexpr int RB = 64;                                // code bytes per row per k-slice
constexpr int TILE = BM * RB;                         // one operand's slice in LDS
constexpr int BUF = 2 * TILE;                         // one ring slot (A then B)
constexpr int NBUF = 3;                               // ring depth
constexpr int CPT = BM * (RB / 16) / GT;              // 16-byte chunks per thread per operand
constexpr unsigned OOB = 0x80000000u;                 // a buffer offset past every record
constexpr int RSRC_FLAGS = 0x00020000;                // raw 32-bit buffer
static_assert(BM == BN && BM == GT, "one thread per row stages the row-major scales");

template <int FMT>
struct GemmShape {
  static constexpr int BK = FMT == 0 ? 128 : 64;     // k per slice
  static constexpr int NS = BK / 64;                 // k-steps per slice
  static constexpr int NG = BK / 32;                 // scale groups per slice
};

static __device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), (short)0, (int)bytes, RSRC_FLAGS);
}

// Keeps a selected buffer offset a plain value, so that the compiler does
// not turn "load at (c ? offset : OOB)" back into a branch around two loads.
static __device__ __forceinline__ void opaque_offset(unsigned &off) { asm volatile("" : "+v"(off)); }

// Scale layouts: SL 0 row-major bytes; SL 1 blocked (a lane's word for its
// 32-row block and 256-deep k-span is one coalesced 32-bit load); SL 2
// row-major with groups % NG == 0, so a thread's NG bytes of a slice are one
// aligned load.
template <int FMT, int OUT, int SL, bool TAIL>
__global__ __launch_bounds__(GT) void k_mx_gemm(const uint8_t *__restrict__ A, const uint8_t *__restrict__ As,
                                                 const uint8_t *__restrict__ B, const uint8_t *__restrict__ Bs,
                                                 int64_t M, int64_t N, int64_t K, float alpha,
                                                 void *__restrict__ C) {
  using S = GemmShape<FMT>;
  constexpr int BK = S::BK, NG = S::NG;
  constexpr int CBSZ = FMT == 0 ? 4 : 0;  // FP4 E2M1 : FP8 E4M3
  constexpr int NW = SL == 1 ? 4 : 2 * (BM + BN);  // row-major scale words per ring slot
  __shared__ __attribute__((aligned(16))) uint8_t sm[NBUF * BUF];
  __shared__ __attribute__((aligned(16))) unsigned ssw[NBUF][NW];
  // blocked scale words of two 256-deep k-spans, per wave (SL 1)
  __shared__ __attribute__((aligned(16))) unsigned wsl[SL == 1 ? 2 : 1][4][TI + TJ][64];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r = lane & 31, h = lane >> 5;
  const int64_t m0 = (int64_t)blockIdx.y * BM, n0 = (int64_t)blockIdx.x * BN;
  const int wm = (wave >> 1) * (32 * TI), wn = (wave & 1) * (32 * TJ);
  const int rb = (int)(FMT == 0 ? K / 2 : K);  // code bytes per row (<= 2^23)
  const int groups = (int)(K / 32);
  const int gblocks = (groups + 7) / 8;
  const int nslices = (int)((K + BK - 1) / BK);
  const int mrows = (int)(M - m0 < BM ? M - m0 : BM), nrows = (int)(N - n0 < BN ? N - n0 : BN);

  // ---- buffer resources over this workgroup's rows; reads past the
  // records return zero ------------------------------------------------------
  const __amdgpu_buffer_rsrc_t rA = make_rsrc(A + m0 * rb, (uint32_t)mrows * (uint32_t)rb);
  const __amdgpu_buffer_rsrc_t rB = make_rsrc(B + n0 * rb, (uint32_t)nrows * (uint32_t)rb);
  __amdgpu_buffer_rsrc_t rAs, rBs;
  if constexpr (SL == 1) {
    const int blk = gblocks * 256;  // bytes per 32-row block
    rAs = make_rsrc(As + (m0 / 32) * blk, (uint32_t)((mrows + 31) / 32) * (uint32_t)blk);
    rBs = make_rsrc(Bs + (n0 / 32) * blk, (uint32_t)((nrows + 31) / 32) * (uint32_t)blk);
  } else {
    rAs = make_rsrc(As + m0 * groups, (uint32_t)mrows * (uint32_t)groups);
    rBs = make_rsrc(Bs + n0 * groups, (uint32_t)nrows * (uint32_t)groups);
  }

  // this thread's chunks: rows tid/4 + 64 it, logical chunk tid%4, stored at
  // physical chunk (tid%4) ^ ((row/4)%4) = (tid%4) ^ ((tid/16)%4)
  const int crow = tid >> 2, cchunk = tid & 3;
  const int wr_off = crow * RB + 16 * (cchunk ^ ((tid >> 4) & 3));
  // fragment read offsets: row r of a 32-row tile, logical chunk c at c ^ ((r/4)%4)
  const int sw = (r >> 2) & 3;
  int rd_off[2];
  if constexpr (FMT == 0) {
    rd_off[0] = r * RB + 16 * ((0 + h) ^ sw);  // k-step 0: chunk h
    rd_off[1] = r * RB + 16 * ((2 + h) ^ sw);  // k-step 1: chunk 2 + h
  } else {
    rd_off[0] = r * RB + 16 * ((0 + h) ^ sw);  // bytes [16h, 16h + 16) of group 0
    rd_off[1] = r * RB + 16 * ((2 + h) ^ sw);  // and of group 1
  }
  auto tile_off = [&](int f) { return f < TI ? (wm + 32 * f) * RB : TILE + (wn + 32 * (f - TI)) * RB; };

  // ---- staged registers: two sets (slice parity) ------------------------------
  // Scale words: SL 0 and 2 stage, per row, the slice's groups split into an
  // even word (groups 0, 2) and an odd word (groups 1, 3), so that a lane of
  // half h finds its k-step s scale in byte s of word h.  SL 1 words (byte t
  // = k-step t of a 256-deep span) change once per span and have their own
  // pipeline below.
  constexpr int NSW = SL == 1 ? 1 : 4;
  struct Staged {
    u32x4 a[CPT], b[CPT];
    unsigned w[NSW];
  };
  Staged st[2];

  // row offsets of this thread's chunks; the slice offset goes in the
  // instruction's scalar offset.  Prefetches past the last slice re-read the
  // last slice (their data is never used), so no load leaves the operands.
  unsigned rowoff[CPT];
#pragma unroll
  for (int it = 0; it < CPT; ++it) rowoff[it] = (unsigned)((crow + 64 * it) * rb + 16 * cchunk);
  auto load_slice = [&](Staged &s, int ks) {
    const int kq = ks < nslices ? ks : nslices - 1;
    const int kb0 = kq * RB;
    unsigned voff[CPT];
#pragma unroll
    for (int it = 0; it < CPT; ++it) {
      voff[it] = rowoff[it];
      if constexpr (TAIL) {
        // the last slice of a K that is not a whole number of slices:
        // chunks past the row read as zero
        voff[it] = 16 * cchunk < rb - kb0 ? voff[it] : OOB;
        opaque_offset(voff[it]);
      }
    }
#pragma unroll
    for (int it = 0; it < CPT; ++it) {
      s.a[it] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rA, (int)voff[it], kb0, 0));
      s.b[it] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rB, (int)voff[it], kb0, 0));
    }
    if constexpr (SL != 1) {
      unsigned wa, wb;
      if constexpr (SL == 2) {
        // NG aligned bytes per row
        if constexpr (NG == 4) {
          wa = __builtin_amdgcn_raw_buffer_load_b32(rAs, tid * groups, kq * NG, 0);
          wb = __builtin_amdgcn_raw_buffer_load_b32(rBs, tid * groups, kq * NG, 0);
        } else {
          wa = __builtin_amdgcn_raw_buffer_load_b16(rAs, tid * groups, kq * NG, 0);
          wb = __builtin_amdgcn_raw_buffer_load_b16(rBs, tid * groups, kq * NG, 0);
        }
      } else {
        // bytes; groups past K re-read the row's last group, whose codes
        // there are zero
        wa = wb = 0;
#pragma unroll
        for (int j = 0; j < NG; ++j) {
          const int g = kq * NG + j < groups ? kq * NG + j : groups - 1;
          wa |= (unsigned)__builtin_amdgcn_raw_buffer_load_b8(rAs, tid * groups, g, 0) << (8 * j);
          wb |= (unsigned)__builtin_amdgcn_raw_buffer_load_b8(rBs, tid * groups, g, 0) << (8 * j);
        }
      }
      // even and odd groups: bytes (0, 2) and (1, 3)
      s.w[0] = __builtin_amdgcn_perm(0u, wa, 0x0c0c0200u);
      s.w[1] = __builtin_amdgcn_perm(0u, wa, 0x0c0c0301u);
      s.w[2] = __builtin_amdgcn_perm(0u, wb, 0x0c0c0200u);
      s.w[3] = __builtin_amdgcn_perm(0u, wb, 0x0c0c0301u);
    }
  };
  auto store_slice = [&](const Staged &s, int buf) {
    uint8_t *base = sm + buf * BUF + wr_off;
#pragma unroll
    for (int it = 0; it < CPT; ++it) {
      *(u32x4 *)(base + it * 64 * RB) = s.a[it];
      *(u32x4 *)(base + TILE + it * 64 * RB) = s.b[it];
    }
    if constexpr (SL != 1) {
      *(uint2 *)&ssw[buf][2 * tid] = uint2{s.w[0], s.w[1]};
      *(uint2 *)&ssw[buf][2 * (BM + tid)] = uint2{s.w[2], s.w[3]};
    }
  };

  // Blocked scale words, once per 256-deep k-span: a wave's 8 tiles x 64
  // words of a span are two 16-byte loads per lane (lane L: tile L/16 of the
  // A or B half, words 4(L%16)..4(L%16)+3), staged in registers one span
  // ahead and written to a per-wave LDS slot, from which lane l reads word l
  // of each tile.  Only the wave itself touches its slots, so program order
  // is the only ordering needed.
  u32x4 wst[2];
  auto load_span_words = [&](int span) {
    const int sp = span < gblocks ? span : gblocks - 1;
    const unsigned va = (unsigned)(((wm >> 5) + (lane >> 4)) * gblocks * 256 + 16 * (lane & 15));
    const unsigned vb = (unsigned)(((wn >> 5) + (lane >> 4)) * gblocks * 256 + 16 * (lane & 15));
    wst[0] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rAs, (int)va, sp * 256, 0));
    wst[1] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rBs, (int)vb, sp * 256, 0));
  };
  auto store_span_words = [&](int span) {
    uint8_t *base = (uint8_t *)&wsl[span & 1][wave][0][0] + 16 * lane;
    *(u32x4 *)base = wst[0];
    *(u32x4 *)(base + 4 * 64 * 4) = wst[1];
  };

  // ---- fragments and scale words ---------------------------------------------
  using Frag = typename std::conditional<FMT == 0, u32x4, i32x8>::type;
  auto read_frag = [&](int buf, int f, int s) -> Frag {
    const uint8_t *p = sm + buf * BUF + tile_off(f);
    if constexpr (FMT == 0) {
      return *(const u32x4 *)(p + rd_off[s]);
    } else {
      const u32x4 lo = *(const u32x4 *)(p + rd_off[0]), hi = *(const u32x4 *)(p + rd_off[1]);
      return i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
    }
  };
  // scale word of tile f for slice ks (ring slot buf)
  auto read_word = [&](int buf, int ks, int f) -> unsigned {
    if constexpr (SL == 1) return wsl[((ks * BK) >> 8) & 1][wave][f][lane];
    else return ssw[buf][2 * (f < TI ? wm + 32 * f + r : BM + wn + 32 * (f - TI) + r) + h];
  };

  f32x16 acc[TI][TJ];
#pragma unroll
  for (int i = 0; i < TI; ++i)
#pragma unroll
    for (int j = 0; j < TJ; ++j) acc[i][j] = f32x16{};

  // 16 MFMAs of one k-step; the scale byte is picked by the instruction's
  // byte select (BYTE)
  auto mfma = [&](auto BYTE, const Frag *fr, const unsigned *w) {
    constexpr int byte = decltype(BYTE)::value;
#pragma unroll
    for (int i = 0; i < TI; ++i)
#pragma unroll
      for (int j = 0; j < TJ; ++j) {
        i32x8 fa, fb;
        if constexpr (FMT == 0) {
          const u32x4 a = fr[i], b = fr[TI + j];  // upper halves unused for E2M1
          fa = i32x8{(int)a.x, (int)a.y, (int)a.z, (int)a.w, 0, 0, 0, 0};
          fb = i32x8{(int)b.x, (int)b.y, (int)b.z, (int)b.w, 0, 0, 0, 0};
        } else {
          fa = fr[i];
          fb = fr[TI + j];
        }
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fa, fb, acc[i][j], CBSZ, CBSZ, byte,
                                                                    (int)w[i], byte, (int)w[TI + j]);
      }
  };

  // fragments of the next k-step to run, and the scale words of its slice
  Frag fr[2][TI + TJ];
  unsigned wd[TI + TJ];

  if (nslices > 0) {
    if constexpr (SL == 1) {
      load_span_words(0);
      store_span_words(0);
      load_span_words(1);
    }
    load_slice(st[0], 0);
    store_slice(st[0], 0);
    load_slice(st[1], 1);
    store_slice(st[1], 1);
    load_slice(st[0], 2);
    load_slice(st[1], 3);
    __syncthreads();
#pragma unroll
    for (int f = 0; f < TI + TJ; ++f) {
      fr[0][f] = read_frag(0, f, 0);
      wd[f] = read_word(0, 0, f);
    }
  }

  // one k-slice: ks in ring slot b0, at position Q of its 256-deep k-span
  // (slices start a span at Q = 0); the staged set Q%2 holds slice ks+2 and
  // is refilled with slice ks+4
  auto slice = [&](auto Qc, int ks, int b0) {
    constexpr int q = decltype(Qc)::value, p = q & 1;
    const int b1 = b0 == NBUF - 1 ? 0 : b0 + 1, b2 = b1 == NBUF - 1 ? 0 : b1 + 1;
    if constexpr (FMT == 0) {
      // k-step 0; read k-step 1's fragments and stage slice ks+2
      mfma(std::integral_constant<int, SL == 1 ? 2 * q : 0>{}, fr[0], wd);
#pragma unroll
      for (int f = 0; f < TI + TJ; ++f) fr[1][f] = read_frag(b0, f, 1);
      store_slice(st[p], b2);
      if constexpr (SL == 1 && q == 0) {
        // the next span's words to LDS, the one after into registers
        store_span_words(((ks * BK) >> 8) + 1);
        load_span_words(((ks * BK) >> 8) + 2);
      }
#pragma unroll
      for (int k = 0; k < TI * TJ; ++k) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
        if (k < TI + TJ) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // fragment read
        __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);  // LDS write
      }
      // k-step 1; load slice ks+4, read slice ks+1's first fragments
      unsigned wcur[TI + TJ];
#pragma unroll
      for (int f = 0; f < TI + TJ; ++f) wcur[f] = wd[f];
      mfma(std::integral_constant<int, SL == 1 ? 2 * q + 1 : 1>{}, fr[1], wcur);
      load_slice(st[p], ks + 4);
#pragma unroll
      for (int f = 0; f < TI + TJ; ++f) {
        fr[0][f] = read_frag(b1, f, 0);
        wd[f] = read_word(b1, ks + 1, f);
      }
#pragma unroll
      for (int k = 0; k < TI * TJ; ++k) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
        __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // global load
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // LDS read
      }
    } else {
      // the slice's one k-step; stage slice ks+2, load slice ks+4, read
      // slice ks+1's fragments into the other set
      unsigned wcur[TI + TJ];
#pragma unroll
      for (int f = 0; f < TI + TJ; ++f) wcur[f] = wd[f];
      mfma(std::integral_constant<int, SL == 1 ? q : 0>{}, fr[p], wcur);
      store_slice(st[p], b2);
      if constexpr (SL == 1 && q == 0) {
        store_span_words(((ks * BK) >> 8) + 1);
        load_span_words(((ks * BK) >> 8) + 2);
      }
      load_slice(st[p], ks + 4);
#pragma unroll
      for (int f = 0; f < TI + TJ; ++f) {
        fr[p ^ 1][f] = read_frag(b1, f, 0);
        wd[f] = read_word(b1, ks + 1, f);
      }
#pragma unroll
      for (int k = 0; k < TI * TJ; ++k) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
        __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);  // LDS write
        __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // global load
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // LDS reads
      }
    }
    __syncthreads();
    return b1;
  };

  // slices per 256-deep k-span: the loop runs whole spans, so that every
  // scale byte select is a constant
  constexpr int U = 256 / BK;
  int ks = 0, b0 = 0;
  for (; ks + U <= nslices; ks += U) {
    b0 = slice(std::integral_constant<int, 0>{}, ks, b0);
    b0 = slice(std::integral_constant<int, 1>{}, ks + 1, b0);
    if constexpr (U == 4) {
      b0 = slice(std::integral_constant<int, 2>{}, ks + 2, b0);
      b0 = slice(std::integral_constant<int, 3>{}, ks + 3, b0);
    }
  }
  // the last, partial span
  if (ks < nslices) b0 = slice(std::integral_constant<int, 0>{}, ks, b0);
  if (ks + 1 < nslices) b0 = slice(std::integral_constant<int, 1>{}, ks + 1, b0);
  if constexpr (U == 4) {
    if (ks + 2 < nslices) b0 = slice(std::integral_constant<int, 2>{}, ks + 2, b0);
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

template <int SL, bool TAIL>
static void run_gemm(int fmt, int out_dtype, dim3 grid, const uint8_t *a, const uint8_t *as, const uint8_t *b,
                     const uint8_t *bs, int64_t M, int64_t N, int64_t K, float alpha, void *c, hipStream_t st) {
  if (fmt == 0 && out_dtype == 0) k_mx_gemm<0, 0, SL, TAIL><<<grid, GT, 0, st>>>(a, as, b, bs, M, N, K, alpha, c);
  else if (fmt == 0) k_mx_gemm<0, 1, SL, TAIL><<<grid, GT, 0, st>>>(a, as, b, bs, M, N, K, alpha, c);
  else if (out_dtype == 0) k_mx_gemm<1, 0, SL, TAIL><<<grid, GT, 0, st>>>(a, as, b, bs, M, N, K, alpha, c);
  else k_mx_gemm<1, 1, SL, TAIL><<<grid, GT, 0, st>>>(a, as, b, bs, M, N, K, alpha, c);
}

template <int SL>
static void run_gemm_k(int fmt, int out_dtype, dim3 grid, const uint8_t *a, const uint8_t *as, const uint8_t *b,
                       const uint8_t *bs, int64_t M, int64_t N, int64_t K, float alpha, void *c, hipStream_t st) {
  // a K that is not a whole number of slices reads its last slice with
  // per-chunk bounds
  const int64_t bk = fmt == 0 ? GemmShape<0>::BK : GemmShape<1>::BK;
  if (K % bk == 0) run_gemm<SL, false>(fmt, out_dtype, grid, a, as, b, bs, M, N, K, alpha, c, st);
  else run_gemm<SL, true>(fmt, out_dtype, grid, a, as, b, bs, M, N, K, alpha, c, st);
}

hipError_t launch_gemm(int fmt, const uint8_t *a, const uint8_t *as, const uint8_t *b, const uint8_t *bs,
                       int scale_layout, int64_t M, int64_t N, int64_t K, float alpha, int out_dtype, void *c,
                       hipStream_t st) {
  const dim3 grid((unsigned)((N + BN - 1) / BN), (unsigned)((M + BM - 1) / BM));
  if (scale_layout == 1) {
    run_gemm_k<1>(fmt, out_dtype, grid, a, as, b, bs, M, N, K, alpha, c, st);
  } else {
    // whole-word row-major scale loads when every slice's groups are aligned
    const int ng = fmt == 0 ? 4 : 2;
    const bool aligned = (K / 32) % ng == 0 && (uintptr_t)as % ng == 0 && (uintptr_t)bs % ng == 0;
    if (aligned) run_gemm_k<2>(fmt, out_dtype, grid, a, as, b, bs, M, N, K, alpha, c, st);
    else run_gemm_k<0>(fmt, out_dtype, grid, a, as, b, bs, M, N, K, alpha, c, st);
  }
  return hipGetLastError();
}

}  // namespace mx
