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
// reads 8 fragments from LDS for 16 MFMAs.  A k-slice is 128 code bytes of
// every row (four E2M1 or two E4M3 k-steps: 2048 matrix-core cycles per wave
// either way).
//
// Data path (measured on gfx950 with GEMM-shaped slices, one workgroup per
// CU: loads of whole 128-byte row segments stream at 91 GB/s per CU, 64-byte
// ones at 57 GB/s whatever the number in flight; LDS writes from registers
// run at a third of the LDS read rate):
//   codes go from global memory straight into LDS (buffer loads with an LDS
//   destination), one wave instruction per 8 rows x 128 bytes, into one of
//   two static LDS slots; rows past the operands and the K tail read as zero
//   through the buffer resource;
//   the fragments of each k-step are read from LDS while the matrix cores run
//   the previous k-step;
//   two barriers per slice: the first, once every wave has read the slice's
//   last fragments, frees its slot for the slice after next; the second,
//   before the last 8 MFMAs, publishes the next slice, so that those MFMAs
//   overlap the reads of the next slice's first fragments;
//   the loads are paced, one per 64 cycles per wave, between the two
//   barriers, after the second and through the next slice's first k-steps
//   (see "Pacing" below).
// LDS rows are 128 bytes with the 16-byte chunks XOR-swizzled by (row/2)%8,
// which keeps the 16-lane fragment reads free of bank conflicts.
#include <type_traits>

#include "launch.h"
#include "mx_device.h"

namespace mx {

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
#define MX_LDS(p) ((__attribute__((address_space(3))) void *)(p))

constexpr int GT = 256, TI = 4, TJ = 4;               // threads; MFMA tiles per wave (rows, columns)
constexpr int BM = 64 * TI, BN = 64 * TJ;             // workgroup tile
constexpr int RB = 128;                               // code bytes per row per k-slice
constexpr int TILE = BM * RB;                         // one operand's slice in LDS (32 KB)
constexpr int SLOT = 2 * TILE;                        // one LDS slot: A then B
constexpr int DMA_W = TILE / 1024 / 4;                // 1 KB loads per wave per operand per slice
constexpr unsigned OOB = 0x80000000u;                 // a buffer offset past every record
constexpr int RSRC_FLAGS = 0x00020000;                // raw 32-bit buffer
static_assert(BM == BN && BM == GT, "one thread per row stages the row-major scales");

template <int N>
using IC = std::integral_constant<int, N>;

// Pacing of a slice's loads.  A wave that issues loads with an LDS
// destination faster than the address unit takes them (16 cycles per 1 KB
// instruction, shared by the CU's four waves) stalls at issue, and its
// matrix-core work with it; so each wave issues at most one per 64 cycles:
// one per two E2M1 MFMAs, one per E4M3 MFMA.  Measured on gfx950 with
// GEMM-shaped slices (64 KB per CU): loads alone take 0.78 us per slice and
// MFMAs alone 1.05 us; a burst of each wave's 16 loads ahead of its 64 MFMAs
// takes 1.5 us, the same loads issued by other waves 1.15 us.
// A slice's load jobs issued between its two barriers (JA), after the
// publishing barrier (JB) and, for E2M1, during the next slice's first
// k-step (JS0); the rest go out in its second.  E2M1 also takes two
// barriers per slice (one measured 3-4% slower once the loads were paced).
constexpr int GEMM_JA4 = 4, GEMM_JB4 = 4, GEMM_JS04 = 8;  // E2M1
constexpr int GEMM_JA8 = 8, GEMM_JB8 = 8;                  // E4M3
constexpr bool GEMM_SPLIT4 = true;


// the number of n events, spread evenly over m slots, that fall in slot k
__device__ __forceinline__ constexpr int spread(int k, int n, int m) { return ((k + 1) * n) / m - (k * n) / m; }

// a scheduling group of n (0..4) vector-memory instructions
__device__ __forceinline__ void sched_vmem(int n) {
  if (n == 1) __builtin_amdgcn_sched_group_barrier(0x010, 1, 0);
  else if (n == 2) __builtin_amdgcn_sched_group_barrier(0x010, 2, 0);
  else if (n == 3) __builtin_amdgcn_sched_group_barrier(0x010, 3, 0);
  else if (n >= 4) __builtin_amdgcn_sched_group_barrier(0x010, 4, 0);
}

template <int FMT>
struct GemmShape {
  static constexpr int BK = FMT == 0 ? 256 : 128;    // k per slice
  static constexpr int NS = BK / 64;                 // k-steps per slice
  static constexpr int NG = BK / 32;                 // scale groups per slice
};

// Barrier that publishes LDS written by this workgroup's buffer loads with
// an LDS destination: each wave first waits for all of its own vector-memory
// operations (vmcnt(0)), so that after the barrier every wave's loads have
// landed.  A plain __syncthreads() does not imply that wait at workgroup
// scope: the compiler inserts it only where it sees a dependence, and across
// the k-loop's back-edge it did not (one of the two barriers per iteration
// went without it, so a slice could be read before other waves' loads of it
// had landed).
static __device__ __forceinline__ void publish_lds_loads() {
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
  __syncthreads();
}

static __device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), (short)0, (int)bytes, RSRC_FLAGS);
}

// Scale layouts: SL 0 row-major bytes; SL 1 blocked (a wave's words for its
// 8 tiles and one 256-deep k-span are two 1 KB loads straight into LDS);
// SL 2 row-major with groups % NG == 0, so a row's NG bytes of a slice are
// whole aligned dwords; SL 3 row-major with groups % 16 == 0 and 16-byte
// aligned scales, loaded by 16-byte spans of 16 groups (two E2M1 slices or
// four E4M3 slices; the group-parity split of the LDS-loaded forms is done
// when a slice starts).
template <int FMT, int OUT, int SL, bool TAIL>
__global__ __launch_bounds__(GT) void k_mx_gemm(const uint8_t *__restrict__ A, const uint8_t *__restrict__ As,
                                                 const uint8_t *__restrict__ B, const uint8_t *__restrict__ Bs,
                                                 int64_t M, int64_t N, int64_t K, float alpha,
                                                 void *__restrict__ C) {
  using S = GemmShape<FMT>;
  constexpr int BK = S::BK, NS = S::NS, NG = S::NG;
  constexpr int CBSZ = FMT == 0 ? 4 : 0;  // FP4 E2M1 : FP8 E4M3
  constexpr int NWB = SL == 1 ? 4 * (TI + TJ) * 64 : 4;   // blocked words per slot
  constexpr int NWR = SL == 1 || SL == 3 ? 4 : 2 * (BM + BN);  // row-major words per slot
  // Row-major scales:
  //  - SL 3 (SPAN): 16 bytes of every row (16 groups: two E2M1 slices, four
  //    E4M3 slices) straight into LDS, one load per row and span into one of
  //    two span buffers.  A load of scales covers 64 rows, one line each, so
  //    its address-unit time is several code loads'; spans take the fewest;
  //  - E4M3, SL 2 (SDMA): one dword per row and slice straight into LDS
  //    (9% faster than through registers);
  //  - otherwise (SREG) through registers: E2M1 at SL 2 (its two dwords per
  //    row and slice would take twice the LDS-destination loads of one
  //    8-byte load per thread, measured 6% slower) and the byte loads of
  //    SL 0.
  constexpr bool SPAN = SL == 3;
  constexpr int SPLC = 16 / NG;  // slices per span
  constexpr bool SDMA = SL == 2 && FMT == 1;
  constexpr bool SREG = SL == 0 || (SL == 2 && FMT == 0);
  // Each slice is published with two barriers (see the slice loop), so that
  // a slot starts taking the loads of the slice after next as soon as its
  // last fragments have been read: E4M3 2.12 -> 1.95 ms (row-major scales)
  // and 1.79 -> 1.69 ms (blocked) when the loads went out in one burst; with
  // paced loads, E2M1 gains 3-4% over one barrier.
  constexpr bool SPLIT = FMT == 1 || GEMM_SPLIT4;
  // a slice's load jobs: the code loads, then the scale loads that travel
  // with it; JA are issued between the two barriers (SPLIT), JB after the
  // publishing barrier, JS0 and JS1 during the next slice's k-steps 0 and 1
  constexpr int NJ = 2 * DMA_W + (SL == 1 || SDMA ? 2 : 0);
  constexpr int JA0 = !SPLIT ? 0 : FMT == 0 ? GEMM_JA4 : GEMM_JA8, JA = JA0 < NJ ? JA0 : NJ;
  constexpr int JB0 = FMT == 0 ? GEMM_JB4 : GEMM_JB8, JB = JB0 < NJ - JA ? JB0 : NJ - JA;
  constexpr int JS0 = FMT == 0 ? (NJ - JA - JB < GEMM_JS04 ? NJ - JA - JB : GEMM_JS04) : NJ - JA - JB;
  constexpr int JS1 = NJ - JA - JB - JS0;
  static_assert(JA >= 0 && JB >= 0 && JS0 >= 0 && JS1 >= 0 && (NS == 4 || JS1 == 0), "job schedule");
  // register scale loads issued with the slice after next (SREG)
  constexpr int NSREG = !(SL == 0 || (SL == 2 && FMT == 0)) ? 0 : SL == 2 ? 2 : 2 * NG;
  static_assert(DMA_W == 8, "16 code loads per wave and slice");
  constexpr int NSP = SPAN ? (BM + BN) * 16 : 16;       // span buffer bytes
  __shared__ __attribute__((aligned(1024))) uint8_t sm0[SLOT], sm1[SLOT];
  __shared__ __attribute__((aligned(1024))) unsigned wb0[NWB], wb1[NWB];
  __shared__ __attribute__((aligned(1024))) unsigned wr0[NWR], wr1[NWR];
  __shared__ __attribute__((aligned(1024))) uint8_t wsp[2][NSP];

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

  // ---- code loads: wave load i of an operand fills 1 KB of LDS, rows
  // 8g..8g+7 (g = 4i + wave); lane L takes row 8g + L/8 and physical chunk
  // L%8, which holds logical chunk (L%8) ^ ((row/2)%8) ------------------------
  unsigned dvoff[DMA_W];
  int dchunk[DMA_W];
#pragma unroll
  for (int i = 0; i < DMA_W; ++i) {
    const int row = 8 * (4 * i + wave) + (lane >> 3);
    dchunk[i] = (lane & 7) ^ ((row >> 1) & 7);
    dvoff[i] = (unsigned)(row * rb + 16 * dchunk[i]);
  }
  auto slot_of = [&](auto Pc) -> uint8_t * { return decltype(Pc)::value ? sm1 : sm0; };
  // The loads of slice ks into slot P, as NJ jobs in issue order: job j <
  // 2*DMA_W is code load j/2 of operand j%2 (A, B), then the slice's scale
  // loads (blocked words, or the SDMA dwords).  Jobs [LO, HI) are issued;
  // prefetches past the last slice re-read it.
  auto load_jobs = [&](auto Pc, int ks, auto LO, auto HI) {
    constexpr int lo = decltype(LO)::value, hi = decltype(HI)::value;
    uint8_t *slot = slot_of(Pc);
    const int kq = ks < nslices ? ks : nslices - 1;
    const int kb0 = kq * RB;
#pragma unroll
    for (int jb = lo; jb < hi; ++jb) {
      if (jb < 2 * DMA_W) {
        const int i = jb >> 1;
        unsigned off = dvoff[i];
        if constexpr (TAIL) {
          // the last slice of a K that is not a whole number of slices:
          // chunks past the row read as zero
          off = 16 * dchunk[i] < rb - kb0 ? off : OOB;
          opaque_offset(off);
        }
        uint8_t *dst = slot + (4 * i + wave) * 1024 + (jb & 1) * TILE;
        __builtin_amdgcn_raw_ptr_buffer_load_lds((jb & 1) ? rB : rA, MX_LDS(dst), 16, off, kb0, 0, 0);
      } else if constexpr (SL == 1) {
        // blocked words of the slice's 256-deep span: lane L takes words
        // 4(L%16)..4(L%16)+3 of tile L/16 (A tiles, then B tiles)
        unsigned *wb = decltype(Pc)::value ? wb1 : wb0;
        const int span = (kq * BK) >> 8;
        if (jb == 2 * DMA_W) {
          const unsigned va = (unsigned)(((wm >> 5) + (lane >> 4)) * gblocks * 256 + 16 * (lane & 15));
          __builtin_amdgcn_raw_ptr_buffer_load_lds(rAs, MX_LDS(wb + wave * (TI + TJ) * 64), 16, va, span * 256, 0, 0);
        } else {
          const unsigned vb = (unsigned)(((wn >> 5) + (lane >> 4)) * gblocks * 256 + 16 * (lane & 15));
          __builtin_amdgcn_raw_ptr_buffer_load_lds(rBs, MX_LDS(wb + (wave * (TI + TJ) + TI) * 64), 16, vb,
                                                   span * 256, 0, 0);
        }
      } else if constexpr (SDMA) {
        // the slice's NG = 4 scale bytes of every row, straight into LDS as
        // [row][4]: wave w takes rows 64w..64w+63 of each operand, a dword
        // per lane
        static_assert(NG == 4, "one dword per row");
        unsigned *wr = decltype(Pc)::value ? wr1 : wr0;
        const unsigned voff = (unsigned)((64 * wave + lane) * groups);
        if (jb == 2 * DMA_W) __builtin_amdgcn_raw_ptr_buffer_load_lds(rAs, MX_LDS(wr + 64 * wave), 4, voff, kq * NG, 0, 0);
        else __builtin_amdgcn_raw_ptr_buffer_load_lds(rBs, MX_LDS(wr + BM + 64 * wave), 4, voff, kq * NG, 0, 0);
      }
    }
  };

  // ---- row-major scales by 16-byte spans (SPAN): span j holds groups
  // 16j..16j+15 of every row, i.e. slices SPLC*j .. SPLC*j + SPLC-1, in
  // buffer j % 2 as [row][16]; wave w loads rows 64w..64w+63 of each
  // operand, a row per lane.  The launch takes this path only when the
  // groups of a row are a multiple of 16, so no span reaches past its row ---
  auto load_span = [&](int j) {
    const int nspans = nslices / SPLC;
    const int jq = j < nspans ? j : nspans - 1;  // past the end: re-read the last span, unused
    uint8_t *d = wsp[j & 1];
    const unsigned voff = (unsigned)((64 * wave + lane) * groups + 16 * jq);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rAs, MX_LDS(d + 64 * wave * 16), 16, voff, 0, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rBs, MX_LDS(d + (BM + 64 * wave) * 16), 16, voff, 0, 0, 0);
  };

  // ---- row-major scales through registers (SREG): a thread loads its A
  // row's and B row's NG bytes of a slice and stores them split by group
  // parity: word h holds groups h, 2+h, 4+h, 6+h, so byte t is the scale of
  // k-step t for lanes of half h ----------------------------------------------
  struct RowScales {
    u32x2 a, b;
  };
  auto load_row_scales = [&](int ks) -> RowScales {
    const int kq = ks < nslices ? ks : nslices - 1;
    RowScales v{};
    if constexpr (SL == 2) {
      // E2M1 (NG = 8): one aligned 8-byte load per row
      v.a = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(rAs, tid * groups, kq * NG, 0));
      v.b = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(rBs, tid * groups, kq * NG, 0));
    } else {
      // bytes; groups past K re-read the row's last group, whose codes there
      // are zero
#pragma unroll
      for (int j = 0; j < NG; ++j) {
        const int g = kq * NG + j < groups ? kq * NG + j : groups - 1;
        const unsigned ba = __builtin_amdgcn_raw_buffer_load_b8(rAs, tid * groups, g, 0);
        const unsigned bb = __builtin_amdgcn_raw_buffer_load_b8(rBs, tid * groups, g, 0);
        if (j < 4) {
          v.a.x |= ba << (8 * j);
          v.b.x |= bb << (8 * j);
        } else {
          v.a.y |= ba << (8 * (j - 4));
          v.b.y |= bb << (8 * (j - 4));
        }
      }
    }
    return v;
  };
  auto store_row_scales = [&](auto Pc, const RowScales &v) {
    unsigned *wr = decltype(Pc)::value ? wr1 : wr0;
    *(u32x2 *)&wr[2 * tid] = u32x2{__builtin_amdgcn_perm(v.a.y, v.a.x, 0x06040200u),
                                   __builtin_amdgcn_perm(v.a.y, v.a.x, 0x07050301u)};
    *(u32x2 *)&wr[2 * (BM + tid)] = u32x2{__builtin_amdgcn_perm(v.b.y, v.b.x, 0x06040200u),
                                          __builtin_amdgcn_perm(v.b.y, v.b.x, 0x07050301u)};
  };

  // ---- fragments and scale words ---------------------------------------------
  // lane offsets: row r of a 32-row tile, logical chunk c at c ^ ((r/2)%8)
  const int sw = (r >> 1) & 7;
  int rd[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    // E2M1: k-step t is chunk 2t + h; E4M3: k-step t/2's chunk 4(t/2) + 2(t%2) + h
    const int c = FMT == 0 ? 2 * t + h : 4 * (t >> 1) + 2 * (t & 1) + h;
    rd[t] = r * RB + 16 * (c ^ sw);
  }
  using Frag = typename std::conditional<FMT == 0, u32x4, i32x8>::type;
  auto tile_off = [&](int f) { return f < TI ? (wm + 32 * f) * RB : TILE + (wn + 32 * (f - TI)) * RB; };
  auto read_frag = [&](auto Pc, int f, int t) -> Frag {
    const uint8_t *p = slot_of(Pc) + tile_off(f);
    if constexpr (FMT == 0) {
      return *(const u32x4 *)(p + rd[t]);
    } else {
      const u32x4 lo = *(const u32x4 *)(p + rd[2 * t]), hi = *(const u32x4 *)(p + rd[2 * t + 1]);
      return i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
    }
  };
  // A scale word as read from LDS (SDMA and SPAN: the row's NG bytes of the
  // slice as loaded, split by group parity only when the slice starts, so
  // that the split does not wait for the read in the middle of the MFMAs it
  // overlaps), and its value: byte t is the scale of k-step t for lanes of
  // half h.
  using Word = typename std::conditional<SDMA || SPAN, u32x2, unsigned>::type;
  // (H: the slice's phase ks % SPLC in its span, for SPAN)
  auto read_word = [&](auto Pc, auto Hc, int f, int ks) -> Word {
    if constexpr (SPAN) {
      // slice ks = SPLC*j + H: bytes NG*H .. NG*H + NG-1 of the row in span
      // buffer j % 2
      constexpr int H = decltype(Hc)::value;
      const uint8_t *b = wsp[(ks / SPLC) & 1] + 16 * (f < TI ? wm + 32 * f + r : BM + wn + 32 * (f - TI) + r);
      if constexpr (FMT == 0) return *(const u32x2 *)(b + 8 * H);
      else return u32x2{*(const unsigned *)(b + 4 * H), 0u};
    } else if constexpr (SL == 1) {
      const unsigned *wb = decltype(Pc)::value ? wb1 : wb0;
      return wb[(wave * (TI + TJ) + f) * 64 + lane];
    } else if constexpr (SDMA) {
      const unsigned *wr = decltype(Pc)::value ? wr1 : wr0;
      return u32x2{wr[f < TI ? wm + 32 * f + r : BM + wn + 32 * (f - TI) + r], 0u};
    } else {
      const unsigned *wr = decltype(Pc)::value ? wr1 : wr0;
      return wr[2 * (f < TI ? wm + 32 * f + r : BM + wn + 32 * (f - TI) + r) + h];
    }
  };
  auto word_value = [&](const Word &w) -> unsigned {
    if constexpr (SDMA || SPAN) return __builtin_amdgcn_perm(w.y, w.x, h ? 0x07050301u : 0x06040200u);  // groups h, 2+h, ..
    else return w;
  };

  f32x16 acc[TI][TJ];
#pragma unroll
  for (int i = 0; i < TI; ++i)
#pragma unroll
    for (int j = 0; j < TJ; ++j) acc[i][j] = f32x16{};

  // MFMAs [lo, hi) of one k-step's 16 (row-major over the 4 x 4 tiles); the
  // scale byte is picked by the instruction's byte select (BYTE)
  auto mfma = [&](auto BYTE, const Frag *fr, const unsigned *w, int lo = 0, int hi = TI * TJ) {
    constexpr int byte = decltype(BYTE)::value;
#pragma unroll
    for (int i = 0; i < TI; ++i)
#pragma unroll
      for (int j = 0; j < TJ; ++j) {
        if (TJ * i + j < lo || TJ * i + j >= hi) continue;
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
  using P0 = std::integral_constant<int, 0>;
  using P1 = std::integral_constant<int, 1>;

  // fragments of the next k-step to run, and the scale words of its slice
  Frag fr[2][TI + TJ];
  Word wd[TI + TJ];
  RowScales rs_next{};  // row-major scales of the slice after next (SREG)

  if (nslices > 0) {
    load_jobs(P0{}, 0, IC<0>{}, IC<NJ>{});
    load_jobs(P1{}, 1, IC<0>{}, IC<JA + JB>{});  // the rest during slice 0
    if constexpr (SPAN) load_span(0);  // span 1 goes out during slice 0
    if constexpr (SREG) {
      store_row_scales(P0{}, load_row_scales(0));
      rs_next = load_row_scales(1);
    }
    publish_lds_loads();
#pragma unroll
    for (int f = 0; f < TI + TJ; ++f) {
      fr[0][f] = read_frag(P0{}, f, 0);
      wd[f] = read_word(P0{}, IC<0>{}, f, 0);
    }
  }

  // one k-slice ks in slot P (P = ks % 2), at phase H = ks % SPLC of its
  // span (SPAN)
  auto slice = [&](auto Pc, auto Hc, int ks) {
    constexpr int P = decltype(Pc)::value;
    using Q = std::integral_constant<int, P ^ 1>;
    constexpr int H = decltype(Hc)::value;
    using HN = IC<(H + 1) % SPLC>;  // the next slice's phase
    // SPAN: the first slice of span j+1 loads span j+2 into the buffer of
    // span j, whose words every wave has read (the last of them, for span j's
    // last slice, before the barrier that published it), paced among the
    // MFMAs of k-step SPAN_T; span j+2 is first read a whole span later
    constexpr bool SPAN_LOAD = SPAN && H == 0;
    constexpr int SPAN_T = NS == 4 ? 1 : 0;
    // scale byte of k-step t: blocked E4M3 slices are half a span
    auto byte_of = [](auto T) { return std::integral_constant<int, (SL == 1 && FMT == 1 ? 2 * P : 0) + decltype(T)::value>{}; };
    // the slice's scale words (wd is refilled with the next slice's before
    // the last k-step)
    unsigned wcur[TI + TJ];
#pragma unroll
    for (int f = 0; f < TI + TJ; ++f) wcur[f] = word_value(wd[f]);
    // k-steps 0..NS-2, each reading the next step's fragments
    auto step = [&](auto T) {
      constexpr int t = decltype(T)::value;
      constexpr int lo = JA + JB + (t == 0 ? 0 : JS0), cnt = t == 0 ? JS0 : t == 1 ? JS1 : 0;
      mfma(byte_of(T), fr[t & 1], wcur);
#pragma unroll
      for (int f = 0; f < TI + TJ; ++f) fr[(t + 1) & 1][f] = read_frag(Pc, f, t + 1);
      // the rest of the next slice's loads, into the other slot, paced
      if constexpr (cnt > 0) load_jobs(Q{}, ks + 1, IC<lo>{}, IC<lo + cnt>{});
      if constexpr (SPAN_LOAD && t == SPAN_T) load_span(ks / SPLC + 1);
      constexpr int nv = cnt + (SPAN_LOAD && t == SPAN_T ? 2 : 0);
#pragma unroll
      for (int k = 0; k < TI * TJ; ++k) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
        __builtin_amdgcn_sched_group_barrier(0x100, FMT == 0 ? 1 : 2, 0);  // fragment reads
        sched_vmem(spread(k, nv, TI * TJ));
      }
    };
    step(std::integral_constant<int, 0>{});
    if constexpr (NS == 4) {
      step(std::integral_constant<int, 1>{});
      step(std::integral_constant<int, 2>{});
    }
    if constexpr (SREG) store_row_scales(Q{}, rs_next);
    constexpr int AFTER = 8;  // MFMAs after the barrier that publishes the next slice
    const auto last = byte_of(std::integral_constant<int, NS - 1>{});
    if constexpr (!SPLIT) {
      // The last k-step: most of its MFMAs, then the barrier that publishes
      // the next slice (once every wave's loads have landed) and frees this
      // slice's slot, then the rest of the MFMAs overlapping the reads of
      // the next slice's first fragments and the loads of the slice after
      // next into this slot: those loads get a whole slice to land.
      mfma(last, fr[(NS - 1) & 1], wcur, 0, TI * TJ - AFTER);
      publish_lds_loads();
      mfma(last, fr[(NS - 1) & 1], wcur, TI * TJ - AFTER, TI * TJ);
#pragma unroll
      for (int f = 0; f < TI + TJ; ++f) {
        fr[0][f] = read_frag(Q{}, f, 0);
        wd[f] = read_word(Q{}, HN{}, f, ks + 1);
      }
      load_jobs(Pc, ks + 2, IC<0>{}, IC<JB>{});
      if constexpr (SREG) rs_next = load_row_scales(ks + 2);
      constexpr int nv = JB + NSREG;
#pragma unroll
      for (int k = 0; k < AFTER; ++k) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
        __builtin_amdgcn_sched_group_barrier(0x100, 2 * (TI + TJ) / AFTER * (FMT == 0 ? 1 : 2), 0);  // LDS reads
        sched_vmem(spread(k, nv, AFTER));  // loads of the slice after next
      }
    } else {
      // Two barriers.  A (LDS only): every wave has read this slice's last
      // fragments (during the previous k-step), so the slot takes the loads
      // of the slice after next before the last k-step starts.  B, before
      // the last AFTER MFMAs, publishes the next slice: its loads were all
      // issued before the (at least) 16 code loads just issued, and loads
      // complete in order, so waiting until at most 16 are in flight
      // suffices.  Both are written as asm, without the fences of
      // __syncthreads(): at workgroup scope those wait for every
      // outstanding load with an LDS destination (vmcnt(0)), which would
      // give the new loads no time at all.
      asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
      if constexpr (SREG) rs_next = load_row_scales(ks + 2);  // before the loads: waiting for it must not wait for them
      load_jobs(Pc, ks + 2, IC<0>{}, IC<JA>{});
      mfma(last, fr[(NS - 1) & 1], wcur, 0, TI * TJ - AFTER);
#pragma unroll
      for (int k = 0; k < TI * TJ - AFTER; ++k) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
        sched_vmem(spread(k, JA + NSREG, TI * TJ - AFTER));  // loads of the slice after next
      }
      asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(JA + NSREG) : "memory");
      mfma(last, fr[(NS - 1) & 1], wcur, TI * TJ - AFTER, TI * TJ);
#pragma unroll
      for (int f = 0; f < TI + TJ; ++f) {
        fr[0][f] = read_frag(Q{}, f, 0);
        wd[f] = read_word(Q{}, HN{}, f, ks + 1);
      }
      load_jobs(Pc, ks + 2, IC<JA>{}, IC<JA + JB>{});
      constexpr int nv = JB;
#pragma unroll
      for (int k = 0; k < AFTER; ++k) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
        __builtin_amdgcn_sched_group_barrier(0x100, 2 * (TI + TJ) / AFTER * (FMT == 0 ? 1 : 2), 0);  // LDS reads
        sched_vmem(spread(k, nv, AFTER));  // loads of the slice after next
      }
    }
  };

  int ks = 0;
  if constexpr (SPLC == 4 && SPAN) {
    // E4M3 spans: a phase per slice of a span (the launch takes this path
    // only when groups % 16 == 0, so the slices are a multiple of four)
    for (; ks + 3 < nslices; ks += 4) {
      slice(P0{}, IC<0>{}, ks);
      slice(P1{}, IC<1>{}, ks + 1);
      slice(P0{}, IC<2>{}, ks + 2);
      slice(P1{}, IC<3>{}, ks + 3);
    }
  } else {
    // the phase of a two-slice span is the slot parity
    for (; ks + 1 < nslices; ks += 2) {
      slice(P0{}, IC<0>{}, ks);
      slice(P1{}, IC<1 % SPLC>{}, ks + 1);
    }
    if (ks < nslices) slice(P0{}, IC<0>{}, ks);
  }
  // the last slice's prefetch (a re-read of the last slice, never used) is
  // still landing in LDS: drain it before the workgroup can end
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)

  // accumulator: lane l, register a holds C[8(a/4) + 4(l/32) + a%4][l%32]
  //
  // bf16 output of a tile inside C (N % 8 == 0): staged through LDS, so that
  // C is written in 16-byte row pieces.  The accumulator layout holds
  // columns, and its direct 2-byte stores cover 64-byte row segments (7% of
  // the MXFP4 GEMM's time on 8192x8192x28672).  Each wave stages its 128 x
  // 128 quarter in 32 KB of a slot: lane pairs exchange one value so that
  // each lane writes bf16 pairs, then each lane reads 16-byte row pieces
  // back and stores them.
  if (OUT == 0 && m0 + BM <= M && n0 + BN <= N && N % 8 == 0) {
    publish_lds_loads();  // every wave's loads have landed and its fragment reads are done
    uint8_t *reg = (wave >> 1 ? sm1 : sm0) + (wave & 1) * TILE;  // a slot holds two 32 KB regions
    const bool even = (r & 1) == 0;
#pragma unroll
    for (int i = 0; i < TI; ++i)
#pragma unroll
      for (int j = 0; j < TJ; ++j)
#pragma unroll
        for (int a = 0; a < 16; a += 2) {
          const float x0 = alpha * acc[i][j][a], x1 = alpha * acc[i][j][a + 1];
          const unsigned v0 = x0 != x0 ? 0x7FC0u : bf16_rne(x0), v1 = x1 != x1 ? 0x7FC0u : bf16_rne(x1);
          // even lanes keep row a (columns r, r+1), odd lanes row a+1
          // (columns r-1, r)
          const unsigned q = dpp<DPP_QUAD_1032>(even ? v1 : v0);
          const int row = 32 * i + 8 * (a / 4) + 4 * h + a % 4 + (even ? 0 : 1);
          const int col = 32 * j + r - (even ? 0 : 1);
          *(unsigned *)(reg + row * 256 + col * 2) = even ? (v0 | (q << 16)) : (q | (v1 << 16));
        }
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    __builtin_amdgcn_wave_barrier();
    uint16_t *c0 = (uint16_t *)C + (m0 + wm) * N + n0 + wn;
#pragma unroll 8
    for (int k = 0; k < 32; ++k) {
      const int idx = 64 * k + lane, row = idx >> 4, piece = idx & 15;
      const u32x4 v = *(const u32x4 *)(reg + row * 256 + piece * 16);
      __builtin_nontemporal_store(v, (u32x4 *)(c0 + (int64_t)row * N + piece * 8));
    }
    return;
  }
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
    // aligned loads per row when every slice's groups line up, 16-byte spans
    // when the groups of a row are a multiple of 16
    const int ng = fmt == 0 ? GemmShape<0>::NG : GemmShape<1>::NG;
    const bool aligned = (K / 32) % ng == 0 && (uintptr_t)as % 4 == 0 && (uintptr_t)bs % 4 == 0;
    const bool spans = (K / 32) % 16 == 0 && (uintptr_t)as % 16 == 0 && (uintptr_t)bs % 16 == 0;
    if (spans) run_gemm<3, false>(fmt, out_dtype, grid, a, as, b, bs, M, N, K, alpha, c, st);
    else if (aligned) run_gemm_k<2>(fmt, out_dtype, grid, a, as, b, bs, M, N, K, alpha, c, st);
    else run_gemm_k<0>(fmt, out_dtype, grid, a, as, b, bs, M, N, K, alpha, c, st);
  }
  return hipGetLastError();
}

}  // namespace mx
