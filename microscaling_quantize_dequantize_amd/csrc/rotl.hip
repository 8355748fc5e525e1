// Rotated MX and NVFP4 kernels with the rotation matrix held in registers
// and every lane owning whole 16-byte pieces of the output.  The library
// runs MX quantize and NVFP4 QDQ and quantize here (rotation 128); MX QDQ,
// which measured 4-12% slower here, runs on the 16-block short-lived kernel
// of rot.hip.
//
// "[Transform] [Quantization] Add QuTLASS support to vLLM", Online
// rotations: each r-chunk x of a row becomes y = x . R (y[j] = sum_t x[t]
// R[t][j]) before the scale is computed, with R loaded at run time.  These
// kernels serve r = 128 (R itself) and also run r = 16, 32, 64 as the
// 128 x 128 block-diagonal matrix Reff = diag(R, ..., R): the zero blocks add
// exact zeros, and since K is a multiple of r no chunk straddles a row, so
// the matrix is one flat array of 128-element blocks.
//
// Tile: 16 consecutive blocks (4 KiB of bf16).  The contraction runs on
// v_mfma_f32_16x16x32_bf16, D[16 x 16] += A[16 x 32] . B[32 x 16], with the
// tile as A and Reff as B (k = t, 4 steps of 32):
//   A row m   = block beta(m) = 4 (m % 4) + m / 4 of the tile;
//   B column n of j-tile jt = output column pi(16 jt + n) = 8 n + jt;
//   lane l = 16 p + n supplies A[n][8p .. 8p+7] and B[8p .. 8p+7][n] of
//   each k step, and holds D[4p + i][n], i = 0..3, of each j-tile.
// So after the 8 j-tiles, lane (p, n) holds, for i = 0..3, the 8 outputs
// y[block 4i + p][8n .. 8n+7]: piece n of block 4i + p.  For each i the 64
// lanes hold 4 whole blocks (1 KiB of bf16 output) in lane order, a 32-group
// is 4 consecutive lanes (its abs-max takes two DPP steps; an NVFP4 16-group
// is a lane pair, one step), and every output goes from registers straight
// to memory with coalesced stores: the layout of the unrotated kernels.
//
// Data path:
//   - R: each lane loads the 8 x 8 sub-blocks of Reff that its B fragments
//     cover (rows 32 kb + 8p .. +7, columns 8n .. 8n+7: 16 bytes per row,
//     straight from R, zeros off the diagonal blocks) and transposes them in
//     registers (fragment jt is column jt).  The 32 fragments (128 VGPRs)
//     stay in registers for all of the wave's tiles; no LDS and no barrier.
//   - Input tiles go from memory straight into LDS (buffer loads with an LDS
//     destination; each wave instruction fills 1 KiB) into a ring of NB
//     buffers per wave, so that NB - 1 tiles are in flight while one is
//     rotated, without holding registers.  A tile's loads are waited for
//     with an exact vmcnt: the vector-memory operations of a wave complete
//     in issue order, and the count of those issued after them is known.
//   - Piece c of block b sits at 16-byte slot 16 b + (c ^ b) of its buffer,
//     so each 16-lane group of a fragment read (16 blocks, one piece each)
//     is free of bank conflicts; each 16-lane group of a load reads one
//     block's 256 contiguous bytes.
//   - One wave per workgroup, 8 per CU (the register budget allows 2 per
//     SIMD), as a persistent grid whose waves interleave their work units of
//     1 or 2 tiles (wave w takes units w, w + W, w + 2W, ... of the W
//     waves), so that they sweep the tensor together in one contiguous
//     window.  Measured on MI355X (8192 x 57344, rotation 128): against runs
//     of 8 to 64 consecutive tiles per wave and against short-lived
//     workgroups, quantize 4-7% faster; against 4-wave workgroups, MXFP4
//     quantize 3-6% faster.
#include <type_traits>

#include "launch.h"
#include "mx_device.h"

namespace mx {

namespace rl {

constexpr int THREADS = 64;                  // one wave per workgroup (the code also takes 4)
constexpr int WAVES = THREADS / 64;
constexpr int RB = 128;                      // elements per rotation block
constexpr int TB = 16;                       // blocks per tile
constexpr int TILE_ELEMS = TB * RB;          // 2048
constexpr int TILE_BYTES = TILE_ELEMS * 2;   // 4 KiB of bf16
constexpr int RSRC_FLAGS = 0x00020000;       // raw 32-bit buffer
constexpr unsigned OOB_OFFSET = 0x80000000u;  // a buffer offset past every record
constexpr int AUX_NT = 2;                    // cache policy of the tile loads and code stores: non-temporal

template <int NB> struct Lds {
  static constexpr int ring = WAVES * NB * TILE_BYTES;
  static constexpr int bytes = ring + WAVES * 256;  // + one blocked scale unit per wave
};

#define RL_LDS(p) ((__attribute__((address_space(3))) void *)(p))

// Waits until at most N vector-memory operations of this wave are in flight.
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const uint16_t *src, int64_t n_elem, int64_t tile) {
  const int64_t e0 = tile * TILE_ELEMS;
  int64_t left = n_elem - e0;
  left = left < 0 ? 0 : (left > TILE_ELEMS ? TILE_ELEMS : left);
  const uint16_t *base = left > 0 ? src + e0 : src;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t *>(base), (short)0, (int)(left * 2), RSRC_FLAGS);
}

// The MX step of one lane's piece: v[0..7] are 8 consecutive rotated values
// of a 32-group whose other 24 are in the 3 neighbouring lanes of its quad.
template <int FMT>
__device__ __forceinline__ void piece_codes(const float v[8], unsigned &sb, float &sc, u32x2 &c) {
  unsigned m = abs_max_bits<8>(v);
  m = umax(m, dpp<DPP_QUAD_1032>(m));
  m = umax(m, dpp<DPP_QUAD_2301>(m));
  sb = scale_byte<FMT>(m);
  sc = scale_operand(sb);
  if (FMT == 0) {
    unsigned w = fp4_from_f32x2<0>(0u, v[0], v[1], sc);
    w = fp4_from_f32x2<1>(w, v[2], v[3], sc);
    w = fp4_from_f32x2<2>(w, v[4], v[5], sc);
    c.x = fp4_from_f32x2<3>(w, v[6], v[7], sc);
    c.y = 0u;
  } else {
    const float cl = __uint_as_float(((sb + 8u) << 23) | 0x600000u);  // 448 * 2^s
    float y[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) y[e] = clamp_f32(v[e], cl);
    c.x = fp8_from_f32x2<true>(fp8_from_f32x2<false>(0u, y[0], y[1], sc), y[2], y[3], sc);
    c.y = fp8_from_f32x2<true>(fp8_from_f32x2<false>(0u, y[4], y[5], sc), y[6], y[7], sc);
  }
}

// The NVFP4 steps of one lane's piece (8 consecutive rotated values, half of
// a 16-group whose other half is in the neighbouring lane): scale byte, its
// value and the 8 E2M1 codes of x * (g / value), with the fp32 operations of
// the stated NVFP4 steps (nv_mul: the correctly rounded quotient).
template <bool FAST>
__device__ __forceinline__ void piece_nv(const float v[8], const NvTensor &t, unsigned &sb, float &sbv,
                                         unsigned &c) {
  unsigned m = abs_max_bits<8>(v);
  m = umax(m, dpp<DPP_QUAD_1032>(m));
  sb = nv_scale_byte(__uint_as_float(m) * t.c6);
  sbv = nv_scale_value(sb);
  const float mul = nv_mul<FAST>(t, sbv);
  unsigned w = fp4_from_f32x2<0>(0u, v[0] * mul, v[1] * mul, 1.0f);
  w = fp4_from_f32x2<1>(w, v[2] * mul, v[3] * mul, 1.0f);
  w = fp4_from_f32x2<2>(w, v[4] * mul, v[5] * mul, 1.0f);
  c = fp4_from_f32x2<3>(w, v[6] * mul, v[7] * mul, 1.0f);
}

// Vector-memory operations of one tile's stores, for the exact waits: QDQ 4
// (one 16-byte piece per lane and block set); quantize 4 code stores and the
// scale bytes (MX row-major: 1; blocked: 4 byte stores; NVFP4: 4 byte
// stores; blocked by units: none, and one unit store every 4th tile, left
// out of the count, which only makes the waits wait longer).
template <int FMT, int OP, int SL> constexpr int stores_per_tile() {
  return OP == OP_QDQ ? 4 : (SL == 2 ? 4 : (FMT == 2 || SL == 1 ? 8 : 5));
}

// Orders a wave's LDS accesses around an exchange between its lanes.
__device__ __forceinline__ void wave_lds_fence() {
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  __builtin_amdgcn_wave_barrier();
}

// SL 2 epilogue of tile `tile` (tile % 4 is its place in its unit, whose 4
// tiles the wave takes in a row): codes by buffer stores (rows past M and a
// second column block past K are dropped), scale bytes into the wave's unit
// buffer, and after the unit's last tile the unit itself.  Tile block b is
// row r0 + b / 2, column block b % 2; lane (p, n) of set i holds piece n of
// block 4i + p: row r0 + 2i + p / 2, columns c0 + 128 (p % 2) + 8n ..
template <int FMT>
__device__ __forceinline__ void unit_tile_epilogue(const f32x4 (&acc)[8], int64_t tile, int64_t K,
                                                   int64_t col_pairs, const BlockedScales &bl,
                                                   uint8_t *__restrict__ codes, uint8_t *__restrict__ scales,
                                                   int64_t n_elem, uint8_t *unit_bytes, int lane) {
  const int p = lane >> 4, n = lane & 15;
  const int64_t u = tile >> 2;
  const int q = (int)(tile & 3);
  const int64_t r0 = (u / col_pairs) * 32 + 8 * q, c0 = (u % col_pairs) * 256;
  const bool second = c0 + RB < K;  // the unit's second column block exists
  if (q == 0) {
    ((unsigned *)unit_bytes)[lane] = 0x7F7F7F7Fu;  // padding scale 2^0
    wave_lds_fence();
  }
  constexpr int CB = FMT == 0 ? 1 : 2;  // code bytes per 2 elements
  const int64_t e0 = r0 * K + c0;
  int64_t left = (n_elem - e0) * CB / 2;
  const int64_t span = (7 * K + 2 * RB) * CB / 2;
  left = left < 0 ? 0 : (left > span ? span : left);
  const __amdgpu_buffer_rsrc_t rc = __builtin_amdgcn_make_buffer_rsrc(left > 0 ? codes + e0 * CB / 2 : codes, (short)0,
                                                                      (int)left, RSRC_FLAGS);
  const bool lane_cols = second || (p & 1) == 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float v[8];
#pragma unroll
    for (int jt = 0; jt < 8; ++jt) v[jt] = acc[jt][i];
    unsigned sb;
    float sc;
    u32x2 c;
    piece_codes<FMT>(v, sb, sc, c);
    unsigned off = lane_cols ? (unsigned)((((2 * i + (p >> 1)) * K) + RB * (p & 1) + 8 * n) * CB / 2) : OOB_OFFSET;
    opaque_offset(off);
    if (FMT == 0) {
      if (sb == 255u) c.x = 0u;
      __builtin_amdgcn_raw_buffer_store_b32(c.x, rc, off, 0, AUX_NT);
    } else {
      if (sb == 255u) c = u32x2{0x7F7F7F7Fu, 0x7F7F7F7Fu};
      __builtin_amdgcn_raw_buffer_store_b64(c, rc, off, 0, AUX_NT);
    }
    // group n/4 of this block at unit position: word 32 h + row, byte g8 / 2,
    // g8 = 4 (p % 2) + n / 4 the group within the unit, h = g8 % 2
    const int row = 8 * q + 2 * i + (p >> 1), g8 = 4 * (p & 1) + (n >> 2);
    if ((n & 3) == 0 && lane_cols && r0 + 2 * i + (p >> 1) < bl.rows)
      unit_bytes[4 * (32 * (g8 & 1) + row) + (g8 >> 1)] = (uint8_t)sb;
  }
  if (q == 3) {
    wave_lds_fence();
    const unsigned w = ((const unsigned *)unit_bytes)[lane];
    __builtin_nontemporal_store(w, (unsigned *)(scales + u * 256) + lane);
    wave_lds_fence();
  }
}

// The wave's tiles, once its B fragments are in registers.  FMT: 0 MXFP4,
// 1 MXFP8, 2 NVFP4 (g: the per-tensor multiplier; NVFAST selects the
// division-free quotients).  SL (MX quantize): 0 row-major scales, 1 the
// blocked layout `bl` with a byte store per group, 2 the blocked layout by
// whole units (below).
//
// SL 2: a blocked scale unit covers 32 rows x 8 groups (256 columns), so
// its tiles are not 16 consecutive blocks but 8 rows of two 128-column
// blocks: unit u = (row block u / cb, column pair u % cb), cb = ceil(K/256),
// and its 4 tiles q = 0..3 take rows 8q .. 8q+7 of it (UNIT = 4, so a wave
// does a unit's tiles in a row).  The wave gathers the unit's 256 scale bytes in LDS (starting from
// the padding value 127) and writes them with one coalesced 256-byte store.
// Loads past the tensor read as zero and stores past it are dropped by the
// buffer resources, so every tile issues the same stores.
template <int FMT, int OP, int SL, int NB, int UNIT, bool NVFAST>
__device__ __forceinline__ void rot_lanes_tiles(const uint16_t *__restrict__ src, const u32x4 (&rb)[8][4],
                                                uint16_t *__restrict__ dst, uint8_t *__restrict__ codes,
                                                uint8_t *__restrict__ scales, int64_t n_elem,
                                                const BlockedScales &bl, float g, uint8_t *ring,
                                                uint8_t *unit_bytes, int lane, int64_t wave_id, int64_t n_waves) {
  const int p = lane >> 4, n = lane & 15;
  static_assert(SL != 2 || (UNIT == 4 && OP == OP_QUANT && FMT != 2), "unit tiles: MX quantize, 4 per unit");
  static_assert(FMT == 2 || OP == OP_QUANT, "MX QDQ runs on k_rot_t16");
  const int64_t K = SL == 2 ? bl.groups * 32 : 0;
  const int64_t col_pairs = SL == 2 ? bl.gblocks : 1;  // (used only with SL 2)
  const int64_t n_tiles = SL == 2 ? 4 * ((bl.rows + 31) / 32) * col_pairs : (n_elem + TILE_ELEMS - 1) / TILE_ELEMS;
  const int64_t n_units = (n_tiles + UNIT - 1) / UNIT;
  // SL 2: first row and column of a tile, and whether its columns exist
  auto unit_tile = [&](int64_t tile, int64_t &r0, int64_t &c0) -> bool {
    const int64_t u = tile >> 2, q = tile & 3;
    r0 = (u / col_pairs) * 32 + 8 * q;
    c0 = (u % col_pairs) * 256;
    return c0 + RB < K;  // whether the second column block exists
  };
  NvTensor nvt{};
  if constexpr (FMT == 2) nvt = nv_tensor<NVFAST>(g);

  // the k-th tile of this wave is tile (w + (k / UNIT) W) UNIT + k % UNIT;
  // lane s of load instruction q fills slot 64 q + s: block b = 4q + s/16,
  // piece (s % 16) ^ b
  unsigned voff[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int b = 4 * q + (lane >> 4);
    // SL 2: block b is row b / 2, column block b % 2 of the tile
    const unsigned base = SL == 2 ? (unsigned)(2 * (K * (b >> 1) + RB * (b & 1))) : 256u * b;
    voff[q] = base + 16 * ((lane & 15) ^ b);
  }
  auto tile_of = [&](int64_t k) -> int64_t { return (wave_id + (k / UNIT) * n_waves) * UNIT + k % UNIT; };
  auto issue = [&](int64_t k) {
    const int64_t tile = tile_of(k);
    __amdgpu_buffer_rsrc_t rs;
    bool second = true;
    if constexpr (SL == 2) {
      int64_t r0 = 0, c0 = 0;
      second = unit_tile(tile, r0, c0);
      const int64_t e0 = r0 * K + c0;
      int64_t left = tile < n_tiles ? n_elem - e0 : 0;
      const int64_t span = 7 * K + 2 * RB;
      left = left < 0 ? 0 : (left > span ? span : left);
      rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t *>(left > 0 ? src + e0 : src), (short)0,
                                             (int)(left * 2), RSRC_FLAGS);
    } else {
      rs = tile_rsrc(src, n_elem, tile < n_tiles ? tile : n_tiles);
    }
    uint8_t *buf = ring + (int)(k % NB) * TILE_BYTES;
    // SL 2 without a second column block: its lanes (odd block) read zeros
    const bool drop = SL == 2 && !second && ((lane >> 4) & 1);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      unsigned off = drop ? OOB_OFFSET : voff[q];
      opaque_offset(off);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, RL_LDS(buf + 1024 * q), 16, off, 0, 0, AUX_NT);
    }
  };
  // A fragment reads: lane (p, m = n) takes block beta(m), piece 4 kb + p
  const int bm = 4 * (n & 3) + (n >> 2);
  int aslot[4];
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) aslot[kb] = 16 * bm + ((4 * kb + p) ^ bm);

  const int64_t my_units = wave_id < n_units ? (n_units - 1 - wave_id) / n_waves + 1 : 0;
  const int64_t my_tiles = my_units * UNIT;  // tiles past the tensor read as zero and store nothing
#pragma unroll
  for (int k = 0; k < NB - 1; ++k) issue(k);
  constexpr int S = stores_per_tile<FMT, OP, SL>();
  for (int64_t k = 0; k < my_tiles; ++k) {
    issue(k + NB - 1);
    // ops after tile k's loads: the loads of k+1 .. k+NB-1, and the stores
    // of the tiles before k that were issued after them (at most NB - 1)
    if (k >= NB - 1) wait_vm<4 * (NB - 1) + (NB - 1) * S>();
    else if (k == 0) wait_vm<4 * (NB - 1)>();
    else if (k == 1) wait_vm<4 * (NB - 1) + S>();
    else if (k == 2) wait_vm<4 * (NB - 1) + (NB > 3 ? 2 : NB - 1) * S>();
    else if (k == 3) wait_vm<4 * (NB - 1) + (NB > 4 ? 3 : NB - 1) * S>();
    else wait_vm<4 * (NB - 1) + (NB > 5 ? 4 : NB - 1) * S>();
    const int64_t tile = tile_of(k);
    const u32x4 *buf = (const u32x4 *)(ring + (int)(k % NB) * TILE_BYTES);
    u32x4 a[4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) a[kb] = buf[aslot[kb]];
    f32x4 acc[8];
#pragma unroll
    for (int jt = 0; jt < 8; ++jt) {
      acc[jt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
        acc[jt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a[kb]),
                                                          __builtin_bit_cast(bf16x8, rb[jt][kb]), acc[jt], 0, 0, 0);
    }
    if (tile >= n_tiles) continue;  // wave-uniform: nothing to store
    if constexpr (SL == 2) {
      unit_tile_epilogue<FMT>(acc, tile, K, col_pairs, bl, codes, scales, n_elem, unit_bytes, lane);
      continue;
    }
    const int64_t e_tile = tile * TILE_ELEMS;
    // A tile inside the tensor stores every piece: it runs an instance of
    // the epilogue without the per-lane bounds tests.
    auto epilogue = [&](auto full_c) {
      constexpr bool FULL = decltype(full_c)::value;
      unsigned sbw[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float v[8];
#pragma unroll
        for (int jt = 0; jt < 8; ++jt) v[jt] = acc[jt][i];
        // piece n of block 4i + p: elements e_tile + 512 i + 8 lane
        const int64_t e = e_tile + 512 * i + 8 * lane;
        const bool ok = FULL || e < n_elem;
        if constexpr (FMT == 2) {
          unsigned sb, c;
          float sbv;
          piece_nv<NVFAST>(v, nvt, sb, sbv, c);
          if (OP == OP_QDQ) {
            const float kf = nv_kf<NVFAST>(nvt, sbv);
            const u32x4 o = {nv_bf16_pair<0>(c, kf), nv_bf16_pair<1>(c, kf), nv_bf16_pair<2>(c, kf),
                             nv_bf16_pair<3>(c, kf)};
            if (ok) __builtin_nontemporal_store(o, (u32x4 *)(dst + e));
          } else {
            if (ok) __builtin_nontemporal_store(c, (unsigned *)(codes + e / 2));
            if ((lane & 1) == 0 && ok) scales[e >> 4] = (uint8_t)sb;  // the pair's 16-group
          }
          continue;
        } else {
          unsigned sb;
          float sc;
          u32x2 c;
          piece_codes<FMT>(v, sb, sc, c);
          if (FMT == 0) {
            if (sb == 255u) c.x = 0u;
            if (ok) __builtin_nontemporal_store(c.x, (unsigned *)(codes + e / 2));
          } else {
            if (sb == 255u) c = u32x2{0x7F7F7F7Fu, 0x7F7F7F7Fu};
            if (ok) __builtin_nontemporal_store(c, (u32x2 *)(codes + e));
          }
          if (SL == 1) {
            if ((lane & 3) == 0 && ok) {
              const int64_t gf = e >> 5, row = gf / bl.groups;
              scales[blocked_offset(row, gf - row * bl.groups, bl.gblocks)] = (uint8_t)sb;
            }
          } else {
            // lanes 16p .. 16p+15 hold the 4 groups of block 4i + p: after
            // two row rotations every lane of the row holds their 4 bytes
            unsigned w = sb << (8 * ((lane >> 2) & 3));
            w |= dpp<DPP_ROW_ROR4>(w);
            w |= dpp<DPP_ROW_ROR8>(w);
            sbw[i] = w;
          }
        }
      }
      if (FMT != 2 && OP == OP_QUANT && SL == 0) {
        // lane 16p + i (i < 4) stores the 4 scale bytes of block 4i + p
        const int i = lane & 15;
        const unsigned w = i == 0 ? sbw[0] : (i == 1 ? sbw[1] : (i == 2 ? sbw[2] : sbw[3]));
        const int64_t g0 = e_tile / 32 + 16 * i + 4 * p;  // first group of block 4i + p
        if (i < 4) {
          if (FULL || 32 * g0 + RB <= n_elem) {
            *(unsigned *)(scales + g0) = w;
          } else {
            // the tensor ends inside this block (r < 128): its groups up to the end
            for (int q = 0; q < 4; ++q)
              if (32 * (g0 + q) < n_elem) scales[g0 + q] = (uint8_t)(w >> (8 * q));
          }
        }
      }
    };
    if (e_tile + TILE_ELEMS <= n_elem)
      epilogue(std::true_type{});
    else
      epilogue(std::false_type{});
  }
  wait_vm<0>();  // no load may land in LDS after the workgroup has left it
}

template <int FMT, int OP, int SL, int NB, int UNIT>
__global__ __launch_bounds__(THREADS) __attribute__((amdgpu_waves_per_eu(2)))
void k_rot_lanes(const uint16_t *__restrict__ src, const uint16_t *__restrict__ rot, int r,
                 uint16_t *__restrict__ dst, uint8_t *__restrict__ codes, uint8_t *__restrict__ scales,
                 int64_t n_elem, BlockedScales bl, const float *__restrict__ gp) {
  static_assert(NB >= 2 && NB <= 6, "ring of 2 to 6 tiles per wave");
  static_assert(THREADS == 64 || THREADS == 256, "workgroups of 1 or 4 waves");
  __shared__ __attribute__((aligned(1024))) uint8_t lds[Lds<NB>::bytes];
  const int lane = threadIdx.x & 63, p = lane >> 4, n = lane & 15;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform: buffer resources and M0
  const int64_t n_waves = (int64_t)gridDim.x * WAVES;
  const int64_t wave_id = (int64_t)blockIdx.x * WAVES + wave;
  if (SL == 1) write_blocked_pads(scales, bl, (int64_t)blockIdx.x * THREADS + threadIdx.x,
                                  (int64_t)gridDim.x * THREADS);  // SL 2 writes whole units, padding included

  // R into registers: the 8 B fragments of k step kb (jt = 0..7) of lane
  // (p, n) are the 8 x 8 sub-block of Reff at rows 32 kb + 8p .. +7 and
  // columns 8n .. 8n+7 (fragment jt is its column jt)
  u32x4 rrow[4][8];
#pragma unroll
  for (int kb = 0; kb < 4; ++kb)
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int t = 32 * kb + 8 * p + i;
      rrow[kb][i] = (t / r == (8 * n) / r) ? *(const u32x4 *)(rot + (t % r) * r + (8 * n) % r)
                                           : u32x4{0u, 0u, 0u, 0u};
    }
  u32x4 rb[8][4];
#pragma unroll
  for (int kb = 0; kb < 4; ++kb)
#pragma unroll
    for (int jt = 0; jt < 8; ++jt) {
      // element (i, jt) of the sub-block is half jt % 2 of word jt / 2 of row i
      unsigned w[4];
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        const unsigned a = rrow[kb][2 * d][jt >> 1], b = rrow[kb][2 * d + 1][jt >> 1];
        w[d] = (jt & 1) ? ((a >> 16) | (b & 0xFFFF0000u)) : ((a & 0xFFFFu) | (b << 16));
      }
      rb[jt][kb] = u32x4{w[0], w[1], w[2], w[3]};
    }

  uint8_t *ring = lds + wave * NB * TILE_BYTES;
  uint8_t *unit_bytes = lds + Lds<NB>::ring + wave * 256;
  if constexpr (FMT == 2) {
    const float g = *gp;
    if (nv_fast(g))
      rot_lanes_tiles<FMT, OP, SL, NB, UNIT, true>(src, rb, dst, codes, scales, n_elem, bl, g, ring, unit_bytes,
                                                   lane, wave_id, n_waves);
    else
      rot_lanes_tiles<FMT, OP, SL, NB, UNIT, false>(src, rb, dst, codes, scales, n_elem, bl, g, ring, unit_bytes,
                                                    lane, wave_id, n_waves);
  } else {
    rot_lanes_tiles<FMT, OP, SL, NB, UNIT, true>(src, rb, dst, codes, scales, n_elem, bl, 0.0f, ring, unit_bytes,
                                                 lane, wave_id, n_waves);
  }
}

template <int FMT, int OP, int SL, int NB, int UNIT>
static void launch(const void *src, const void *rot, int r, void *dst, uint8_t *codes, uint8_t *scales, int64_t n,
                   hipStream_t st, const BlockedScales &bl, const float *gp, int64_t grid_cap) {
  const int64_t tiles = (n + TILE_ELEMS - 1) / TILE_ELEMS;
  const int64_t units = (tiles + UNIT - 1) / UNIT;
  int64_t g = (units + WAVES - 1) / WAVES;
  if (g > grid_cap) g = grid_cap;
  if (g < 1) g = 1;
  k_rot_lanes<FMT, OP, SL, NB, UNIT><<<(unsigned)g, THREADS, 0, st>>>(
      (const uint16_t *)src, (const uint16_t *)rot, r, (uint16_t *)dst, codes, scales, n, bl, gp);
}

}  // namespace rl

// Launch shape of the lane-owned rotated kernels: tiles in flight per wave
// (NB), workgroups per CU in the persistent grid (PER_CU), and consecutive
// tiles per work unit: 2 for MXFP8 quantize (and NVFP4 QDQ), 1 otherwise.
// Measured on MI355X, 8192 x 57344, rotation 128, the variants interleaved
// in one process: 2-tile units 4% faster than 1 for MXFP8 quantize and
// NVFP4 QDQ, 7% slower for MXFP4 and NVFP4 quantize; 4-tile units slower
// still; a ring of 4 tiles as fast as 5.
constexpr int RL_NB = 4, RL_PER_CU = 8;
template <int FMT, int OP> constexpr int rl_unit() { return (FMT == 1 && OP == OP_QUANT) || (FMT == 2 && OP == OP_QDQ) ? 2 : 1; }

hipError_t launch_rot_lanes(int fmt, int op, const void *src, const void *rot, int r, void *dst, uint8_t *codes,
                            uint8_t *scales, int64_t n, hipStream_t st, const BlockedScales *bl, const float *gp) {
  const int64_t cap = (int64_t)device_cu_count() * RL_PER_CU;
  const BlockedScales none{0, 0, 0};
  const BlockedScales &b = bl ? *bl : none;
  constexpr int NB = RL_NB;
  // MX QDQ at r = 128 runs on the 16-block short-lived kernel (rot.hip),
  // which measured 4-12% faster; this kernel takes MX quantize and NVFP4
  if (fmt == 2) {
    if (op == OP_QDQ) rl::launch<2, OP_QDQ, 0, NB, rl_unit<2, OP_QDQ>()>(src, rot, r, dst, codes, scales, n, st, b, gp, cap);
    else rl::launch<2, OP_QUANT, 0, NB, rl_unit<2, OP_QUANT>()>(src, rot, r, dst, codes, scales, n, st, b, gp, cap);
    return hipGetLastError();
  }
  if (op != OP_QUANT) return hipErrorInvalidValue;
  if (bl == nullptr) {
    if (fmt == 0) rl::launch<0, OP_QUANT, 0, NB, rl_unit<0, OP_QUANT>()>(src, rot, r, dst, codes, scales, n, st, b, gp, cap);
    else rl::launch<1, OP_QUANT, 0, NB, rl_unit<1, OP_QUANT>()>(src, rot, r, dst, codes, scales, n, st, b, gp, cap);
  } else {
    // blocked scales: whole units (4 tiles of 16 rows x 128 columns each)
    if (fmt == 0) rl::launch<0, OP_QUANT, 2, NB, 4>(src, rot, r, dst, codes, scales, n, st, b, gp, cap);
    else rl::launch<1, OP_QUANT, 2, NB, 4>(src, rot, r, dst, codes, scales, n, st, b, gp, cap);
  }
  return hipGetLastError();
}

}  // namespace mx
