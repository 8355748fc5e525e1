// Unrotated MX kernels: fused QDQ, quantize and dequantize.
//
// The matrix is handled as one flat row-major array: K is a multiple of 32,
// so no 32-group straddles a row and group g covers elements [32g, 32g+32),
// with its scale at scales[g] ("use cute-dsl to speedup mxfp QDQ",
// Description: contiguous input, group size 32, K divisible by 32).
//
// bf16 layout on the wave: each lane owns one 16-byte piece (8 elements), so
// 4 consecutive lanes hold one group and a wave reads 1 KiB of contiguous
// input per instruction.  The group abs-max is reduced in registers (packed
// u16 max on sign-cleared bits) and then across the 4 lanes with two DPP
// quad permutations; no LDS is touched.
//
// Launch shape (measured on MI355X, 8192 x 57344 bf16): small blocks, one
// block per THREADS*UNROLL pieces and no persistent loop, stream HBM best --
// QDQ with 64 threads and one piece per thread, quantize with 128 threads
// and two.  The grid is capped only for inputs beyond 2^22 blocks, which
// then loop.
#include "launch.h"
#include "mx_device.h"

namespace mx {

constexpr int64_t MAX_BLOCKS = (int64_t)1 << 22;

__device__ __forceinline__ u32x4 load_piece(const u32x4 *p) { return __builtin_nontemporal_load(p); }

// Sign-cleared u16 maximum of the 8 bf16 values in a piece.
__device__ __forceinline__ unsigned piece_amax_bf16(u32x4 w) {
  u16x2 a = __builtin_bit_cast(u16x2, w.x & 0x7FFF7FFFu);
  u16x2 b = __builtin_bit_cast(u16x2, w.y & 0x7FFF7FFFu);
  u16x2 c = __builtin_bit_cast(u16x2, w.z & 0x7FFF7FFFu);
  u16x2 d = __builtin_bit_cast(u16x2, w.w & 0x7FFF7FFFu);
  u16x2 m = __builtin_elementwise_max(__builtin_elementwise_max(a, b), __builtin_elementwise_max(c, d));
  return umax(m[0], m[1]);
}

// OP_QDQ: dst (bf16) = dequantized values.  OP_QUANT: codes + scales.
// SL (OP_QUANT only): 0 = row-major scales, 1 = the blocked layout `bl`.
template <int FMT, int OP, int THREADS, int UNROLL, int SL>
__global__ __launch_bounds__(THREADS) void k_unrot_bf16(const u32x4 *__restrict__ src,
                                                        u32x4 *__restrict__ dst,
                                                        uint8_t *__restrict__ codes,
                                                        uint8_t *__restrict__ scales,
                                                        int64_t n_pieces, BlockedScales bl) {
  constexpr int64_t SWEEP = THREADS * UNROLL;  // pieces per block per sweep
  const int tid = threadIdx.x;
  if (SL == 1)
    write_blocked_pads(scales, bl, (int64_t)blockIdx.x * THREADS + tid, (int64_t)gridDim.x * THREADS);
  for (int64_t sweep = blockIdx.x; sweep * SWEEP < n_pieces; sweep += gridDim.x) {
    const int64_t base = sweep * SWEEP + tid;
    u32x4 w[UNROLL];
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      const int64_t p = base + (int64_t)u * THREADS;
      w[u] = p < n_pieces ? load_piece(src + p) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      const int64_t p = base + (int64_t)u * THREADS;
      // group abs-max: this lane's 8 values, then the 4 lanes of the group
      unsigned m = piece_amax_bf16(w[u]);
      m = umax(m, dpp<DPP_QUAD_1032>(m));
      m = umax(m, dpp<DPP_QUAD_2301>(m));
      const unsigned sb = scale_byte<FMT>(m << 16);
      const float sc = scale_operand(sb);
      u32x4 x = w[u];
      if (FMT == 1) {
        const unsigned c2 = e4m3_clamp_bf16x2(sb);
        x.x = clamp_bf16x2(x.x, c2);
        x.y = clamp_bf16x2(x.y, c2);
        x.z = clamp_bf16x2(x.z, c2);
        x.w = clamp_bf16x2(x.w, c2);
      }
      if (OP == OP_QDQ) {
        u32x4 o = (FMT == 0) ? bf16x8_from_fp4(fp4_from_bf16x8(x, sc), sc)
                             : bf16x8_from_fp8(fp8_from_bf16x8(x, sc), sc);
        if (sb == 255u) {
          const unsigned nn = BF16_NAN | (BF16_NAN << 16);
          o = u32x4{nn, nn, nn, nn};
        }
        if (p < n_pieces) __builtin_nontemporal_store(o, dst + p);
      } else {
        if (FMT == 0) {
          unsigned c = fp4_from_bf16x8(x, sc);
          if (sb == 255u) c = 0u;
          if (p < n_pieces) __builtin_nontemporal_store(c, (unsigned *)codes + p);
        } else {
          u32x2 c = fp8_from_bf16x8(x, sc);
          if (sb == 255u) c = u32x2{0x7F7F7F7Fu, 0x7F7F7F7Fu};
          if (p < n_pieces) __builtin_nontemporal_store(c, (u32x2 *)codes + p);
        }
        if (SL == 1) {
          // blocked layout: the group's first lane stores its byte
          if ((tid & 3) == 0 && p < n_pieces) {
            const int64_t gf = p >> 2, i = gf / bl.groups;
            scales[blocked_offset(i, gf - i * bl.groups, bl.gblocks)] = (uint8_t)sb;
          }
          continue;
        }
        // Scale bytes: lanes 16k..16k+15 hold 4 consecutive groups; gather
        // the 4 bytes into lane 16k (row rotations by 4 and 8) and store one
        // dword per 4 groups.
        unsigned v = sb << (8 * ((tid >> 2) & 3));
        v |= dpp<DPP_ROW_ROR4>(v);
        v |= dpp<DPP_ROW_ROR8>(v);
        if ((tid & 15) == 0 && p < n_pieces) {
          const int64_t g0 = p >> 2;
          if (p + 16 <= n_pieces) {
            *(unsigned *)(scales + g0) = v;
          } else {
            for (int k = 0; k < 4; ++k)
              if (p + 4 * k < n_pieces) scales[g0 + k] = (uint8_t)(v >> (8 * k));
          }
        }
      }
    }
  }
}

// fp32 source, QDQ only: one 16-byte piece = 4 elements, 8 lanes per group.
template <int FMT, int THREADS, int UNROLL>
__global__ __launch_bounds__(THREADS) void k_unrot_f32(const u32x4 *__restrict__ src,
                                                       u32x4 *__restrict__ dst, int64_t n_pieces) {
  constexpr int64_t SWEEP = THREADS * UNROLL;
  const int tid = threadIdx.x;
  for (int64_t sweep = blockIdx.x; sweep * SWEEP < n_pieces; sweep += gridDim.x) {
    const int64_t base = sweep * SWEEP + tid;
    u32x4 w[UNROLL];
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      const int64_t p = base + (int64_t)u * THREADS;
      w[u] = p < n_pieces ? load_piece(src + p) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      const int64_t p = base + (int64_t)u * THREADS;
      const u32x4 x = w[u];
      const float f[4] = {__uint_as_float(x.x), __uint_as_float(x.y), __uint_as_float(x.z), __uint_as_float(x.w)};
      unsigned m = abs_max_bits<4>(f);
      m = umax(m, dpp<DPP_ROW_HALF_MIRROR>(m));  // lanes i and 7-i of each 8
      m = umax(m, dpp<DPP_QUAD_1032>(m));
      m = umax(m, dpp<DPP_QUAD_2301>(m));
      const unsigned sb = scale_byte<FMT>(m);
      const float sc = scale_operand(sb);
      const int s = (int)sb - 127;
      float y0 = __uint_as_float(x.x), y1 = __uint_as_float(x.y);
      float y2 = __uint_as_float(x.z), y3 = __uint_as_float(x.w);
      unsigned c;
      if (FMT == 0) {
        c = fp4_from_f32x2<0>(0u, y0, y1, sc);
        c = fp4_from_f32x2<1>(c, y2, y3, sc);
      } else {
        const float cl = __uint_as_float(((sb + 8u) << 23) | 0x600000u);  // 448 * 2^s
        c = fp8_from_f32x2<false>(0u, clamp_f32(y0, cl), clamp_f32(y1, cl), sc);
        c = fp8_from_f32x2<true>(c, clamp_f32(y2, cl), clamp_f32(y3, cl), sc);
      }
      constexpr int CB = FMT == 0 ? 4 : 8;  // bits per code
      constexpr unsigned CM = (1u << CB) - 1u;
      u32x4 o;
      o.x = __float_as_uint(decode_code<FMT>(c & CM, s));
      o.y = __float_as_uint(decode_code<FMT>((c >> CB) & CM, s));
      o.z = __float_as_uint(decode_code<FMT>((c >> (2 * CB)) & CM, s));
      o.w = __float_as_uint(decode_code<FMT>((c >> (3 * CB)) & CM, s));
      if (sb == 255u) o = u32x4{F32_NAN, F32_NAN, F32_NAN, F32_NAN};
      if (p < n_pieces) __builtin_nontemporal_store(o, dst + p);
    }
  }
}

// Dequantize: one lane per 8 elements (a quarter group), UNROLL pieces per
// lane (THREADS apart) whose loads are issued together.  For bf16 output two
// pieces measured 17% faster than one for MXFP4 on the 8192 x 57344 layer
// (1% for MXFP8; four were slower); fp32 output, whose lanes already store
// two 16-byte pieces each, stays at one.
template <int FMT, int DT, int THREADS, int UNROLL>
__global__ __launch_bounds__(THREADS) void k_dequant(const uint8_t *__restrict__ codes,
                                                     const uint8_t *__restrict__ scales,
                                                     void *__restrict__ dst, int64_t n_pieces) {
  constexpr int64_t SWEEP = THREADS * UNROLL;
  for (int64_t sweep = blockIdx.x; sweep * SWEEP < n_pieces; sweep += gridDim.x) {
    unsigned sbs[UNROLL], cw[UNROLL][2];
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      const int64_t p = sweep * SWEEP + u * THREADS + threadIdx.x;
      sbs[u] = 0u;
      cw[u][0] = cw[u][1] = 0u;
      if (p < n_pieces) {
        sbs[u] = scales[p >> 2];
        if (FMT == 0) {
          cw[u][0] = __builtin_nontemporal_load((const unsigned *)codes + p);
        } else {
          const u32x2 c = __builtin_nontemporal_load((const u32x2 *)codes + p);
          cw[u][0] = c.x;
          cw[u][1] = c.y;
        }
      }
    }
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      const int64_t p = sweep * SWEEP + u * THREADS + threadIdx.x;
      if (p >= n_pieces) continue;
      const unsigned sb = sbs[u];
      const float sc = scale_operand(sb);
      const int s = (int)sb - 127;
      if (DT == 0) {
        u32x4 o = (FMT == 0) ? bf16x8_from_fp4(cw[u][0], sc) : bf16x8_from_fp8(u32x2{cw[u][0], cw[u][1]}, sc);
        if (sb == 255u) {
          const unsigned nn = BF16_NAN | (BF16_NAN << 16);
          o = u32x4{nn, nn, nn, nn};
        }
        __builtin_nontemporal_store(o, (u32x4 *)dst + p);
      } else {
        constexpr int CB = FMT == 0 ? 4 : 8;
        constexpr unsigned CM = (1u << CB) - 1u;
        unsigned v[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          const unsigned code = (cw[u][(k * CB) / 32] >> ((k * CB) % 32)) & CM;
          v[k] = sb == 255u ? F32_NAN : __float_as_uint(decode_code<FMT>(code, s));
        }
        u32x4 *d = (u32x4 *)dst + 2 * p;
        __builtin_nontemporal_store(u32x4{v[0], v[1], v[2], v[3]}, d);
        __builtin_nontemporal_store(u32x4{v[4], v[5], v[6], v[7]}, d + 1);
      }
    }
  }
}

static unsigned grid_for(int64_t n_pieces, int64_t per_block) {
  const int64_t want = (n_pieces + per_block - 1) / per_block;
  return (unsigned)(want < MAX_BLOCKS ? want : MAX_BLOCKS);
}

// Launch shapes: threads per block and pieces per thread.
// bf16 QDQ runs one-wave blocks: a copy-shaped stream (16 bytes in and 16
// out per lane) measured 2% faster with 64-thread blocks than with 128 or
// 256 (MXFP4 QDQ on the 8192 x 57344 layer 288 -> 281 us, MXFP8 285 -> 282
// us, same-process A/B), while quantize and dequantize, whose streams are
// mostly reads or mostly writes, measured 1-10% slower with them.  fp32
// QDQ, also copy-shaped, likewise: 1% faster than 128 threads (MXFP4 577 ->
// 571 us, MXFP8 568 -> 562 us on the layer in fp32), and 128 threads with
// two pieces, 256 threads, or 64 with two pieces were slower.
constexpr int QDQ_T = 64, QDQ_U = 1;
constexpr int F32_T = 64, F32_U = 1;
constexpr int QNT_T = 128, QNT_U = 2;
constexpr int DEQ_T = 128;
template <int DT> constexpr int deq_unroll() { return DT == 0 ? 2 : 1; }

hipError_t launch_unrot(int fmt, int op, int dtype, const void *src, void *dst, uint8_t *codes,
                        uint8_t *scales, int64_t n, hipStream_t stream, const BlockedScales *bl) {
  const u32x4 *s = (const u32x4 *)src;
  if (dtype == 1) {  // fp32, QDQ only
    const int64_t np = n / 4;
    const unsigned g = grid_for(np, F32_T * F32_U);
    if (fmt == 0) k_unrot_f32<0, F32_T, F32_U><<<g, F32_T, 0, stream>>>(s, (u32x4 *)dst, np);
    else k_unrot_f32<1, F32_T, F32_U><<<g, F32_T, 0, stream>>>(s, (u32x4 *)dst, np);
    return hipGetLastError();
  }
  const int64_t np = n / 8;
  u32x4 *d = (u32x4 *)dst;
  const BlockedScales none{0, 0, 0};
  if (op == OP_QDQ) {
    const unsigned g = grid_for(np, QDQ_T * QDQ_U);
    if (fmt == 0) k_unrot_bf16<0, OP_QDQ, QDQ_T, QDQ_U, 0><<<g, QDQ_T, 0, stream>>>(s, d, nullptr, nullptr, np, none);
    else k_unrot_bf16<1, OP_QDQ, QDQ_T, QDQ_U, 0><<<g, QDQ_T, 0, stream>>>(s, d, nullptr, nullptr, np, none);
  } else {
    const unsigned g = grid_for(np, QNT_T * QNT_U);
    if (bl == nullptr) {
      if (fmt == 0)
        k_unrot_bf16<0, OP_QUANT, QNT_T, QNT_U, 0><<<g, QNT_T, 0, stream>>>(s, nullptr, codes, scales, np, none);
      else
        k_unrot_bf16<1, OP_QUANT, QNT_T, QNT_U, 0><<<g, QNT_T, 0, stream>>>(s, nullptr, codes, scales, np, none);
    } else {
      if (fmt == 0)
        k_unrot_bf16<0, OP_QUANT, QNT_T, QNT_U, 1><<<g, QNT_T, 0, stream>>>(s, nullptr, codes, scales, np, *bl);
      else
        k_unrot_bf16<1, OP_QUANT, QNT_T, QNT_U, 1><<<g, QNT_T, 0, stream>>>(s, nullptr, codes, scales, np, *bl);
    }
  }
  return hipGetLastError();
}

hipError_t launch_dequant(int fmt, int dtype, const uint8_t *codes, const uint8_t *scales,
                          void *dst, int64_t n, hipStream_t stream) {
  const int64_t np = n / 8;
  const unsigned g0 = grid_for(np, DEQ_T * deq_unroll<0>()), g1 = grid_for(np, DEQ_T * deq_unroll<1>());
  if (fmt == 0) {
    if (dtype == 0) k_dequant<0, 0, DEQ_T, deq_unroll<0>()><<<g0, DEQ_T, 0, stream>>>(codes, scales, dst, np);
    else k_dequant<0, 1, DEQ_T, deq_unroll<1>()><<<g1, DEQ_T, 0, stream>>>(codes, scales, dst, np);
  } else {
    if (dtype == 0) k_dequant<1, 0, DEQ_T, deq_unroll<0>()><<<g0, DEQ_T, 0, stream>>>(codes, scales, dst, np);
    else k_dequant<1, 1, DEQ_T, deq_unroll<1>()><<<g1, DEQ_T, 0, stream>>>(codes, scales, dst, np);
  }
  return hipGetLastError();
}

}  // namespace mx
