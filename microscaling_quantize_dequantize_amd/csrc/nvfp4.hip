// NVFP4 quantize / QDQ / dequantize, unrotated (the rotated forms live with
// the other rotated kernels).
//
// The pages name NVFP4 beside MXFP4 ("[Transform] [Quantization] Add QuTLASS
// support to vLLM", Purpose) and show only its call shape (review of
// benchmarks/kernels/bench_nvfp4_qutlass.py: fusedQuantizeNv(a, rotation,
// global_scale), scales viewed as [-1, K/16]).  The steps, as fp32
// operations rounded to nearest-even (they decide the codes, so they are
// fixed exactly):
//   c6 = g / 6 (per tensor);  q = amax * c6;  scale byte = E4M3(q)
//   (nearest-even, saturating at 448);  m = g / value(scale) (0 for a zero
//   scale);  code = E2M1(x * m) (nearest-even, saturating, sign kept);
//   dequantized value = value(code) * (value(scale) / g).
// Groups are 16 elements, i.e. two 16-byte pieces: a lane pair.
#include "launch.h"
#include "mx_device.h"

namespace mx {

constexpr int64_t NV_MAX_BLOCKS = (int64_t)1 << 22;
constexpr int NV_T = 128, NV_QDQ_U = 2;

// E2M1 codes of the 8 bf16 values of a piece times m (8 nibbles, element 0
// in bits 3:0).
static __device__ __forceinline__ unsigned nv_codes(u32x4 w, float m) {
  const unsigned u[4] = {w.x, w.y, w.z, w.w};
  float v[8];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    v[2 * k] = __uint_as_float(u[k] << 16) * m;
    v[2 * k + 1] = __uint_as_float(u[k] & 0xFFFF0000u) * m;
  }
  unsigned c = fp4_from_f32x2<0>(0u, v[0], v[1], 1.0f);
  c = fp4_from_f32x2<1>(c, v[2], v[3], 1.0f);
  c = fp4_from_f32x2<2>(c, v[4], v[5], 1.0f);
  return fp4_from_f32x2<3>(c, v[6], v[7], 1.0f);
}

// Dequantized fp32 value of nibble k of c.
static __device__ __forceinline__ float nv_value(unsigned c, int k, float kf) {
  return decode_code<0>((c >> (4 * k)) & 0xFu, 0) * kf;
}

// The 8 dequantized values of a code word as bf16.
static __device__ __forceinline__ u32x4 nv_bf16x8(unsigned c, float kf) {
  return u32x4{nv_bf16_pair<0>(c, kf), nv_bf16_pair<1>(c, kf), nv_bf16_pair<2>(c, kf), nv_bf16_pair<3>(c, kf)};
}

// QDQ: one lane per 16-byte piece, a lane pair per 16-group, NV_QDQ_U
// pieces per lane (NV_T apart), whose loads are issued together; the
// per-tensor constants are then formed once per two pieces (measured 3%
// faster than one piece per lane on the 8192 x 57344 layer).
template <bool FAST>
__device__ __forceinline__ void nv_qdq_loop(const u32x4 *__restrict__ src, u32x4 *__restrict__ dst,
                                            const NvTensor &t, int64_t n_pieces) {
  constexpr int64_t SWEEP = NV_T * NV_QDQ_U;
  const int tid = threadIdx.x;
  for (int64_t sweep = blockIdx.x; sweep * SWEEP < n_pieces; sweep += gridDim.x) {
    u32x4 w[NV_QDQ_U];
#pragma unroll
    for (int u = 0; u < NV_QDQ_U; ++u) {
      const int64_t p = sweep * SWEEP + u * NV_T + tid;
      w[u] = p < n_pieces ? __builtin_nontemporal_load(src + p) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < NV_QDQ_U; ++u) {
      const int64_t p = sweep * SWEEP + u * NV_T + tid;
      // group abs-max: this lane's 8 values, then the other lane of the pair
      unsigned mb = 0;
      {
        const u32x4 x = w[u];
        u16x2 a = __builtin_bit_cast(u16x2, x.x & 0x7FFF7FFFu), b = __builtin_bit_cast(u16x2, x.y & 0x7FFF7FFFu);
        u16x2 c = __builtin_bit_cast(u16x2, x.z & 0x7FFF7FFFu), d = __builtin_bit_cast(u16x2, x.w & 0x7FFF7FFFu);
        u16x2 mm = __builtin_elementwise_max(__builtin_elementwise_max(a, b), __builtin_elementwise_max(c, d));
        mb = umax(mm[0], mm[1]);
      }
      mb = umax(mb, dpp<DPP_QUAD_1032>(mb));
      const float amax = __uint_as_float(mb << 16);
      const unsigned sb = nv_scale_byte(amax * t.c6);
      const float sbv = nv_scale_value(sb);
      const u32x4 o = nv_bf16x8(nv_codes(w[u], nv_mul<FAST>(t, sbv)), nv_kf<FAST>(t, sbv));
      if (p < n_pieces) __builtin_nontemporal_store(o, dst + p);
    }
  }
}

__global__ __launch_bounds__(NV_T) void k_nv_qdq(const u32x4 *__restrict__ src, u32x4 *__restrict__ dst,
                                                 const float *__restrict__ gp, int64_t n_pieces) {
  const float g = *gp;
  if (nv_fast(g)) nv_qdq_loop<true>(src, dst, nv_tensor<true>(g), n_pieces);
  else nv_qdq_loop<false>(src, dst, nv_tensor<false>(g), n_pieces);
}

// Quantize with one lane per 16-group (two 16-byte pieces): the scale, its
// value and the quotient g / value are computed once per group instead of
// by both lanes of a pair, and the abs-max needs no lane exchange (measured
// 11% faster on the 8192 x 57344 layer).  Each wave takes 64 consecutive
// groups: its loads stay coalesced (lane l reads pieces l and 64 + l) and a
// wave-private LDS buffer hands each lane its group's two pieces, 9% faster
// than each lane loading its own 32 bytes.  QDQ stays on lane pairs: here
// its output would be two 16-byte stores 32 bytes apart per lane, which
// measured 6% slower than the pairs' contiguous stores.
template <bool FAST>
__device__ __forceinline__ void nv_quant_loop(const u32x4 *__restrict__ src, uint8_t *__restrict__ codes,
                                              uint8_t *__restrict__ scales, const NvTensor &t, int64_t n_groups) {
  __shared__ u32x4 buf[NV_T / 64][128];
  const int lane = threadIdx.x & 63;
  u32x4 *B = buf[threadIdx.x >> 6];
  const int64_t stride = (int64_t)gridDim.x * NV_T;
  for (int64_t base = (int64_t)blockIdx.x * NV_T + (threadIdx.x & ~63); base < n_groups; base += stride) {
    const int64_t p0 = 2 * base, np = 2 * n_groups;
    const u32x4 lo = p0 + lane < np ? __builtin_nontemporal_load(src + p0 + lane) : u32x4{0u, 0u, 0u, 0u};
    const u32x4 hi = p0 + 64 + lane < np ? __builtin_nontemporal_load(src + p0 + 64 + lane) : u32x4{0u, 0u, 0u, 0u};
    B[lane] = lo;
    B[64 + lane] = hi;
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    __builtin_amdgcn_wave_barrier();
    const u32x4 w0 = B[2 * lane], w1 = B[2 * lane + 1];
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    __builtin_amdgcn_wave_barrier();
    const int64_t q = base + lane;
    unsigned mb;
    {
      u16x2 a = __builtin_bit_cast(u16x2, w0.x & 0x7FFF7FFFu), b = __builtin_bit_cast(u16x2, w0.y & 0x7FFF7FFFu);
      u16x2 c = __builtin_bit_cast(u16x2, w0.z & 0x7FFF7FFFu), d = __builtin_bit_cast(u16x2, w0.w & 0x7FFF7FFFu);
      u16x2 e = __builtin_bit_cast(u16x2, w1.x & 0x7FFF7FFFu), f = __builtin_bit_cast(u16x2, w1.y & 0x7FFF7FFFu);
      u16x2 gg = __builtin_bit_cast(u16x2, w1.z & 0x7FFF7FFFu), hh = __builtin_bit_cast(u16x2, w1.w & 0x7FFF7FFFu);
      u16x2 mm = __builtin_elementwise_max(__builtin_elementwise_max(__builtin_elementwise_max(a, b),
                                                                     __builtin_elementwise_max(c, d)),
                                           __builtin_elementwise_max(__builtin_elementwise_max(e, f),
                                                                     __builtin_elementwise_max(gg, hh)));
      mb = umax(mm[0], mm[1]);
    }
    const float amax = __uint_as_float(mb << 16);
    const unsigned sb = nv_scale_byte(amax * t.c6);
    const float m = nv_mul<FAST>(t, nv_scale_value(sb));
    if (q < n_groups) {
      __builtin_nontemporal_store(u32x2{nv_codes(w0, m), nv_codes(w1, m)}, (u32x2 *)codes + q);
      scales[q] = (uint8_t)sb;
    }
  }
}

__global__ __launch_bounds__(NV_T) void k_nv_quant_g(const u32x4 *__restrict__ src, uint8_t *__restrict__ codes,
                                                     uint8_t *__restrict__ scales, const float *__restrict__ gp,
                                                     int64_t n_groups) {
  const float g = *gp;
  if (nv_fast(g)) nv_quant_loop<true>(src, codes, scales, nv_tensor<true>(g), n_groups);
  else nv_quant_loop<false>(src, codes, scales, nv_tensor<false>(g), n_groups);
}

// Dequantize: one lane per 8 elements, U pieces per lane (NV_T apart) whose
// loads are issued together, as in the MX dequantize: two for bf16 output
// (15% faster than one on the 8192 x 57344 layer), one for fp32 output
// (two were 25% slower there).
template <int DT, int U>
__global__ __launch_bounds__(NV_T) void k_nv_dequant(const uint8_t *__restrict__ codes,
                                                     const uint8_t *__restrict__ scales,
                                                     const float *__restrict__ gp, void *__restrict__ dst,
                                                     int64_t n_pieces) {
  constexpr int64_t SWEEP = NV_T * U;
  const float g = *gp;
  for (int64_t sweep = blockIdx.x; sweep * SWEEP < n_pieces; sweep += gridDim.x) {
    unsigned sbs[U], cw[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t p = sweep * SWEEP + u * NV_T + threadIdx.x;
      sbs[u] = p < n_pieces ? scales[p >> 1] : 0u;
      cw[u] = p < n_pieces ? __builtin_nontemporal_load((const unsigned *)codes + p) : 0u;
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t p = sweep * SWEEP + u * NV_T + threadIdx.x;
      if (p >= n_pieces) continue;
      const float kf = nv_scale_value(sbs[u]) / g;
      if (DT == 0) {
        __builtin_nontemporal_store(nv_bf16x8(cw[u], kf), (u32x4 *)dst + p);
      } else {
        unsigned v[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) v[k] = __float_as_uint(nv_value(cw[u], k, kf));
        u32x4 *d = (u32x4 *)dst + 2 * p;
        __builtin_nontemporal_store(u32x4{v[0], v[1], v[2], v[3]}, d);
        __builtin_nontemporal_store(u32x4{v[4], v[5], v[6], v[7]}, d + 1);
      }
    }
  }
}

static unsigned nv_grid(int64_t n_pieces) {
  const int64_t want = (n_pieces + NV_T - 1) / NV_T;
  return (unsigned)(want < NV_MAX_BLOCKS ? want : NV_MAX_BLOCKS);
}

hipError_t launch_nv_unrot(int op, const void *src, void *dst, uint8_t *codes, uint8_t *scales, const float *g,
                           int64_t n, hipStream_t stream) {
  if (op == OP_QDQ) {
    const int64_t np = n / 8;
    k_nv_qdq<<<nv_grid((np + NV_QDQ_U - 1) / NV_QDQ_U), NV_T, 0, stream>>>((const u32x4 *)src, (u32x4 *)dst, g, np);
  } else {
    const int64_t ng = n / 16;
    k_nv_quant_g<<<nv_grid(ng), NV_T, 0, stream>>>((const u32x4 *)src, codes, scales, g, ng);
  }
  return hipGetLastError();
}

hipError_t launch_nv_dequant(int dtype, const uint8_t *codes, const uint8_t *scales, const float *g, void *dst,
                             int64_t n, hipStream_t stream) {
  const int64_t np = n / 8;
  if (dtype == 0) k_nv_dequant<0, 2><<<nv_grid((np + 1) / 2), NV_T, 0, stream>>>(codes, scales, g, dst, np);
  else k_nv_dequant<1, 1><<<nv_grid(np), NV_T, 0, stream>>>(codes, scales, g, dst, np);
  return hipGetLastError();
}

}  // namespace mx
