// Device helpers for the MX kernels (gfx950 / CDNA4 only).
//
// Scale: a group's E8M0 byte comes straight from the exponent field of its
// abs-max (OCP MX v1.0 rule s = floor(log2 amax) - emax_elem, clamped to
// [-127, 127]).
//
// Elements: the CDNA4 scaled conversions v_cvt_scalef32_pk_{fp4,fp8}_{bf16,
// f32} take the scale as an fp32 whose exponent field is the E8M0 byte (so
// byte 0 means 2^-127) and round to nearest-even.  Characterised on gfx950
// against the CPU oracle over every finite bf16 value and every scale byte:
// FP4 matches exactly; FP8 matches exactly once the magnitude is first
// clamped to 448 * 2^s (the hardware returns NaN instead of saturating).  The
// up-conversions to bf16 round to nearest-even, subnormals included.
//
// Software forms of the same steps (quant_mag, decode_mag) are kept for the
// fp32 outputs, where every value is exact in fp32.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mx {

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short i16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

// Element formats: OCP MX v1.0 E2M1 (MXFP4) and E4M3 (MXFP8).
template <int FMT> struct Fmt;
template <> struct Fmt<0> {
  static constexpr int mbits = 1, emin = 0, emax = 2, bias = 1, maxcode = 7;
  static constexpr unsigned sign_bit = 0x8, nan_code = 0x0;
  static constexpr float maxnorm = 6.0f;
};
template <> struct Fmt<1> {
  static constexpr int mbits = 3, emin = -6, emax = 8, bias = 7, maxcode = 126;
  static constexpr unsigned sign_bit = 0x80, nan_code = 0x7F;
  static constexpr float maxnorm = 448.0f;
};

constexpr unsigned BF16_NAN = 0x7FC0u;
constexpr unsigned F32_NAN = 0x7FC00000u;

// E8M0 byte of a group from its abs-max laid out as fp32 bits with the sign
// cleared (a bf16 abs-max is its bits << 16).  The biased exponent e gives
// floor(log2 amax) = e - 127 (e = 0: zero or subnormal, which clamps), so
// byte = clamp(e - 127 - emax, -127, 127) + 127 = max(e - emax, 0).
// 255 marks a group holding NaN or Inf.
template <int FMT>
__device__ __forceinline__ unsigned scale_byte(unsigned amax_bits) {
  int e = (int)(amax_bits >> 23);
  if (e == 255) return 255u;
  int b = e - Fmt<FMT>::emax;
  return b < 0 ? 0u : (unsigned)b;
}

// The scale operand of the scaled conversions: an fp32 whose exponent field
// is the E8M0 byte.
__device__ __forceinline__ float scale_operand(unsigned sb) { return __uint_as_float(sb << 23); }

// bf16 bits of 448 * 2^(sb-127) = 1.75 * 2^(sb-119), replicated in both
// halves: the FP8 saturation bound for a pair of bf16 magnitudes.
__device__ __forceinline__ unsigned e4m3_clamp_bf16x2(unsigned sb) {
  unsigned c = ((sb + 8u) << 7) | 0x60u;
  return c | (c << 16);
}

// Clamp the magnitudes of two packed bf16 values to c (bits), keeping signs.
__device__ __forceinline__ unsigned clamp_bf16x2(unsigned w, unsigned c2) {
  u16x2 m = __builtin_bit_cast(u16x2, w & 0x7FFF7FFFu);
  m = __builtin_elementwise_min(m, __builtin_bit_cast(u16x2, c2));
  return (w & 0x80008000u) | __builtin_bit_cast(unsigned, m);
}

// Clamp an fp32 value to [-c, c] (c > 0): one v_med3_f32.  For a NaN y the
// result is unspecified; every caller replaces the outputs of a group whose
// abs-max is NaN.
__device__ __forceinline__ float clamp_f32(float y, float c) { return __builtin_amdgcn_fmed3f(y, -c, c); }

// Bits of max |v[i]| over N fp32 values, with the IEEE 754-2019 maximum
// (a NaN operand gives a NaN): gfx950's v_maximum3_f32 takes two new values
// per instruction with the absolute value as a source modifier.  For
// non-NaN values this equals the largest of the sign-cleared bit patterns;
// for a NaN it is a positive NaN, exponent field 255, as that largest
// pattern would be, so the scale steps see the same exponent either way.
template <int N>
__device__ __forceinline__ unsigned abs_max_bits(const float *v) {
  float m = __builtin_fabsf(v[0]);
#pragma unroll
  for (int i = 1; i < N; ++i) m = __builtin_elementwise_maximum(m, __builtin_fabsf(v[i]));
  return __float_as_uint(m);
}

// ---- conversions of 8 bf16 (one 16-byte piece) -------------------------

// An empty asm that hides a value from the optimizer.  The ROCm 7.2 middle
// end folds calls of the bf16-source FP4 conversion intrinsic as if their
// result did not depend on the source (distinct calls are merged into one);
// passing each source through this barrier keeps them apart.  It emits no
// instruction.
__device__ __forceinline__ unsigned opaque(unsigned v) {
  asm("" : "+v"(v));
  return v;
}

// E2M1: 8 nibbles, element 2k in the low nibble of byte k.
__device__ __forceinline__ unsigned fp4_from_bf16x8(u32x4 w, float sc) {
  unsigned c = 0;
  c = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(c, __builtin_bit_cast(bf16x2, opaque(w.x)), sc, 0);
  c = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(c, __builtin_bit_cast(bf16x2, opaque(w.y)), sc, 1);
  c = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(c, __builtin_bit_cast(bf16x2, opaque(w.z)), sc, 2);
  c = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(c, __builtin_bit_cast(bf16x2, opaque(w.w)), sc, 3);
  return c;
}

__device__ __forceinline__ u32x4 bf16x8_from_fp4(unsigned c, float sc) {
  u32x4 o;
  o.x = __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(c, sc, 0));
  o.y = __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(c, sc, 1));
  o.z = __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(c, sc, 2));
  o.w = __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(c, sc, 3));
  return o;
}

// E4M3: 8 bytes, element k in byte k; w must already be clamped.
__device__ __forceinline__ unsigned fp8_pair_word(unsigned lo_pair, unsigned hi_pair, float sc) {
  i16x2 c = {0, 0};
  c = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(c, __builtin_bit_cast(bf16x2, lo_pair), sc, false);
  c = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(c, __builtin_bit_cast(bf16x2, hi_pair), sc, true);
  return __builtin_bit_cast(unsigned, c);
}

__device__ __forceinline__ u32x2 fp8_from_bf16x8(u32x4 w, float sc) {
  u32x2 c;
  c.x = fp8_pair_word(w.x, w.y, sc);
  c.y = fp8_pair_word(w.z, w.w, sc);
  return c;
}

__device__ __forceinline__ u32x4 bf16x8_from_fp8(u32x2 c, float sc) {
  u32x4 o;
  o.x = __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c.x, sc, false));
  o.y = __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c.x, sc, true));
  o.z = __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c.y, sc, false));
  o.w = __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c.y, sc, true));
  return o;
}

// ---- conversions of fp32 pairs (rotated values) ---------------------------

// Two fp32 -> one byte of two E2M1 nibbles at byte position SEL of `old`.
template <int SEL>
__device__ __forceinline__ unsigned fp4_from_f32x2(unsigned old, float a, float b, float sc) {
  return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(old, a, b, sc, SEL);
}

// Two fp32 -> two E4M3 bytes in the low (HI=false) or high half of `old`;
// the inputs must already be clamped.
template <bool HI>
__device__ __forceinline__ unsigned fp8_from_f32x2(unsigned old, float a, float b, float sc) {
  i16x2 c = __builtin_bit_cast(i16x2, old);
  c = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(c, a, b, sc, HI);
  return __builtin_bit_cast(unsigned, c);
}

// ---- software element steps (exact in fp32) ------------------------------

// Element value of a magnitude code times 2^s (exact in fp32: at most 4
// significant bits, exponent >= -136).
template <int FMT>
__device__ __forceinline__ float decode_mag(unsigned mag, int s) {
  using F = Fmt<FMT>;
  unsigned ef = mag >> F::mbits;
  unsigned m = mag & ((1u << F::mbits) - 1u);
  int mant = ef ? (int)(m | (1u << F::mbits)) : (int)m;
  int ex = (ef ? (int)ef : 1) - F::bias - F::mbits;
  return __builtin_amdgcn_ldexpf((float)mant, ex + s);
}

// Signed code -> fp32 value times 2^s (NaN for the E4M3 NaN code).
template <int FMT>
__device__ __forceinline__ float decode_code(unsigned code, int s) {
  using F = Fmt<FMT>;
  unsigned mag = code & (F::sign_bit - 1u);
  if (FMT == 1 && mag == 0x7Fu) return __uint_as_float(F32_NAN);
  float v = decode_mag<FMT>(mag, s);
  return (code & F::sign_bit) ? -v : v;
}

// fp32 -> bf16 bits, round to nearest-even (finite or infinite inputs).
__device__ __forceinline__ unsigned bf16_rne(float f) {
  unsigned u = __float_as_uint(f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// Two fp32 -> a packed bf16 pair, nearest-even (the hardware conversion).
__device__ __forceinline__ unsigned bf16x2_rne(float a, float b) {
  return __builtin_bit_cast(unsigned, __builtin_convertvector(f32x2{a, b}, bf16x2));
}

// ---- NVFP4 scale steps --------------------------------------------------------

// E4M3 scale byte of q >= 0, nearest-even and saturating (the hardware
// conversion returns NaN past 448, so q is clamped first; 448 is itself a
// grid value).
__device__ __forceinline__ unsigned nv_scale_byte(float q) {
  return fp8_from_f32x2<false>(0u, fminf(q, 448.0f), 0.0f, 1.0f) & 0xFFu;
}

// fp32 value of an E4M3 scale byte: the hardware conversion (OCP E4M3:
// sign, subnormals, NaN for 0x7F and 0xFF), exact.  The quantize paths only
// produce bytes 0..0x7E; dequantize takes whatever bytes it is given.
__device__ __forceinline__ float nv_scale_value(unsigned sb) {
  return __builtin_amdgcn_cvt_scalef32_f32_fp8(sb, 1.0f, 0);
}

// The two per-group quotients of the NVFP4 steps, m = g / v and
// kf = v / g (v the value of an E4M3 scale byte, g the per-tensor
// multiplier), correctly rounded fp32 like a division, but without one
// while g lies in [2^-60, 2^60] (nv_fast; outside it they divide):
//  - v has at most 4 significant bits, so g / v is never halfway between two
//    fp32 values and lies at least 1/30 ulp from every such midpoint; the
//    Newton-corrected product q + (g - q v) rcp(v), q = g rcp(v), is within
//    2^-16 ulp of g / v for any rcp within 2^-20 and rounds the same way;
//  - v / g lies at least 2^-49 (relative) from every fp32 midpoint; the fp64
//    product v * (1/g) (1/g correctly rounded in fp64) is within 2^-52 of it,
//    so its conversion to fp32 is the correctly rounded quotient.
// The same Newton form gives g / 6 (6 has 2 significant bits).  In range,
// no intermediate overflows, underflows or goes subnormal.  The kernels
// test the range once and run one of two instances of their loop.
__device__ __forceinline__ bool nv_fast(float g) { return g >= 0x1p-60f && g <= 0x1p60f; }

// g / d for d > 0 with at most 4 significant bits and g in range.
__device__ __forceinline__ float nv_div_short(float g, float d) {
  const float y = __builtin_amdgcn_rcpf(d);
  const float q = g * y;
  return __builtin_fmaf(__builtin_fmaf(-q, d, g), y, q);
}

struct NvTensor {
  float g, c6;  // g and g / 6 (fp32, nearest-even)
  double ig;    // 1 / g (fp64, nearest-even)
};

template <bool FAST>
__device__ __forceinline__ NvTensor nv_tensor(float g) {
  return NvTensor{g, FAST ? nv_div_short(g, 6.0f) : g / 6.0f, 1.0 / (double)g};
}

template <bool FAST>
__device__ __forceinline__ float nv_mul(const NvTensor &t, float v) {
  if (!FAST) return v == 0.0f ? 0.0f : t.g / v;
  const float m = nv_div_short(t.g, v);
  return v == 0.0f ? 0.0f : m;
}

template <bool FAST>
__device__ __forceinline__ float nv_kf(const NvTensor &t, float v) {
  return FAST ? (float)((double)v * t.ig) : v / t.g;
}

// Dequantized NVFP4 pair as packed bf16: E2M1 nibbles 2*BYTE and 2*BYTE+1
// of the code word c (exact values from the hardware conversion with scale
// 1), each times kf (fp32, nearest-even), then nearest-even to bf16.
template <int BYTE>
__device__ __forceinline__ unsigned nv_bf16_pair(unsigned c, float kf) {
  const f32x2 v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c, 1.0f, BYTE);
  return bf16x2_rne(v.x * kf, v.y * kf);
}

// ---- blocked scale layout ---------------------------------------------------
// The operand order of the 32x32x64 scaled MFMA: rows padded to 32, groups
// to 8; 256-byte blocks of 32 rows x 8 groups in row-major block order; word
// l of a block holds row l%32 and, in bytes 0..3, groups h, 2+h, 4+h, 6+h of
// the block (h = l/32); padding bytes are 127 (2^0).
// Keeps a selected buffer offset a plain value, so that the compiler does
// not turn "access at (c ? offset : out-of-range)" back into a branch around
// two accesses.
__device__ __forceinline__ void opaque_offset(unsigned &off) { asm volatile("" : "+v"(off)); }

struct BlockedScales {
  int64_t rows, groups, gblocks;  // M, K/32, ceil(K/32 / 8)
};

__device__ __forceinline__ int64_t blocked_offset(int64_t i, int64_t g, int64_t gblocks) {
  return ((((i >> 5) * gblocks) + (g >> 3)) << 8) + 4 * (32 * (g & 1) + (i & 31)) + ((g & 7) >> 1);
}

// Writes the padding bytes (groups past K of every row, then the rows past M)
// with a grid-stride loop over threads t of nt.
__device__ __forceinline__ void write_blocked_pads(uint8_t *__restrict__ out, const BlockedScales &bl, int64_t t,
                                                   int64_t nt) {
  const int64_t gp = bl.gblocks * 8, per_row = gp - bl.groups;
  const int64_t a = bl.rows * per_row, total = a + (((bl.rows + 31) & ~(int64_t)31) - bl.rows) * gp;
  for (; t < total; t += nt) {
    int64_t i, g;
    if (t < a) {
      i = t / per_row;
      g = bl.groups + (t - i * per_row);
    } else {
      i = bl.rows + (t - a) / gp;
      g = (t - a) % gp;
    }
    out[blocked_offset(i, g, bl.gblocks)] = 127;
  }
}

// ---- cross-lane helpers ---------------------------------------------------

// DPP controls (gfx9 encodings).
enum : int {
  DPP_QUAD_1032 = 0xB1,  // quad_perm [1,0,3,2]
  DPP_QUAD_2301 = 0x4E,  // quad_perm [2,3,0,1]
  DPP_ROW_SHL2 = 0x102,  // lane i reads lane i+2 of its row (0 past the row's end)
  DPP_ROW_SHL4 = 0x104,
  DPP_ROW_ROR4 = 0x124,
  DPP_ROW_ROR8 = 0x128,
  DPP_ROW_HALF_MIRROR = 0x141,
};

template <int CTRL>
__device__ __forceinline__ unsigned dpp(unsigned v) {
  return (unsigned)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
}

__device__ __forceinline__ unsigned umax(unsigned a, unsigned b) { return a > b ? a : b; }

// Max of v over lanes l and l^32 (v_permlane32_swap exchanges the upper
// half-wave of its first operand with the lower half-wave of its second).
__device__ __forceinline__ unsigned max_across_halves(unsigned v) {
  auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return umax(r[0], r[1]);
}

// Half-wave exchange (one v_permlane32_swap).  After the call:
//   lanes l < 32:  a = a[l],      b = a[l + 32]
//   lanes l >= 32: a = b[l - 32], b = b[l]
// i.e. the upper half's `a` and the lower half's `b` trade places.
__device__ __forceinline__ void swap_halves(unsigned &a, unsigned &b) {
  auto r = __builtin_amdgcn_permlane32_swap(a, b, false, false);
  a = r[0];
  b = r[1];
}

}  // namespace mx
