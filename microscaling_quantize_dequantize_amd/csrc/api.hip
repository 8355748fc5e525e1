// C ABI of libmxqdq: argument validation and kernel selection.  Everything
// here runs on the host before the single kernel launch of each call; no
// call allocates, frees or synchronizes.
#include <stdint.h>

#include <atomic>

#include "../../include/libmxqdq.h"
#include "launch.h"

namespace {

thread_local hipStream_t tl_stream = nullptr;

// Largest accepted element count (2^46); far beyond any device memory, and it
// keeps every 64-bit index computation in range.
constexpr int64_t MAX_ELEMS = (int64_t)1 << 46;

bool aligned(const void *p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

int check_fmt(int fmt) { return (fmt == MX_FMT_E2M1 || fmt == MX_FMT_E4M3) ? MX_OK : MX_EFMT; }

int check_dtype(int dt) { return (dt == MX_DTYPE_BF16 || dt == MX_DTYPE_F32) ? MX_OK : MX_EDTYPE; }

int check_shape(int64_t M, int64_t K) {
  if (M < 0 || K < 0 || K % 32 != 0) return MX_ESHAPE;
  if (K > 0 && M > MAX_ELEMS / K) return MX_ESHAPE;
  return MX_OK;
}

int check_rot(const void *rot, int r, int64_t K, bool allow_none) {
  if (r == 0) return allow_none ? MX_OK : MX_EROT;
  if (r != 16 && r != 32 && r != 64 && r != 128) return MX_EROT;
  if (K % r != 0) return MX_EROT;
  if (rot == nullptr) return MX_EROT;
  return MX_OK;
}

int launched(hipError_t e) { return e == hipSuccess ? MX_OK : MX_ELAUNCH; }

}  // namespace

namespace mx {

int device_cu_count() {
  // per device, filled on first use (threads that race here store the same value)
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int n = cache[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cache[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

}  // namespace mx

extern "C" {

MX_API int mx_qdq(int fmt, const void *src, int src_dtype, int64_t M, int64_t K, const void *rot,
                  int rot_size, void *dst) {
  int st;
  if ((st = check_fmt(fmt)) || (st = check_dtype(src_dtype)) || (st = check_shape(M, K)) ||
      (st = check_rot(rot, rot_size, K, true)))
    return st;
  if (M == 0 || K == 0) return MX_OK;
  if (!src || !dst) return MX_ENULL;
  if (!aligned(src, 16) || !aligned(dst, 16) || (rot_size && !aligned(rot, 16))) return MX_EALIGN;
  const int64_t n = M * K;
  if (rot_size == 0)
    return launched(mx::launch_unrot(fmt, mx::OP_QDQ, src_dtype, src, dst, nullptr, nullptr, n, tl_stream));
  return launched(mx::launch_rot(fmt, mx::OP_QDQ, src_dtype, src, rot, rot_size, dst, nullptr, nullptr, n,
                                 tl_stream));
}

MX_API int mx_quantize(int fmt, const void *src, int64_t M, int64_t K, const void *rot, int rot_size,
                       uint8_t *codes, uint8_t *scales) {
  int st;
  if ((st = check_fmt(fmt)) || (st = check_shape(M, K)) || (st = check_rot(rot, rot_size, K, true)))
    return st;
  if (M == 0 || K == 0) return MX_OK;
  if (!src || !codes || !scales) return MX_ENULL;
  if (!aligned(src, 16) || !aligned(codes, 16) || !aligned(scales, 4) || (rot_size && !aligned(rot, 16)))
    return MX_EALIGN;
  const int64_t n = M * K;
  if (rot_size == 0)
    return launched(mx::launch_unrot(fmt, mx::OP_QUANT, MX_DTYPE_BF16, src, nullptr, codes, scales, n,
                                     tl_stream));
  return launched(mx::launch_rot(fmt, mx::OP_QUANT, MX_DTYPE_BF16, src, rot, rot_size, nullptr, codes, scales,
                                 n, tl_stream));
}

MX_API int mx_dequantize(int fmt, const uint8_t *codes, const uint8_t *scales, int64_t M, int64_t K,
                         int dst_dtype, void *dst) {
  int st;
  if ((st = check_fmt(fmt)) || (st = check_dtype(dst_dtype)) || (st = check_shape(M, K))) return st;
  if (M == 0 || K == 0) return MX_OK;
  if (!codes || !scales || !dst) return MX_ENULL;
  if (!aligned(codes, 16) || !aligned(dst, 16)) return MX_EALIGN;
  return launched(mx::launch_dequant(fmt, dst_dtype, codes, scales, dst, M * K, tl_stream));
}

MX_API int mx_rotate(const void *src, int src_dtype, int64_t M, int64_t K, const void *rot, int rot_size,
                     float *dst) {
  int st;
  if ((st = check_dtype(src_dtype)) || (st = check_shape(M, K)) || (st = check_rot(rot, rot_size, K, false)))
    return st;
  if (M == 0 || K == 0) return MX_OK;
  if (!src || !dst) return MX_ENULL;
  if (!aligned(src, 16) || !aligned(dst, 16) || !aligned(rot, 16)) return MX_EALIGN;
  return launched(mx::launch_rot(0, mx::OP_ROTATE, src_dtype, src, rot, rot_size, dst, nullptr, nullptr, M * K,
                                 tl_stream));
}

MX_API int64_t mx_blocked_scales_bytes(int64_t M, int64_t K) {
  if (check_shape(M, K) != MX_OK) return MX_ESHAPE;
  return ((M + 31) / 32) * ((K / 32 + 7) / 8) * 256;
}

MX_API int mx_scales_to_blocked(const uint8_t *scales, int64_t M, int64_t K, uint8_t *blocked) {
  int st;
  if ((st = check_shape(M, K))) return st;
  if (M == 0 || K == 0) return MX_OK;
  if (!scales || !blocked) return MX_ENULL;
  if (!aligned(blocked, 4)) return MX_EALIGN;
  const mx::BlockedScales bl{M, K / 32, (K / 32 + 7) / 8};
  if ((M + 31) / 32 > (int64_t)INT32_MAX || (bl.gblocks + 7) / 8 > 65535) return MX_ESHAPE;  // grid limits
  return launched(mx::launch_scales_to_blocked(scales, bl, blocked, tl_stream));
}

MX_API int mx_quantize_blocked(int fmt, const void *src, int64_t M, int64_t K, const void *rot, int rot_size,
                               uint8_t *codes, uint8_t *blocked_scales) {
  int st;
  if ((st = check_fmt(fmt)) || (st = check_shape(M, K)) || (st = check_rot(rot, rot_size, K, true)))
    return st;
  if (M == 0 || K == 0) return MX_OK;
  if (!src || !codes || !blocked_scales) return MX_ENULL;
  if (!aligned(src, 16) || !aligned(codes, 16) || !aligned(blocked_scales, 4) || (rot_size && !aligned(rot, 16)))
    return MX_EALIGN;
  const mx::BlockedScales bl{M, K / 32, (K / 32 + 7) / 8};
  const int64_t n = M * K;
  if (rot_size == 0)
    return launched(mx::launch_unrot(fmt, mx::OP_QUANT, MX_DTYPE_BF16, src, nullptr, codes, blocked_scales, n,
                                     tl_stream, &bl));
  return launched(mx::launch_rot(fmt, mx::OP_QUANT, MX_DTYPE_BF16, src, rot, rot_size, nullptr, codes,
                                 blocked_scales, n, tl_stream, &bl));
}

MX_API int mx_matmul(int fmt, const uint8_t *a_codes, const uint8_t *a_scales, const uint8_t *b_codes,
                     const uint8_t *b_scales, int scale_layout, int64_t M, int64_t N, int64_t K, float alpha,
                     int out_dtype, void *c) {
  int st;
  if ((st = check_fmt(fmt)) || (st = check_dtype(out_dtype)) || (st = check_shape(M, K)) ||
      (st = check_shape(N, K)))
    return st;
  if (scale_layout != MX_SCALES_ROWMAJOR && scale_layout != MX_SCALES_BLOCKED) return MX_ELAYOUT;
  if (M > ((int64_t)65535 << 7) || (N + 127) / 128 > (int64_t)INT32_MAX) return MX_ESHAPE;  // grid limits
  if ((fmt == MX_FMT_E2M1 ? K / 2 : K) > ((int64_t)1 << 23)) return MX_ESHAPE;  // 32-bit buffer offsets
  if (M == 0 || N == 0) return MX_OK;
  if (!c) return MX_ENULL;
  if (K > 0 && (!a_codes || !a_scales || !b_codes || !b_scales)) return MX_ENULL;
  if (!aligned(a_codes, 16) || !aligned(b_codes, 16) || !aligned(c, 16)) return MX_EALIGN;
  if (scale_layout == MX_SCALES_BLOCKED && (!aligned(a_scales, 4) || !aligned(b_scales, 4))) return MX_EALIGN;
  return launched(mx::launch_gemm(fmt, a_codes, a_scales, b_codes, b_scales, scale_layout, M, N, K, alpha,
                                  out_dtype, c, tl_stream));
}

namespace {

int check_nv(int64_t M, int64_t K, const void *rot, int r) {
  if (M < 0 || K < 0 || K % 16 != 0) return MX_ESHAPE;
  if (K > 0 && M > MAX_ELEMS / K) return MX_ESHAPE;
  if (r != 0 && K % 32 != 0) return MX_EROT;  // rotation blocks hold whole 32-element tiles
  return check_rot(rot, r, K, true);
}

}  // namespace

MX_API int mx_nvfp4_quantize(const void *src, int64_t M, int64_t K, const void *rot, int rot_size,
                             const float *global_scale, uint8_t *codes, uint8_t *scales) {
  int st;
  if ((st = check_nv(M, K, rot, rot_size))) return st;
  if (M == 0 || K == 0) return MX_OK;
  if (!src || !global_scale || !codes || !scales) return MX_ENULL;
  if (!aligned(src, 16) || !aligned(codes, 16) || !aligned(scales, 4) || !aligned(global_scale, 4) ||
      (rot_size && !aligned(rot, 16)))
    return MX_EALIGN;
  if (rot_size == 0)
    return launched(mx::launch_nv_unrot(mx::OP_QUANT, src, nullptr, codes, scales, global_scale, M * K, tl_stream));
  return launched(mx::launch_nv_rot(mx::OP_QUANT, src, rot, rot_size, nullptr, codes, scales, global_scale, M * K,
                                    tl_stream));
}

MX_API int mx_nvfp4_qdq(const void *src, int64_t M, int64_t K, const void *rot, int rot_size,
                        const float *global_scale, void *dst) {
  int st;
  if ((st = check_nv(M, K, rot, rot_size))) return st;
  if (M == 0 || K == 0) return MX_OK;
  if (!src || !global_scale || !dst) return MX_ENULL;
  if (!aligned(src, 16) || !aligned(dst, 16) || !aligned(global_scale, 4) || (rot_size && !aligned(rot, 16)))
    return MX_EALIGN;
  if (rot_size == 0)
    return launched(mx::launch_nv_unrot(mx::OP_QDQ, src, dst, nullptr, nullptr, global_scale, M * K, tl_stream));
  return launched(mx::launch_nv_rot(mx::OP_QDQ, src, rot, rot_size, dst, nullptr, nullptr, global_scale, M * K,
                                    tl_stream));
}

MX_API int mx_nvfp4_dequantize(const uint8_t *codes, const uint8_t *scales, int64_t M, int64_t K,
                               const float *global_scale, int dst_dtype, void *dst) {
  int st;
  if ((st = check_dtype(dst_dtype)) || (st = check_nv(M, K, nullptr, 0))) return st;
  if (M == 0 || K == 0) return MX_OK;
  if (!codes || !scales || !global_scale || !dst) return MX_ENULL;
  if (!aligned(codes, 16) || !aligned(dst, 16) || !aligned(global_scale, 4)) return MX_EALIGN;
  return launched(mx::launch_nv_dequant(dst_dtype, codes, scales, global_scale, dst, M * K, tl_stream));
}

MX_API void mx_set_stream(void *stream) { tl_stream = (hipStream_t)stream; }

MX_API void *mx_get_stream(void) { return (void *)tl_stream; }

MX_API const char *mx_status_string(int status) {
  switch (status) {
    case MX_OK: return "ok";
    case MX_EFMT: return "invalid format (expected MX_FMT_E2M1 or MX_FMT_E4M3)";
    case MX_EDTYPE: return "invalid dtype (expected MX_DTYPE_BF16 or MX_DTYPE_F32)";
    case MX_ESHAPE: return "invalid shape (M, K >= 0, K a multiple of 32, M*K <= 2^46)";
    case MX_EROT: return "invalid rotation (size 16/32/64/128 dividing K, non-NULL matrix)";
    case MX_ENULL: return "a required pointer is NULL";
    case MX_EALIGN: return "misaligned pointer (16 bytes; scales 4 bytes)";
    case MX_ELAUNCH: return "kernel launch failed";
    case MX_ELAYOUT: return "invalid scale layout (expected MX_SCALES_ROWMAJOR or MX_SCALES_BLOCKED)";
    default: return "unknown status";
  }
}

}  // extern "C"
