// Streaming ceilings for the benchmark (not part of libmxqdq).
//
// Three trivial kernels measure what HBM delivers to the simplest access
// pattern on this GPU, so that the MX kernels can be compared with a
// measured ceiling and not only with the nominal 8 TB/s:
//   ceil_copy   dst = src, 16 bytes per lane, non-temporal loads and stores;
//   ceil_read   reads src (16 bytes per lane) and folds it into one word that
//               is stored only if it equals a value the caller passes (so the
//               loads cannot be dropped; the store practically never happens);
//   ceil_write  writes a 32-bit pattern over dst, 16 bytes per lane.
// Each comes in one launch shape per `unroll` (pieces per thread, issued
// together) with 256-thread workgroups, one workgroup per 256 * unroll
// pieces and no persistent loop: the shape the unrotated MX kernels use.
// bytes must be a multiple of 16 and the pointers 16-byte aligned.  Returns
// 0, -1 for a bad argument, or the HIP error of the launch.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

constexpr int THREADS = 256;

template <int U>
__global__ __launch_bounds__(THREADS) void k_copy(const u32x4 *__restrict__ s, u32x4 *__restrict__ d, int64_t n) {
  const int64_t base = (int64_t)blockIdx.x * THREADS * U + threadIdx.x;
  u32x4 v[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int64_t p = base + (int64_t)u * THREADS;
    v[u] = p < n ? __builtin_nontemporal_load(s + p) : u32x4{0u, 0u, 0u, 0u};
  }
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int64_t p = base + (int64_t)u * THREADS;
    if (p < n) __builtin_nontemporal_store(v[u], d + p);
  }
}

template <int U>
__global__ __launch_bounds__(THREADS) void k_read(const u32x4 *__restrict__ s, unsigned *__restrict__ sink, int64_t n,
                                                  unsigned magic) {
  const int64_t base = (int64_t)blockIdx.x * THREADS * U + threadIdx.x;
  unsigned acc = 0;
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int64_t p = base + (int64_t)u * THREADS;
    if (p < n) {
      const u32x4 v = __builtin_nontemporal_load(s + p);
      acc ^= v.x ^ v.y ^ v.z ^ v.w;
    }
  }
  if (acc == magic) sink[0] = acc;
}

template <int U>
__global__ __launch_bounds__(THREADS) void k_write(u32x4 *__restrict__ d, int64_t n, unsigned pattern) {
  const int64_t base = (int64_t)blockIdx.x * THREADS * U + threadIdx.x;
  const u32x4 v = {pattern, pattern, pattern, pattern};
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int64_t p = base + (int64_t)u * THREADS;
    if (p < n) __builtin_nontemporal_store(v, d + p);
  }
}

bool bad(const void *p, int64_t bytes) { return p == nullptr || ((uintptr_t)p & 15u) || bytes < 0 || bytes % 16; }

unsigned grid(int64_t n, int u) { return (unsigned)((n + (int64_t)THREADS * u - 1) / ((int64_t)THREADS * u)); }

}  // namespace

extern "C" {

__attribute__((visibility("default"))) int ceil_copy(const void *src, void *dst, int64_t bytes, int unroll,
                                                     void *stream) {
  if (bad(src, bytes) || bad(dst, bytes) || (unroll != 1 && unroll != 2 && unroll != 4)) return -1;
  const int64_t n = bytes / 16;
  if (n == 0) return 0;
  hipStream_t st = (hipStream_t)stream;
  const u32x4 *s = (const u32x4 *)src;
  u32x4 *d = (u32x4 *)dst;
  if (unroll == 1) k_copy<1><<<grid(n, 1), THREADS, 0, st>>>(s, d, n);
  else if (unroll == 2) k_copy<2><<<grid(n, 2), THREADS, 0, st>>>(s, d, n);
  else k_copy<4><<<grid(n, 4), THREADS, 0, st>>>(s, d, n);
  return (int)hipGetLastError();
}

__attribute__((visibility("default"))) int ceil_read(const void *src, int64_t bytes, void *sink, unsigned magic,
                                                     int unroll, void *stream) {
  if (bad(src, bytes) || bad(sink, 16) || (unroll != 1 && unroll != 2 && unroll != 4)) return -1;
  const int64_t n = bytes / 16;
  if (n == 0) return 0;
  hipStream_t st = (hipStream_t)stream;
  const u32x4 *s = (const u32x4 *)src;
  unsigned *k = (unsigned *)sink;
  if (unroll == 1) k_read<1><<<grid(n, 1), THREADS, 0, st>>>(s, k, n, magic);
  else if (unroll == 2) k_read<2><<<grid(n, 2), THREADS, 0, st>>>(s, k, n, magic);
  else k_read<4><<<grid(n, 4), THREADS, 0, st>>>(s, k, n, magic);
  return (int)hipGetLastError();
}

__attribute__((visibility("default"))) int ceil_write(void *dst, int64_t bytes, unsigned pattern, int unroll,
                                                      void *stream) {
  if (bad(dst, bytes) || (unroll != 1 && unroll != 2 && unroll != 4)) return -1;
  const int64_t n = bytes / 16;
  if (n == 0) return 0;
  hipStream_t st = (hipStream_t)stream;
  u32x4 *d = (u32x4 *)dst;
  if (unroll == 1) k_write<1><<<grid(n, 1), THREADS, 0, st>>>(d, n, pattern);
  else if (unroll == 2) k_write<2><<<grid(n, 2), THREADS, 0, st>>>(d, n, pattern);
  else k_write<4><<<grid(n, 4), THREADS, 0, st>>>(d, n, pattern);
  return (int)hipGetLastError();
}

}  // extern "C"
