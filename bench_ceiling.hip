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
// Each comes in launch shapes of `threads` (64, 128 or 256) per workgroup
// and `unroll` pieces per thread (1, 2 or 4, issued together), one
// workgroup per threads * unroll pieces and no persistent loop: the shapes
// the unrotated MX kernels use.  bytes must be a multiple of 16 and the
// pointers 16-byte aligned.  Returns 0, -1 for a bad argument, or the HIP
// error of the launch.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

template <int THREADS, int U>
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

template <int THREADS, int U>
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

template <int THREADS, int U>
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

unsigned grid(int64_t n, int t, int u) { return (unsigned)((n + (int64_t)t * u - 1) / ((int64_t)t * u)); }

bool bad_shape(int threads, int unroll) {
  return (threads != 64 && threads != 128 && threads != 256) || (unroll != 1 && unroll != 2 && unroll != 4);
}

// Launches K<T, U> for the runtime shape (threads, unroll).
template <template <int, int> class L, typename... A>
void dispatch(int threads, int unroll, int64_t n, hipStream_t st, A... a) {
  if (threads == 64) {
    if (unroll == 1) L<64, 1>::go(grid(n, 64, 1), st, a...);
    else if (unroll == 2) L<64, 2>::go(grid(n, 64, 2), st, a...);
    else L<64, 4>::go(grid(n, 64, 4), st, a...);
  } else if (threads == 128) {
    if (unroll == 1) L<128, 1>::go(grid(n, 128, 1), st, a...);
    else if (unroll == 2) L<128, 2>::go(grid(n, 128, 2), st, a...);
    else L<128, 4>::go(grid(n, 128, 4), st, a...);
  } else {
    if (unroll == 1) L<256, 1>::go(grid(n, 256, 1), st, a...);
    else if (unroll == 2) L<256, 2>::go(grid(n, 256, 2), st, a...);
    else L<256, 4>::go(grid(n, 256, 4), st, a...);
  }
}

template <int T, int U> struct LCopy {
  static void go(unsigned g, hipStream_t st, const u32x4 *s, u32x4 *d, int64_t n) { k_copy<T, U><<<g, T, 0, st>>>(s, d, n); }
};
template <int T, int U> struct LRead {
  static void go(unsigned g, hipStream_t st, const u32x4 *s, unsigned *k, int64_t n, unsigned m) {
    k_read<T, U><<<g, T, 0, st>>>(s, k, n, m);
  }
};
template <int T, int U> struct LWrite {
  static void go(unsigned g, hipStream_t st, u32x4 *d, int64_t n, unsigned p) { k_write<T, U><<<g, T, 0, st>>>(d, n, p); }
};

}  // namespace

extern "C" {

__attribute__((visibility("default"))) int ceil_copy(const void *src, void *dst, int64_t bytes, int threads,
                                                     int unroll, void *stream) {
  if (bad(src, bytes) || bad(dst, bytes) || bad_shape(threads, unroll)) return -1;
  const int64_t n = bytes / 16;
  if (n == 0) return 0;
  dispatch<LCopy>(threads, unroll, n, (hipStream_t)stream, (const u32x4 *)src, (u32x4 *)dst, n);
  return (int)hipGetLastError();
}

__attribute__((visibility("default"))) int ceil_read(const void *src, int64_t bytes, void *sink, unsigned magic,
                                                     int threads, int unroll, void *stream) {
  if (bad(src, bytes) || bad(sink, 16) || bad_shape(threads, unroll)) return -1;
  const int64_t n = bytes / 16;
  if (n == 0) return 0;
  dispatch<LRead>(threads, unroll, n, (hipStream_t)stream, (const u32x4 *)src, (unsigned *)sink, n, magic);
  return (int)hipGetLastError();
}

__attribute__((visibility("default"))) int ceil_write(void *dst, int64_t bytes, unsigned pattern, int threads,
                                                      int unroll, void *stream) {
  if (bad(dst, bytes) || bad_shape(threads, unroll)) return -1;
  const int64_t n = bytes / 16;
  if (n == 0) return 0;
  dispatch<LWrite>(threads, unroll, n, (hipStream_t)stream, (u32x4 *)dst, n, pattern);
  return (int)hipGetLastError();
}

}  // extern "C"
