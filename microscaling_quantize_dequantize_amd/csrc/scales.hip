// Rearrangement of row-major [M x K/32] E8M0 scales into the blocked layout
// read by the gfx950 scaled MFMA (the "to_blocked" step of the pages' MXFP4
// GEMM path, "[Transform] [Quantization] Add QuTLASS support to vLLM",
// review of vllm/qutlass_utils/utils.py, done for this hardware's operand
// order; the layout itself is described in mx_device.h).
#include "launch.h"
#include "mx_device.h"

namespace mx {

constexpr int BT = 256;
constexpr int SPAN = 8;        // group blocks per workgroup (64 groups)
constexpr int TROW = 8 * SPAN + 4;  // LDS row stride in bytes (17 words: conflict-free columns)

// One workgroup per (row block, span of 8 group blocks): the 32 rows x 64
// groups are read row-wise (consecutive threads, consecutive bytes of a
// row) into LDS, then written as 8 whole 256-byte blocks, one 32-bit word
// per thread: word l of a block holds row l%32 and groups 2j + l/32.
__global__ __launch_bounds__(BT) void k_scales_to_blocked(const uint8_t *__restrict__ scales, BlockedScales bl,
                                                          unsigned *__restrict__ out) {
  __shared__ __attribute__((aligned(4))) uint8_t tile[32 * TROW];
  const int t = threadIdx.x;
  const int64_t rb = blockIdx.x, kb0 = (int64_t)blockIdx.y * SPAN;
  {
    const int r = t >> 3, c = t & 7;  // row of the block, 8-group chunk of the span
    const int64_t row = 32 * rb + r, g0 = 8 * (kb0 + c);
    if ((bl.groups & 7) == 0 && ((uintptr_t)scales & 7) == 0 && row < bl.rows && g0 < bl.groups) {
      // a whole, 8-byte aligned chunk; LDS rows are 4-byte aligned
      const u32x2 v = *(const u32x2 *)(scales + row * bl.groups + g0);
      unsigned *d = (unsigned *)(tile + r * TROW + 8 * c);
      d[0] = v.x;
      d[1] = v.y;
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int64_t g = g0 + i;
        tile[r * TROW + 8 * c + i] = (row < bl.rows && g < bl.groups) ? scales[row * bl.groups + g] : (uint8_t)127;
      }
    }
  }
  __syncthreads();
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int w = t + k * BT, b = w >> 6, l = w & 63;
    if (kb0 + b >= bl.gblocks) continue;
    const uint8_t *src = tile + (l & 31) * TROW + 8 * b + (l >> 5);
    const unsigned word = (unsigned)src[0] | ((unsigned)src[2] << 8) | ((unsigned)src[4] << 16) | ((unsigned)src[6] << 24);
    out[(rb * bl.gblocks + kb0 + b) * 64 + l] = word;
  }
}

hipError_t launch_scales_to_blocked(const uint8_t *scales, const BlockedScales &bl, uint8_t *out,
                                    hipStream_t stream) {
  const dim3 grid((unsigned)((bl.rows + 31) / 32), (unsigned)((bl.gblocks + SPAN - 1) / SPAN));
  k_scales_to_blocked<<<grid, BT, 0, stream>>>(scales, bl, (unsigned *)out);
  return hipGetLastError();
}

}  // namespace mx
