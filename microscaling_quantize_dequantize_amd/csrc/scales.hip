// Rearrangement of row-major [M x K/32] E8M0 scales into the blocked layout
// read by the gfx950 scaled MFMA (the "to_blocked" step of the pages' MXFP4
// GEMM path, "[Transform] [Quantization] Add QuTLASS support to vLLM",
// review of vllm/qutlass_utils/utils.py, done for this hardware's operand
// order; the layout itself is described in mx_device.h).
#include "launch.h"
#include "mx_device.h"

namespace mx {

constexpr int BT = 256;

// One thread per 32-bit word of the output: word l of block b holds row
// 32*(b / gblocks) + l%32 and groups 8*(b % gblocks) + 2j + l/32, j = 0..3.
__global__ __launch_bounds__(BT) void k_scales_to_blocked(const uint8_t *__restrict__ scales, BlockedScales bl,
                                                          unsigned *__restrict__ out, int64_t n_words) {
  for (int64_t d = (int64_t)blockIdx.x * BT + threadIdx.x; d < n_words; d += (int64_t)gridDim.x * BT) {
    const int64_t b = d >> 6, rb = b / bl.gblocks, kb = b - rb * bl.gblocks;
    const int l = (int)(d & 63);
    const int64_t row = 32 * rb + (l & 31);
    unsigned w = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t g = 8 * kb + 2 * j + (l >> 5);
      const unsigned v = (row < bl.rows && g < bl.groups) ? scales[row * bl.groups + g] : 127u;
      w |= v << (8 * j);
    }
    out[d] = w;
  }
}

hipError_t launch_scales_to_blocked(const uint8_t *scales, const BlockedScales &bl, uint8_t *out,
                                    hipStream_t stream) {
  const int64_t n_words = ((bl.rows + 31) / 32) * bl.gblocks * 64;
  int64_t g = (n_words + BT - 1) / BT;
  if (g > (1 << 20)) g = 1 << 20;
  k_scales_to_blocked<<<(unsigned)g, BT, 0, stream>>>(scales, bl, (unsigned *)out, n_words);
  return hipGetLastError();
}

}  // namespace mx
