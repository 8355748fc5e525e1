// Internal launchers (host side).  Arguments are validated by the C ABI in
// api.hip before any of these is called; n is the element count M*K (> 0,
// a multiple of 32 and of the rotation block).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mx_device.h"

namespace mx {

enum Op { OP_QDQ = 0, OP_QUANT = 1, OP_ROTATE = 2 };

// Number of compute units of the current device (cached per device).
int device_cu_count();

// bl == nullptr: row-major scales; otherwise the blocked layout it describes.
hipError_t launch_unrot(int fmt, int op, int dtype, const void *src, void *dst, uint8_t *codes,
                        uint8_t *scales, int64_t n, hipStream_t stream, const BlockedScales *bl = nullptr);

hipError_t launch_dequant(int fmt, int dtype, const uint8_t *codes, const uint8_t *scales,
                          void *dst, int64_t n, hipStream_t stream);

hipError_t launch_rot(int fmt, int op, int dtype, const void *src, const void *rot, int r,
                      void *dst, uint8_t *codes, uint8_t *scales, int64_t n, hipStream_t stream,
                      const BlockedScales *bl = nullptr);

// bf16 source, any rotation size: the lane-owned kernels of rotl.hip.  fmt
// 0 MXFP4 and 1 MXFP8, quantize only (op OP_QUANT; anything else returns
// hipErrorInvalidValue; bl: blocked scales, or nullptr for row-major), 2
// NVFP4, QDQ or quantize (g: device pointer to the per-tensor multiplier).
hipError_t launch_rot_lanes(int fmt, int op, const void *src, const void *rot, int r, void *dst, uint8_t *codes,
                            uint8_t *scales, int64_t n, hipStream_t stream, const BlockedScales *bl,
                            const float *g = nullptr);

// NVFP4 (g: device pointer to the per-tensor fp32 multiplier; n = M*K).
hipError_t launch_nv_unrot(int op, const void *src, void *dst, uint8_t *codes, uint8_t *scales, const float *g,
                           int64_t n, hipStream_t stream);
hipError_t launch_nv_dequant(int dtype, const uint8_t *codes, const uint8_t *scales, const float *g, void *dst,
                             int64_t n, hipStream_t stream);
hipError_t launch_nv_rot(int op, const void *src, const void *rot, int r, void *dst, uint8_t *codes,
                         uint8_t *scales, const float *g, int64_t n, hipStream_t stream);

hipError_t launch_scales_to_blocked(const uint8_t *scales, const BlockedScales &bl, uint8_t *out,
                                    hipStream_t stream);

// scale_layout 0: row-major [rows x K/32]; 1: the blocked layout.
hipError_t launch_gemm(int fmt, const uint8_t *a, const uint8_t *as, const uint8_t *b, const uint8_t *bs,
                       int scale_layout, int64_t M, int64_t N, int64_t K, float alpha, int out_dtype, void *c,
                       hipStream_t stream);

}  // namespace mx
