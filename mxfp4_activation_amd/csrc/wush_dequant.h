// Launcher of the dequantization kernel (wush_dequant.hip).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace wush {

// fmt 0 = MXFP4, 1 = NVFP4 (gs: device fp32 tensor scale), 2 = INT4.
// codes [M][K/2], scales [M][K/G], out fp32 [M][K]; K % 16 == 0 and the
// caller has checked sizes, alignment (codes 8 B, out 16 B) and grid limits.
hipError_t launch_dequant(int fmt, const uint8_t* codes, const void* scales, const float* gs, int64_t M, int64_t K,
                          float* out, hipStream_t s);

}  // namespace wush
