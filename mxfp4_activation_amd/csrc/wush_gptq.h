// Launcher of the intra-block GPTQ kernel (wush_gptq.hip).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace wush {

struct GptqArgs {
  const double* Wbar;     // [G][d_out] transformed weights of one block
  const double* R;        // [G][G] upper Cholesky factor of the inverse block Hessian
  int64_t d_out;
  double* Q;              // [G][d_out] dequantized result
  uint8_t* codes;         // row o at codes + o * codes_stride, G/2 bytes
  int64_t codes_stride;   // bytes
  void* scales;           // row o at scales[o * scales_stride] (u8 E8M0 or fp16 bits)
  int64_t scales_stride;  // elements
};

// fmt 0 = MXFP4, 2 = INT4; G = 16 or 32; the caller has validated sizes and alignment.
hipError_t launch_gptq_block(int fmt, int G, const GptqArgs& a, hipStream_t s);

}  // namespace wush
