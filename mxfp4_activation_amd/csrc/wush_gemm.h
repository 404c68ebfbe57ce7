// Internal interface of the MXFP4 GEMM kernel (wush_gemm.hip) for the C-ABI
// layer.  Not part of the public ABI.
#ifndef WUSH_GEMM_H_
#define WUSH_GEMM_H_

#include <stdint.h>

#include <hip/hip_runtime_api.h>

namespace wush {

struct GemmArgs {
  const uint8_t* a_codes;   // [M][K/2] E2M1 pairs
  const uint8_t* a_scales;  // [M][K/32] E8M0
  const uint8_t* b_codes;   // [N][K/2]
  const uint8_t* b_scales;  // [N][K/32]
  void* C;                  // [M][ldc] fp32 or bf16; columns 0..N-1 written
  int64_t M, N, K;          // K % 256 == 0
  int64_t ldc;              // row stride of C in elements, >= N
};

hipError_t launch_gemm_mxfp4(const GemmArgs& g, bool bf16_out, hipStream_t s);

}  // namespace wush

#endif  // WUSH_GEMM_H_
