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

// Operand layouts: kRowMajor (both [rows][K/2] and [rows][K/32]), kPackedB
// (B in the launch_pack_b layout), kPackedAB (A as the packed quantizer
// writes it, too).
constexpr int kRowMajor = 0, kPackedB = 1, kPackedAB = 2;
hipError_t launch_gemm_mxfp4(const GemmArgs& g, bool bf16_out, int layout, hipStream_t s);

// B [N][K/2] codes and [N][K/32] scales -> the packed layout: per 128-row tile
// and 256-element K step, 16 KB of codes and 1 KB of scales in the order the
// GEMM kernel stages them (rows rounded up to a multiple of 128).
hipError_t launch_pack_b(const uint8_t* codes, const uint8_t* scales, int64_t N, int64_t K, uint8_t* packed_codes,
                         uint8_t* packed_scales, hipStream_t s);

}  // namespace wush

#endif  // WUSH_GEMM_H_
