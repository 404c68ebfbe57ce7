// Dequantization of the three 4-bit formats back to fp32.
//
// Used to evaluate the layerwise loss of joint weight-activation
// quantization ("WUSH: Near-Optimal Adaptive Transforms for LLM
// Quantization", deep dive, section 3.4.1, Eq. 5): the quantized product
// q(T_W W)^T q(T_X X) needs the values the codes stand for.
//
// Value of element k of group c in row m:
//   MXFP4  e2m1(code) * 2^(E8M0 - 127)
//   NVFP4  e2m1(code) * fp32(E4M3(scale) * g)
//   INT4   int4(code) * fp16(scale)
// One thread turns 8 code bytes (16 elements, inside one group for G = 16
// and G = 32) into four 16-byte stores.
#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>
#include <stdint.h>

#include "wush_dequant.h"

namespace wush {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float e2m1_value(uint32_t nib) {
  // E2M1: sign bit 3, exponent bits 2:1 (bias 1), mantissa bit 0; exponent 0
  // is subnormal (0 or 0.5).
  const uint32_t e = (nib >> 1) & 3u, f = nib & 1u;
  const float mag = e == 0 ? 0.5f * (float)f : ldexpf(1.0f + 0.5f * (float)f, (int)e - 1);
  return (nib & 8u) ? -mag : mag;
}

__device__ __forceinline__ float e4m3_value(uint32_t c) {
  // OCP E4M3FN, bias 7, subnormals for exponent 0; only non-negative codes occur.
  const uint32_t e = (c >> 3) & 15u, m = c & 7u;
  return e == 0 ? ldexpf((float)m, -9) : ldexpf((float)(8u + m), (int)e - 10);
}

__device__ __forceinline__ float int4_value(uint32_t nib) { return (float)((int)(nib << 28) >> 28); }

template <int FMT>
__global__ __launch_bounds__(256) void dequant_kernel(const uint8_t* __restrict__ codes, const void* __restrict__ scales,
                                                     const float* __restrict__ gs, int64_t M, int64_t K,
                                                     float* __restrict__ out) {
  constexpr int G = FMT == 1 ? 16 : 32;
  const int64_t per_row = K / 16;  // threads per row
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= M * per_row) return;
  const int64_t m = t / per_row, k0 = (t % per_row) * 16;
  const u32x2 w = *reinterpret_cast<const u32x2*>(codes + m * (K / 2) + k0 / 2);
  const int64_t gi = m * (K / G) + k0 / G;
  float s;
  if (FMT == 0) {
    s = ldexpf(1.0f, (int)reinterpret_cast<const uint8_t*>(scales)[gi] - 127);
  } else if (FMT == 1) {
    s = e4m3_value(reinterpret_cast<const uint8_t*>(scales)[gi]) * gs[0];
  } else {
    s = __half2float(reinterpret_cast<const __half*>(scales)[gi]);
  }
  float v[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const uint32_t nib = (w[i >> 3] >> (4 * (i & 7))) & 15u;
    v[i] = (FMT == 2 ? int4_value(nib) : e2m1_value(nib)) * s;
  }
  f32x4* o = reinterpret_cast<f32x4*>(out + m * K + k0);
#pragma unroll
  for (int q = 0; q < 4; ++q) o[q] = f32x4{v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]};
}

}  // namespace

hipError_t launch_dequant(int fmt, const uint8_t* codes, const void* scales, const float* gs, int64_t M, int64_t K,
                          float* out, hipStream_t s) {
  const int64_t n = M * (K / 16);
  const dim3 grid((unsigned)((n + 255) / 256)), block(256);
  if (fmt == 0) hipLaunchKernelGGL((dequant_kernel<0>), grid, block, 0, s, codes, scales, gs, M, K, out);
  else if (fmt == 1) hipLaunchKernelGGL((dequant_kernel<1>), grid, block, 0, s, codes, scales, gs, M, K, out);
  else hipLaunchKernelGGL((dequant_kernel<2>), grid, block, 0, s, codes, scales, gs, M, K, out);
  return hipGetLastError();
}

}  // namespace wush
