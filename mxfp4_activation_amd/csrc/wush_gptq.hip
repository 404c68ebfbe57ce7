// Intra-block GPTQ step of GPTQ-WUSH ("WUSH: Near-Optimal Adaptive
// Transforms for LLM Quantization", deep dive, section 3.4.6, Algorithm 1,
// the GPTQ branch) on the GPU.
//
// Input: the transformed weights Wbar of one block, [G][d_out] float64, and
// R, the upper Cholesky factor of the inverse block Hessian (Hd S Hd^T)^-1.
// Every output channel o is an independent quantization group of G values,
// so thread o owns column o (kept in LDS): it takes the group's scale from
// the AbsMax of its G values, then for j = 0..G-1 quantizes w_j at that
// scale and spreads the error over the values not yet quantized,
//     err = (w_j - q_j) / R[j][j],   w_k -= R[j][k] * err   (k > j).
// With R = I this is plain round-to-nearest.
//
// Scales and elements follow the activation quantizers:
//   MXFP4  E8M0 code = floor(log2 amax) - 2 + 127 (clamped at 0); elements
//          fp32(w / 2^e) rounded to E2M1 (nearest even, saturating at 6).
//   INT4   s = fp16(fp32(amax) / 7); elements rne(fp32(w / s)) clamped to +-7.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "wush_gptq.h"

namespace wush {
namespace {

template <int FMT, int G>
__global__ __launch_bounds__(256) void gptq_block_kernel(GptqArgs a) {
  __shared__ double R[G][G];
  __shared__ double Wl[G][256];  // column of thread t in Wl[.][t]
  for (int e = threadIdx.x; e < G * G; e += blockDim.x) R[e / G][e % G] = a.R[e];
  const int t = threadIdx.x;
  const int64_t o = (int64_t)blockIdx.x * blockDim.x + t;
  const bool live = o < a.d_out;
  double amax = 0.0;
  for (int j = 0; j < G; ++j) {
    const double v = live ? a.Wbar[(int64_t)j * a.d_out + o] : 0.0;
    Wl[j][t] = v;
    amax = fmax(amax, fabs(v));
  }
  __syncthreads();
  if (!live) return;
  const float a32 = (float)amax;
  double s;
  uint32_t scode;
  if (FMT == 0) {
    const int be = (int)(__float_as_uint(a32) >> 23);
    scode = (uint32_t)(be > 2 ? be - 2 : 0);
    s = ldexp(1.0, (int)scode - 127);
  } else {
    const _Float16 h = (_Float16)(a32 / 7.0f);
    scode = (uint32_t)__builtin_bit_cast(uint16_t, h);
    s = (double)(float)h;
  }

  uint32_t packed[G / 8];
#pragma unroll
  for (int i = 0; i < G / 8; ++i) packed[i] = 0;
#pragma unroll
  for (int j = 0; j < G; ++j) {
    const double wj = Wl[j][t];
    const float v = s > 0.0 ? (float)(wj / s) : 0.0f;
    uint32_t nib;
    double q;
    if (FMT == 0) {
      // v_cvt_scalef32_pk_fp4_f32 with scale 1.0: E2M1, nearest even, saturating.
      nib = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, v, 0.0f, 1.0f, 0) & 0xFu;
      const uint32_t e = (nib >> 1) & 3u, f = nib & 1u;
      const double mag = e == 0 ? 0.5 * (double)f : ldexp(1.0 + 0.5 * (double)f, (int)e - 1);
      q = ((nib & 8u) ? -mag : mag) * s;
    } else {
      const float r = fminf(fmaxf(__builtin_rintf(v), -7.0f), 7.0f);
      nib = (uint32_t)(int)r & 0xFu;
      q = (double)r * s;
    }
    packed[j / 8] |= nib << (4 * (j % 8));
    a.Q[(int64_t)j * a.d_out + o] = q;
    const double err = (wj - q) / R[j][j];
    for (int k = j + 1; k < G; ++k) Wl[k][t] -= R[j][k] * err;
  }
  uint32_t* cdst = reinterpret_cast<uint32_t*>(a.codes + o * a.codes_stride);
#pragma unroll
  for (int i = 0; i < G / 8; ++i) cdst[i] = packed[i];
  if (FMT == 0)
    reinterpret_cast<uint8_t*>(a.scales)[o * a.scales_stride] = (uint8_t)scode;
  else
    reinterpret_cast<uint16_t*>(a.scales)[o * a.scales_stride] = (uint16_t)scode;
}

}  // namespace

hipError_t launch_gptq_block(int fmt, int G, const GptqArgs& a, hipStream_t s) {
  const dim3 grid((unsigned)((a.d_out + 255) / 256)), block(256);
  if (fmt == 0 && G == 32) hipLaunchKernelGGL((gptq_block_kernel<0, 32>), grid, block, 0, s, a);
  else if (fmt == 0) hipLaunchKernelGGL((gptq_block_kernel<0, 16>), grid, block, 0, s, a);
  else if (G == 32) hipLaunchKernelGGL((gptq_block_kernel<2, 32>), grid, block, 0, s, a);
  else hipLaunchKernelGGL((gptq_block_kernel<2, 16>), grid, block, 0, s, a);
  return hipGetLastError();
}

}  // namespace wush
