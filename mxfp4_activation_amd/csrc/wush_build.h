// Launcher of the transform construction kernel (wush_build.hip).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace wush {

struct BuildArgs {
  const uint16_t* W;  // bf16 [d_out][d_in]
  const uint16_t* X;  // bf16 [n_cal][d_in]
  int64_t d_out, n_cal, d_in;
  double damp;        // relative damping lam (>= 0)
  int use_hadamard;   // 1: WUSH, 0: WUS (H = I)
  double* T_wush;     // [d_in/G][G][G]
  double* T_xvsh;
  uint16_t* T_wush_bf16;  // optional bf16(fp32(T)) copies
  uint16_t* T_xvsh_bf16;
};

// G is 16 or 32; the caller has validated sizes, alignment and overlap.
hipError_t launch_build(int G, const BuildArgs& a, hipStream_t s);

// Fixed banks: kind 0 = identity, 1 = normalized Sylvester Hadamard, C
// copies, into float64 and/or bf16 outputs (either may be null).
hipError_t launch_fixed(int kind, int64_t C, int G, double* T, uint16_t* T_bf16, hipStream_t s);

// dst[i] = bf16(fp32(src[i])), i < n.
hipError_t launch_f64_to_bf16(const double* src, int64_t n, uint16_t* dst, hipStream_t s);

}  // namespace wush
