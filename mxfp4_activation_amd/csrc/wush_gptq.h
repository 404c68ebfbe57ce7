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

// Float64 GEMM operands: C(i, j) = alpha sum_k A(i, k) B(k, j) + beta C(i, j).
struct GemmF64Args {
  const double* A;
  int64_t sai, sak;  // A(i, k) = A[i * sai + k * sak]
  const double* B;
  int64_t sbk, sbj;  // B(k, j) = B[k * sbk + j * sbj]
  double* C;
  int64_t ldc;       // C(i, j) = C[i * ldc + j]
  int64_t M, N, K;
  double alpha, beta;
  int lower_only;    // skip tiles entirely above the diagonal of C
};

// The whole of GPTQ-WUSH (Algorithm 1) for one layer.
struct GptqWushArgs {
  const double* W;     // [d_out][d_in]
  const double* Xcal;  // [n_cal][d_in]
  int64_t d_out, n_cal, d_in;
  double damp;
  int use_gptq;        // 0: round-to-nearest inside Algorithm 1
  double* Xp;          // [d_in][d_in]: lower Cholesky factor of the damped Hessian
  double* Y;           // [d_out][d_in]: block b's columns = the target block b was fitted to
  double* T_x;         // [d_in/G][G][G]
  double* Wq;          // [d_out][d_in]
  uint8_t* codes;      // [d_out][d_in/2]
  void* scales;        // [d_out][d_in/G]: E8M0 bytes or fp16 bits
};

hipError_t launch_gptq_wush(int fmt, int G, const GptqWushArgs& a, hipStream_t s);

}  // namespace wush
