// Offline construction of the WUSH transforms on the GPU, one workgroup per
// G x G block, in float64.
//
// "WUSH: Near-Optimal Adaptive Transforms for LLM Quantization":
//   * Blockwise uncentered second moments Sigma_w = d_out^-1 W_(c) W_(c)^T and
//     Sigma_x = d_batch^-1 X_(c) X_(c)^T (papernotes.org, "关键设计"; deep
//     dive, sections 3.2 and 3.4.2), each damped by lam * mean(diag) * I.
//   * Lower Cholesky factors W', X' and the SVD W'^T X' = U S V^T (Eq. 7).
//   * T_wush = H S^-1/2 U^T W'^T (activations) and T_xvsh = H S^-1/2 V^T X'^T
//     (weights) (Eq. 8, deep dive, section 3.4.4); H is the normalized
//     Sylvester Hadamard matrix, or I for the WUS variant.
//   * Singular values in descending order; each pair (u_k, v_k) is signed so
//     that v_k's largest-magnitude entry is positive (ties: lowest index).
//
// Per workgroup (256 threads, block c):
//   1. Moments: rows are staged through LDS 64 at a time as float64; thread t
//      accumulates four entries (G = 32) or one (G = 16) of each moment.
//   2. Damping and the two Cholesky factorizations, one column per step.
//   3. M = W'^T X' and its SVD by one-sided (Hestenes) Jacobi rotations on
//      the columns of M, G/2 disjoint column pairs per round in the
//      round-robin order, G/2 threads per pair, until every pair is
//      orthogonal to rounding level.
//   4. Sort, sign canonicalization, and the two G x G x G products.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "wush_build.h"
#include "wush_f64_block.h"

namespace wush {
namespace {

constexpr int kThreads = 256;
constexpr int kRowsPerChunk = 64;
constexpr int kMaxSweeps = 40;

__device__ __forceinline__ double bf16_to_f64(uint16_t b) { return (double)__uint_as_float((uint32_t)b << 16); }

__device__ __forceinline__ uint16_t f64_to_bf16_via_f32(double v) {
  const uint32_t b = __float_as_uint((float)v);  // round to nearest even
  return (uint16_t)((b + 0x7FFFu + ((b >> 16) & 1u)) >> 16);
}

template <int G>
struct BuildLds {
  double rows[kRowsPerChunk][G + 1];
  double Sw[G][G + 1], Sx[G][G + 1];  // moments, then their Cholesky factors (lower)
  double A[G][G + 1];                  // M = W'^T X', rotated into U S
  double V[G][G + 1];
  double sig[G];
  int perm[G];
  int rotated;
};

// Accumulate the moment of rows [0, R) of a bf16 [R][ld] matrix, block
// columns [c G, c G + G), into dst (divided by R).
template <int G>
__device__ void moment(BuildLds<G>& L, const uint16_t* src, int64_t R, int64_t ld, int c, double (*dst)[G + 1]) {
  const int t = threadIdx.x;
  constexpr int kPer = G * G / kThreads;  // 4 for G = 32, 1 for G = 16
  const int i = (t * kPer) / G, j0 = (t * kPer) % G;
  double acc[kPer];
#pragma unroll
  for (int q = 0; q < kPer; ++q) acc[q] = 0.0;
  constexpr int kPartsPerRow = G / 8;  // 16-byte parts of a row's block
  for (int64_t r0 = 0; r0 < R; r0 += kRowsPerChunk) {
    __syncthreads();
    for (int e = t; e < kRowsPerChunk * kPartsPerRow; e += kThreads) {
      const int rr = e / kPartsPerRow, part = e % kPartsPerRow;
      const int64_t r = r0 + rr;
      uint4 v = make_uint4(0, 0, 0, 0);  // rows past the end contribute zero
      if (r < R) v = *reinterpret_cast<const uint4*>(src + r * ld + (int64_t)c * G + 8 * part);
      const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        L.rows[rr][8 * part + 2 * h] = bf16_to_f64((uint16_t)(w[h] & 0xFFFFu));
        L.rows[rr][8 * part + 2 * h + 1] = bf16_to_f64((uint16_t)(w[h] >> 16));
      }
    }
    __syncthreads();
    const int n = (int)min<int64_t>(kRowsPerChunk, R - r0);
    for (int rr = 0; rr < n; ++rr) {
      const double ai = L.rows[rr][i];
#pragma unroll
      for (int q = 0; q < kPer; ++q) acc[q] = fma(ai, L.rows[rr][j0 + q], acc[q]);
    }
  }
  const double inv = 1.0 / (double)R;
#pragma unroll
  for (int q = 0; q < kPer; ++q) dst[i][j0 + q] = acc[q] * inv;
}

// Damping and in-place lower Cholesky of both moments at once: threads
// [0, G) own the rows of Sigma_w, threads [G, 2G) those of Sigma_x.  Entries
// above the diagonal are zeroed.
template <int G>
__device__ void damp_and_cholesky(BuildLds<G>& L, double lam) {
  const int t = threadIdx.x;
  const bool active = t < 2 * G;
  double(*S)[G + 1] = t < G ? L.Sw : L.Sx;
  const int lane = t % G;
  __syncthreads();
  double md = 0.0;
  if (active) {
    for (int k = 0; k < G; ++k) md += S[k][k];
    md *= lam / (double)G;  // lam * mean(diag)
  }
  __syncthreads();
  if (active) S[lane][lane] += md;
  for (int k = 0; k < G; ++k) {
    __syncthreads();
    if (active && lane == k) {
      double d = S[k][k];
      for (int p = 0; p < k; ++p) d -= S[k][p] * S[k][p];
      S[k][k] = sqrt(d);
    }
    __syncthreads();
    if (active && lane > k) {
      double v = S[lane][k];
      for (int p = 0; p < k; ++p) v -= S[lane][p] * S[k][p];
      S[lane][k] = v / S[k][k];
    }
  }
  __syncthreads();
  if (active)
    for (int j = lane + 1; j < G; ++j) S[lane][j] = 0.0;
  __syncthreads();
}

template <int G>
__global__ __launch_bounds__(kThreads) void build_kernel(BuildArgs a) {
  __shared__ BuildLds<G> L;
  const int c = blockIdx.x;
  const int t = threadIdx.x;

  moment<G>(L, a.W, a.d_out, a.d_in, c, L.Sw);
  moment<G>(L, a.X, a.n_cal, a.d_in, c, L.Sx);

  damp_and_cholesky<G>(L, a.damp);

  // M = W'^T X' (M[i][j] = sum_k W'[k][i] X'[k][j]); V = I.
  for (int e = t; e < G * G; e += kThreads) {
    const int i = e / G, j = e % G;
    double m = 0.0;
    for (int k = max(i, j); k < G; ++k) m = fma(L.Sw[k][i], L.Sx[k][j], m);
    L.A[i][j] = m;
    L.V[i][j] = i == j ? 1.0 : 0.0;
  }

  // SVD of M by one-sided Jacobi on its columns: M V = U S.
  jacobi_columns<G>(L.A, L.V, &L.rotated, kMaxSweeps);

  // Singular values (column norms), descending order, sign rule.
  if (t < G) {
    double s = 0.0;
    for (int i = 0; i < G; ++i) s += L.A[i][t] * L.A[i][t];
    L.sig[t] = sqrt(s);
  }
  __syncthreads();
  if (t < G) {
    int rank = 0;
    for (int j = 0; j < G; ++j) rank += (L.sig[j] > L.sig[t]) || (L.sig[j] == L.sig[t] && j < t);
    L.perm[rank] = t;
  }
  __syncthreads();
  // Thread k: output column k comes from Jacobi column perm[k]; find v_k's
  // largest-magnitude entry and the sign that makes it positive.
  double sgn = 1.0;
  int src = 0;
  if (t < G) {
    src = L.perm[t];
    int lead = 0;
    double best = -1.0;
    for (int i = 0; i < G; ++i) {
      const double m = fabs(L.V[i][src]);
      if (m > best) {
        best = m;
        lead = i;
      }
    }
    sgn = L.V[lead][src] < 0.0 ? -1.0 : 1.0;
  }
  // P_w[k][j] = sgn_k U[j][k] / sqrt(s_k) with U[:, k] = A[:, src] / s_k, and
  // P_x[k][j] = sgn_k V[j][k] / sqrt(s_k); stored over the rows buffer.
  double(*Pw)[G + 1] = reinterpret_cast<double(*)[G + 1]>(&L.rows[0][0]);
  double(*Px)[G + 1] = reinterpret_cast<double(*)[G + 1]>(&L.rows[G][0]);
  static_assert(kRowsPerChunk >= 2 * G, "rows buffer too small for P");
  if (t < G) {
    const double s = L.sig[src];
    const double fu = sgn / (s * sqrt(s)), fv = sgn / sqrt(s);
    for (int j = 0; j < G; ++j) {
      Pw[t][j] = L.A[j][src] * fu;
      Px[t][j] = L.V[j][src] * fv;
    }
  }
  __syncthreads();
  // T = Hd P F^T, with F = W' (activation side) or X' (weight side) and Hd
  // the Hadamard matrix or I.  Q[k][l] = sum_j P[k][j] F[l][j] (j <= l).
  for (int e = t; e < G * G; e += kThreads) {
    const int aa = e / G, l = e % G;
    double tw = 0.0, tx = 0.0;
    for (int k = 0; k < G; ++k) {
      const double h = a.use_hadamard ? hadamard_entry<G>(aa, k) : (aa == k ? 1.0 : 0.0);
      if (h == 0.0) continue;
      double qw = 0.0, qx = 0.0;
      for (int j = 0; j <= l; ++j) {
        qw = fma(Pw[k][j], L.Sw[l][j], qw);
        qx = fma(Px[k][j], L.Sx[l][j], qx);
      }
      tw = fma(h, qw, tw);
      tx = fma(h, qx, tx);
    }
    const int64_t o = (int64_t)c * G * G + e;
    a.T_wush[o] = tw;
    a.T_xvsh[o] = tx;
    if (a.T_wush_bf16) a.T_wush_bf16[o] = f64_to_bf16_via_f32(tw);
    if (a.T_xvsh_bf16) a.T_xvsh_bf16[o] = f64_to_bf16_via_f32(tx);
  }
}

// One thread per entry of the bank: identity (kind 0) or the normalized
// Sylvester Hadamard matrix (kind 1), the same in every block.
template <int G>
__global__ void fixed_kernel(int kind, int64_t n, double* T, uint16_t* T_bf16) {
  const int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= n) return;
  const int i = (int)((e / G) % G), j = (int)(e % G);
  const double v = kind ? hadamard_entry<G>(i, j) : (i == j ? 1.0 : 0.0);
  if (T) T[e] = v;
  if (T_bf16) T_bf16[e] = f64_to_bf16_via_f32(v);
}

__global__ void f64_to_bf16_kernel(const double* __restrict__ src, int64_t n, uint16_t* __restrict__ dst) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride)
    dst[i] = f64_to_bf16_via_f32(src[i]);
}

}  // namespace

hipError_t launch_f64_to_bf16(const double* src, int64_t n, uint16_t* dst, hipStream_t s) {
  int64_t blocks = (n + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(f64_to_bf16_kernel, dim3((unsigned)blocks), dim3(256), 0, s, src, n, dst);
  return hipGetLastError();
}

hipError_t launch_fixed(int kind, int64_t C, int G, double* T, uint16_t* T_bf16, hipStream_t s) {
  const int64_t n = C * G * G;
  const dim3 grid((unsigned)((n + 255) / 256)), block(256);
  if (G == 32) hipLaunchKernelGGL((fixed_kernel<32>), grid, block, 0, s, kind, n, T, T_bf16);
  else hipLaunchKernelGGL((fixed_kernel<16>), grid, block, 0, s, kind, n, T, T_bf16);
  return hipGetLastError();
}

hipError_t launch_build(int G, const BuildArgs& a, hipStream_t s) {
  const dim3 grid((unsigned)(a.d_in / G)), block(kThreads);
  if (G == 32) hipLaunchKernelGGL((build_kernel<32>), grid, block, 0, s, a);
  else hipLaunchKernelGGL((build_kernel<16>), grid, block, 0, s, a);
  return hipGetLastError();
}

}  // namespace wush
