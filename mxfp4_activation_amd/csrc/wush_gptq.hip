// GPTQ-WUSH ("WUSH: Near-Optimal Adaptive Transforms for LLM
// Quantization", deep dive, section 3.4.6, Algorithm 1) on the GPU, in
// float64: the weight side is calibrated block by block in reverse order,
// interleaving the transform construction with GPTQ.
//
//   1. Hx = Xcal^T Xcal / n, damped by damp * mean(diag(Hx)) * I; X' its lower
//      Cholesky factor (blocked: panel factorization, triangular solve of
//      the rows below, update of the trailing matrix).
//   2. Y = W X'.
//   3. For b = C-1 .. 0 (gptq_wush_block_kernel; each workgroup of the
//      launch derives the block's transforms, then takes 256 channels):
//        the SVD of Y_b = Y[:, b] through its Gram matrix Y_b^T Y_b, whose
//        eigenvectors V (one-sided Jacobi) and eigenvalues s^2 give
//        U = Y_b V S^-1; each (u_k, v_k) signed so that v_k's largest entry
//        is positive; S <- S / sqrt(d_out);
//        T_X = Hd S^1/2 V^T X'[b, b]^-1 (the activation transform used online);
//        Wbar = sqrt(d_out) Hd S^1/2 U^T = sqrt(d_out) Hd S^1/2 S^-1 V^T Y_b^T;
//        GPTQ of Wbar with the block Hessian Hd S Hd^T, or round-to-nearest;
//      then Y[:, < b] -= Wsub^T T_X X'[b, < b] (Wsub: the quantized block for
//      GPTQ, Wbar for round-to-nearest), a float64 GEMM.
//   4. Wq = the dequantized codes.
//
// Intra-block step: every output channel o is an independent quantization
// group of G values.  Its scale comes from the AbsMax of the group's Wbar;
// then for j = 0..G-1, w_j is quantized at that scale and the error spread
// over the values not yet quantized,
//     err = (w_j - q_j) / R[j][j],   w_k -= R[j][k] * err   (k > j),
// with R the upper Cholesky factor of the inverse block Hessian
// (R = I: plain round-to-nearest).
//
// Scales and elements follow the activation quantizers:
//   MXFP4  E8M0 code = floor(log2 amax) - 2 + 127 (clamped at 0); elements
//          fp32(w / 2^e) rounded to E2M1 (nearest even, saturating at 6).
//   INT4   s = fp16(fp32(amax) / 7); elements rne(fp32(w / s)) clamped to +-7.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "wush_f64_block.h"
#include "wush_gptq.h"

namespace wush {
namespace {

// Scale of one group from its AbsMax: the stored code (E8M0 byte or fp16
// bits) and its value.
template <int FMT>
__device__ __forceinline__ double group_scale(double amax, uint32_t& scode) {
  const float a32 = (float)amax;
  if (FMT == 0) {
    const int be = (int)(__float_as_uint(a32) >> 23);
    scode = (uint32_t)(be > 2 ? be - 2 : 0);
    return ldexp(1.0, (int)scode - 127);
  }
  const _Float16 h = (_Float16)(a32 / 7.0f);
  scode = (uint32_t)__builtin_bit_cast(uint16_t, h);
  return (double)(float)h;
}

// Value of a nibble code at scale s.
template <int FMT>
__device__ __forceinline__ double code_value(uint32_t nib, double s) {
  if (FMT == 0) {
    const uint32_t e = (nib >> 1) & 3u, f = nib & 1u;
    const double mag = e == 0 ? 0.5 * (double)f : ldexp(1.0 + 0.5 * (double)f, (int)e - 1);
    return ((nib & 8u) ? -mag : mag) * s;
  }
  return (double)((int)(nib << 28) >> 28) * s;
}

// One output channel's G transformed weights, an LDS column w (element k at
// w[k * WS]; updated in place), quantized with the error feedback of R (in
// LDS, row stride G).  Writes the dequantized values to q and the nibbles
// to packed; returns the scale code.  With R = I the column is unchanged.
template <int FMT, int G, int WS>
__device__ __forceinline__ uint32_t quant_channel(double* w, const double* R, double (&q)[G],
                                                  uint32_t (&packed)[G / 8]) {
  double amax = 0.0;
#pragma unroll
  for (int j = 0; j < G; ++j) amax = fmax(amax, fabs(w[j * WS]));
  uint32_t scode;
  const double s = group_scale<FMT>(amax, scode);
#pragma unroll
  for (int i = 0; i < G / 8; ++i) packed[i] = 0;
#pragma unroll
  for (int j = 0; j < G; ++j) {
    const double wj = w[j * WS];
    const float v = s > 0.0 ? (float)(wj / s) : 0.0f;
    uint32_t nib;
    if (FMT == 0) {
      // v_cvt_scalef32_pk_fp4_f32 with scale 1.0: E2M1, nearest even, saturating.
      nib = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, v, 0.0f, 1.0f, 0) & 0xFu;
    } else {
      const float r = fminf(fmaxf(__builtin_rintf(v), -7.0f), 7.0f);
      nib = (uint32_t)(int)r & 0xFu;
    }
    q[j] = code_value<FMT>(nib, s);
    packed[j / 8] |= nib << (4 * (j % 8));
    const double err = (wj - q[j]) / R[j * G + j];
    for (int k = j + 1; k < G; ++k) w[k * WS] -= R[j * G + k] * err;
  }
  return scode;
}

template <int FMT, int G>
__global__ __launch_bounds__(256) void gptq_block_kernel(GptqArgs a) {
  __shared__ double R[G * G];
  __shared__ double Wl[G][256];  // column of thread t in Wl[.][t]
  for (int e = threadIdx.x; e < G * G; e += blockDim.x) R[e] = a.R[e];
  __syncthreads();
  const int t = threadIdx.x;
  const int64_t o = (int64_t)blockIdx.x * blockDim.x + t;
  if (o >= a.d_out) return;
  double q[G];
#pragma unroll
  for (int j = 0; j < G; ++j) Wl[j][t] = a.Wbar[(int64_t)j * a.d_out + o];
  uint32_t packed[G / 8];
  const uint32_t scode = quant_channel<FMT, G, 256>(&Wl[0][t], R, q, packed);
#pragma unroll
  for (int j = 0; j < G; ++j) a.Q[(int64_t)j * a.d_out + o] = q[j];
  uint32_t* cdst = reinterpret_cast<uint32_t*>(a.codes + o * a.codes_stride);
#pragma unroll
  for (int i = 0; i < G / 8; ++i) cdst[i] = packed[i];
  if (FMT == 0)
    reinterpret_cast<uint8_t*>(a.scales)[o * a.scales_stride] = (uint8_t)scode;
  else
    reinterpret_cast<uint16_t*>(a.scales)[o * a.scales_stride] = (uint16_t)scode;
}

// ---------------------------------------------------------------- float64 GEMM
//
// C = alpha * A B + beta * C with strided operands: A(i, k) = A[i sai + k sak],
// B(k, j) = B[k sbk + j sbj], C(i, j) = C[i ldc + j].  64 x 64 tiles, 16-deep
// K slices through LDS, 4 x 4 outputs per thread.  With lower_only, tiles
// entirely above the diagonal of C are skipped (symmetric results whose
// upper triangle is not used).  beta = 0 does not read C.
constexpr int kGB = 64, kGK = 16;

__global__ __launch_bounds__(256) void gemm_f64_kernel(GemmF64Args g) {
  __shared__ double As[kGK][kGB + 2];
  __shared__ double Bs[kGK][kGB + 2];
  const int64_t m0 = (int64_t)blockIdx.y * kGB, n0 = (int64_t)blockIdx.x * kGB;
  if (g.lower_only && n0 > m0 + kGB - 1) return;
  const int t = threadIdx.x, tx = t % 16, ty = t / 16;
  double acc[4][4];
#pragma unroll
  for (int r = 0; r < 4; ++r)
#pragma unroll
    for (int c = 0; c < 4; ++c) acc[r][c] = 0.0;
  // Load maps: the contiguous index of each operand runs along the lanes.
  const bool a_k_fast = g.sak == 1, b_j_fast = g.sbj == 1;
  const int ai = a_k_fast ? t / 4 : (t % 16) * 4, ak = a_k_fast ? (t % 4) * 4 : t / 16;
  const int bk = b_j_fast ? t / 16 : (t % 4) * 4, bj = b_j_fast ? (t % 16) * 4 : t / 4;
  for (int64_t k0 = 0; k0 < g.K; k0 += kGK) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int i = a_k_fast ? ai : ai + e, k = a_k_fast ? ak + e : ak;
      const int64_t gi = m0 + i, gk = k0 + k;
      As[k][i] = (gi < g.M && gk < g.K) ? g.A[gi * g.sai + gk * g.sak] : 0.0;
      const int kb = b_j_fast ? bk : bk + e, j = b_j_fast ? bj + e : bj;
      const int64_t gkb = k0 + kb, gj = n0 + j;
      Bs[kb][j] = (gkb < g.K && gj < g.N) ? g.B[gkb * g.sbk + gj * g.sbj] : 0.0;
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < kGK; ++k) {
      double av[4], bv[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) av[r] = As[k][4 * ty + r];
#pragma unroll
      for (int c = 0; c < 4; ++c) bv[c] = Bs[k][4 * tx + c];
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int c = 0; c < 4; ++c) acc[r][c] = fma(av[r], bv[c], acc[r][c]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int64_t i = m0 + 4 * ty + r;
    if (i >= g.M) continue;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int64_t j = n0 + 4 * tx + c;
      if (j >= g.N) continue;
      double* dst = g.C + i * g.ldc + j;
      *dst = g.beta == 0.0 ? g.alpha * acc[r][c] : fma(g.alpha, acc[r][c], g.beta * *dst);
    }
  }
}

// ---------------------------------------------------------------- Cholesky

// H += damp * mean(diag(H)) * I, one workgroup.
__global__ __launch_bounds__(256) void damp_kernel(double* H, int64_t n, double damp) {
  __shared__ double part[256];
  double sum = 0.0;
  for (int64_t i = threadIdx.x; i < n; i += 256) sum += H[i * n + i];
  part[threadIdx.x] = sum;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if ((int)threadIdx.x < w) part[threadIdx.x] += part[threadIdx.x + w];
    __syncthreads();
  }
  const double add = damp * (part[0] / (double)n);
  for (int64_t i = threadIdx.x; i < n; i += 256) H[i * n + i] += add;
}

// In-place lower Cholesky factor of the NB x NB diagonal block at H (row
// stride ld), reading only its lower triangle; zeros above its diagonal.
template <int NB>
__global__ __launch_bounds__(64) void potrf_kernel(double* H, int64_t ld) {
  __shared__ double S[NB][NB + 1];
  const int t = threadIdx.x;
  for (int e = t; e < NB * NB; e += 64) S[e / NB][e % NB] = H[(e / NB) * ld + e % NB];
  for (int k = 0; k < NB; ++k) {
    __syncthreads();
    if (t == k) {
      double d = S[k][k];
      for (int p = 0; p < k; ++p) d -= S[k][p] * S[k][p];
      S[k][k] = sqrt(d);
    }
    __syncthreads();
    if (t > k && t < NB) {
      double v = S[t][k];
      for (int p = 0; p < k; ++p) v -= S[t][p] * S[k][p];
      S[t][k] = v / S[k][k];
    }
  }
  __syncthreads();
  for (int e = t; e < NB * NB; e += 64) {
    const int i = e / NB, j = e % NB;
    H[i * ld + j] = j <= i ? S[i][j] : 0.0;
  }
}

// Rows r0 .. n-1 of the panel at columns [c0, c0 + NB): x L_kk^T = a, with
// L_kk the factored diagonal block at (c0, c0).  One thread per row.
template <int NB>
__global__ __launch_bounds__(256) void trsm_kernel(double* H, int64_t n, int64_t c0, int64_t r0) {
  __shared__ double Lk[NB][NB + 1];
  for (int e = threadIdx.x; e < NB * NB; e += 256) Lk[e / NB][e % NB] = H[(c0 + e / NB) * n + c0 + e % NB];
  __syncthreads();
  const int64_t r = r0 + (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (r >= n) return;
  double* row = H + r * n + c0;
  double x[NB];
#pragma unroll
  for (int j = 0; j < NB; ++j) {
    double v = row[j];
#pragma unroll
    for (int p = 0; p < j; ++p) v -= x[p] * Lk[j][p];
    x[j] = v / Lk[j][j];
  }
#pragma unroll
  for (int j = 0; j < NB; ++j) row[j] = x[j];
}

__global__ void zero_upper_kernel(double* H, int64_t n) {
  const int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= n * n) return;
  if (e % n > e / n) H[e] = 0.0;
}

// ---------------------------------------------------------------- one block of Algorithm 1

template <int G>
struct BlockLds {
  double rows[64][G + 1];  // Gram staging
  double A[G][G + 1];      // Gram matrix, rotated by one-sided Jacobi
  double V[G][G + 1];      // accumulated rotations: eigenvectors
  double Li[G][G + 1];     // X'[b, b]^-1 (lower), after the block itself
  double T[G][G + 1];      // T_X of the block
  double Mb[G][G + 1];     // sqrt(d_out) Hd diag(S^1/2 / S) V^T: Wbar = Mb Y_b^T
  double R[G * G];         // upper Cholesky factor of the inverse block Hessian
  double Wc[G][256];       // channel loop: column of thread t in Wc[.][t]
  double sig[G];           // eigenvalues s^2 of the Gram matrix
  double sk[G];            // sorted singular values (before the 1/sqrt(d_out))
  int perm[G];
  int rotated;
};

// Block b of Algorithm 1 (see the top of this file).  256 threads: the
// Jacobi rounds give each of the G/2 column pairs G/2 threads.  Every
// workgroup of the launch derives the block's transforms (steps 1-4, the
// same operations in the same order, so the same values); the channel loop
// then gives thread t of workgroup w the output channels 256 w + t,
// 256 (w + gridDim.x) + t, ...  Workgroup 0 stores T_X.
template <int FMT, int G>
__global__ __launch_bounds__(256) void gptq_wush_block_kernel(GptqWushArgs a, int b) {
  __shared__ BlockLds<G> L;
  const int t = threadIdx.x;
  const int64_t ld = a.d_in, lo = (int64_t)b * G;
  const double* Yb = a.Y + lo;  // Y_b(o, i) = Yb[o * ld + i]

  // 1. Gram matrix of Y_b over the d_out rows.
  {
    constexpr int kPer = G * G / 256;
    const int i = (t * kPer) / G, j0 = (t * kPer) % G;
    double acc[kPer];
#pragma unroll
    for (int q = 0; q < kPer; ++q) acc[q] = 0.0;
    for (int64_t r0 = 0; r0 < a.d_out; r0 += 64) {
      __syncthreads();
      for (int e = t; e < 64 * G; e += 256) {
        const int rr = e / G, c = e % G;
        L.rows[rr][c] = r0 + rr < a.d_out ? Yb[(r0 + rr) * ld + c] : 0.0;
      }
      __syncthreads();
      for (int rr = 0; rr < 64; ++rr) {
        const double yi = L.rows[rr][i];
#pragma unroll
        for (int q = 0; q < kPer; ++q) acc[q] = fma(yi, L.rows[rr][j0 + q], acc[q]);
      }
    }
#pragma unroll
    for (int q = 0; q < kPer; ++q) {
      L.A[i][j0 + q] = acc[q];
      L.V[i][j0 + q] = i == j0 + q ? 1.0 : 0.0;
    }
  }

  // 2. One-sided Jacobi on the columns of the (symmetric, positive
  // semi-definite) Gram matrix: its columns end orthogonal, V holds the
  // eigenvectors and the column norms are the eigenvalues.
  jacobi_columns<G>(L.A, L.V, &L.rotated, 40);

  // 3. Eigenvalues (column norms), descending order; X'[b, b]^-1 by forward
  // substitution, one column per thread.
  if (t < G) {
    double s = 0.0;
    for (int i = 0; i < G; ++i) s += L.A[i][t] * L.A[i][t];
    L.sig[t] = sqrt(s);
  } else if (t >= 64 && t < 64 + G) {
    const int j = t - 64;
    const double* Xbb = a.Xp + lo * ld + lo;
    double x[G];
#pragma unroll
    for (int i = 0; i < G; ++i) {
      double v = i == j ? 1.0 : 0.0;
#pragma unroll
      for (int p = 0; p < i; ++p) v -= Xbb[i * ld + p] * x[p];
      x[i] = i < j ? 0.0 : v / Xbb[i * ld + i];
    }
#pragma unroll
    for (int i = 0; i < G; ++i) L.Li[i][j] = x[i];
  }
  __syncthreads();
  if (t < G) {
    int rank = 0;
    for (int j = 0; j < G; ++j) rank += (L.sig[j] > L.sig[t]) || (L.sig[j] == L.sig[t] && j < t);
    L.perm[rank] = t;
  }
  __syncthreads();
  // Thread k: sorted column k comes from Jacobi column perm[k]; the sign
  // makes v_k's largest-magnitude entry (lowest index on ties) positive.
  // P[k][i] = sgn_k V[i][perm k] is stored over the staging rows.
  double(*P)[G + 1] = L.rows;
  static_assert(64 >= G, "staging rows too few for P");
  if (t < G) {
    const int src = L.perm[t];
    int lead = 0;
    double best = -1.0;
    for (int i = 0; i < G; ++i) {
      const double m = fabs(L.V[i][src]);
      if (m > best) {
        best = m;
        lead = i;
      }
    }
    const double sgn = L.V[lead][src] < 0.0 ? -1.0 : 1.0;
    for (int i = 0; i < G; ++i) P[t][i] = sgn * L.V[i][src];
    L.sk[t] = sqrt(L.sig[src]);
  }
  __syncthreads();

  // 4. T = Hd diag(rs) P Li and Mb = sqrt(d_out) Hd diag(rs / s) P, with
  // Sn = s / sqrt(d_out) and rs = sqrt(Sn).  R: the upper Cholesky factor
  // of (Hd diag(Sn) Hd^T)^-1 = Hd diag(1 / Sn) Hd^T, or I.
  const double sq_out = sqrt((double)a.d_out);
  for (int e = t; e < G * G; e += 256) {
    const int r = e / G, l = e % G;
    double tv = 0.0, mv = 0.0, hv = 0.0;
    for (int k = 0; k < G; ++k) {
      const double h = hadamard_entry<G>(r, k);
      const double sn = L.sk[k] / sq_out, rs = sqrt(sn);
      double pl = 0.0;
      for (int j = 0; j < G; ++j) pl = fma(P[k][j], L.Li[j][l], pl);
      tv = fma(h * rs, pl, tv);
      // A zero singular value contributes nothing to Wbar (S^1/2 U^T).
      mv = fma(h * (L.sk[k] > 0.0 ? rs / L.sk[k] : 0.0), P[k][l], mv);
      hv = fma(h / sn, hadamard_entry<G>(l, k), hv);
    }
    L.T[r][l] = tv;
    L.Mb[r][l] = sq_out * mv;
    L.A[r][l] = hv;  // Hd diag(1 / Sn) Hd^T, factored below
    if (blockIdx.x == 0) a.T_x[(int64_t)b * G * G + e] = tv;
  }
  __syncthreads();
  if (a.use_gptq) {
    for (int k = 0; k < G; ++k) {
      __syncthreads();
      if (t == k) {
        double d = L.A[k][k];
        for (int p = 0; p < k; ++p) d -= L.A[k][p] * L.A[k][p];
        L.A[k][k] = sqrt(d);
      }
      __syncthreads();
      if (t > k && t < G) {
        double v = L.A[t][k];
        for (int p = 0; p < k; ++p) v -= L.A[t][p] * L.A[k][p];
        L.A[t][k] = v / L.A[k][k];
      }
    }
    __syncthreads();
  }
  for (int e = t; e < G * G; e += 256) {
    const int i = e / G, j = e % G;
    L.R[e] = a.use_gptq ? (j >= i ? L.A[j][i] : 0.0) : (i == j ? 1.0 : 0.0);
  }
  __syncthreads();

  // 5. Channels: Wbar = Mb y_o, its group quantized with R; codes and scale
  // out; Wsub^T T (Wsub = Q for GPTQ, Wbar for round-to-nearest) goes into
  // Wq's block columns for the update of Y that follows this kernel.
  const int64_t C = a.d_in / G;
  for (int64_t o = (int64_t)blockIdx.x * 256 + t; o < a.d_out; o += (int64_t)gridDim.x * 256) {
    double y[G], q[G];
#pragma unroll
    for (int i = 0; i < G; ++i) y[i] = Yb[o * ld + i];
    for (int r = 0; r < G; ++r) {
      double v = 0.0;
#pragma unroll
      for (int i = 0; i < G; ++i) v = fma(L.Mb[r][i], y[i], v);
      L.Wc[r][t] = v;
    }
    uint32_t packed[G / 8];
    const uint32_t scode = quant_channel<FMT, G, 256>(&L.Wc[0][t], L.R, q, packed);
    // Round-to-nearest leaves the column as Wbar, which is then Wsub.
    if (!a.use_gptq) {
#pragma unroll
      for (int j = 0; j < G; ++j) q[j] = L.Wc[j][t];
    }
    uint32_t* cdst = reinterpret_cast<uint32_t*>(a.codes + o * (a.d_in / 2) + lo / 2);
#pragma unroll
    for (int i = 0; i < G / 8; ++i) cdst[i] = packed[i];
    if (FMT == 0)
      reinterpret_cast<uint8_t*>(a.scales)[o * C + b] = (uint8_t)scode;
    else
      reinterpret_cast<uint16_t*>(a.scales)[o * C + b] = (uint16_t)scode;
    double* st = a.Wq + o * ld + lo;
    for (int l = 0; l < G; ++l) {
      double v = 0.0;
#pragma unroll
      for (int j = 0; j < G; ++j) v = fma(q[j], L.T[j][l], v);
      st[l] = v;
    }
  }
}

// Wq = the dequantized codes (value of each nibble at its group's scale).
template <int FMT, int G>
__global__ void decode_kernel(GptqWushArgs a) {
  const int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= a.d_out * a.d_in) return;
  const int64_t o = e / a.d_in, k = e % a.d_in, C = a.d_in / G;
  const uint32_t byte = a.codes[o * (a.d_in / 2) + k / 2];
  const uint32_t nib = (k & 1) ? byte >> 4 : byte & 0xFu;
  double s;
  if (FMT == 0) {
    s = ldexp(1.0, (int)reinterpret_cast<const uint8_t*>(a.scales)[o * C + k / G] - 127);
  } else {
    const uint16_t h = reinterpret_cast<const uint16_t*>(a.scales)[o * C + k / G];
    s = (double)(float)__builtin_bit_cast(_Float16, h);
  }
  a.Wq[e] = code_value<FMT>(nib, s);
}

static void gemm_f64(const GemmF64Args& g, hipStream_t s) {
  if (g.M <= 0 || g.N <= 0) return;
  const dim3 grid((unsigned)((g.N + kGB - 1) / kGB), (unsigned)((g.M + kGB - 1) / kGB)), block(256);
  hipLaunchKernelGGL(gemm_f64_kernel, grid, block, 0, s, g);
}

template <int FMT, int G>
static hipError_t run_gptq_wush(const GptqWushArgs& a, hipStream_t s) {
  const int64_t n = a.d_in, C = n / G;
  // 1. Hx = Xcal^T Xcal / n_cal (lower triangle), damping, blocked Cholesky.
  GemmF64Args h{};
  h.A = a.Xcal; h.sai = 1; h.sak = n;
  h.B = a.Xcal; h.sbk = n; h.sbj = 1;
  h.C = a.Xp; h.ldc = n;
  h.M = n; h.N = n; h.K = a.n_cal;
  h.alpha = 1.0 / (double)a.n_cal; h.beta = 0.0; h.lower_only = 1;
  gemm_f64(h, s);
  hipLaunchKernelGGL(damp_kernel, dim3(1), dim3(256), 0, s, a.Xp, n, a.damp);
  for (int64_t c0 = 0; c0 < n; c0 += G) {
    hipLaunchKernelGGL((potrf_kernel<G>), dim3(1), dim3(64), 0, s, a.Xp + c0 * n + c0, n);
    const int64_t r0 = c0 + G;
    if (r0 >= n) break;
    hipLaunchKernelGGL((trsm_kernel<G>), dim3((unsigned)((n - r0 + 255) / 256)), dim3(256), 0, s, a.Xp, n, c0, r0);
    GemmF64Args u{};
    u.A = a.Xp + r0 * n + c0; u.sai = n; u.sak = 1;  // L21
    u.B = a.Xp + r0 * n + c0; u.sbk = 1; u.sbj = n;  // L21^T
    u.C = a.Xp + r0 * n + r0; u.ldc = n;
    u.M = n - r0; u.N = n - r0; u.K = G;
    u.alpha = -1.0; u.beta = 1.0; u.lower_only = 1;
    gemm_f64(u, s);
  }
  hipLaunchKernelGGL(zero_upper_kernel, dim3((unsigned)((n * n + 255) / 256)), dim3(256), 0, s, a.Xp, n);
  // 2. Y = W X'.
  GemmF64Args y{};
  y.A = a.W; y.sai = n; y.sak = 1;
  y.B = a.Xp; y.sbk = n; y.sbj = 1;
  y.C = a.Y; y.ldc = n;
  y.M = a.d_out; y.N = n; y.K = n;
  y.alpha = 1.0; y.beta = 0.0;
  gemm_f64(y, s);
  // 3. Blocks in reverse order; each updates the columns of the blocks
  // still to come: Y[:, < lo] -= (Wsub^T T) X'[lo:lo+G, < lo].  A block's
  // output channels are spread over workgroups of 256 (at most 256 of
  // them); each workgroup first derives the block's transforms itself, the
  // same float64 operations in the same order, so all hold identical
  // values, and workgroup 0 stores T_X.
  const unsigned n_wg = (unsigned)((a.d_out + 255) / 256 < 256 ? (a.d_out + 255) / 256 : 256);
  for (int64_t b = C - 1; b >= 0; --b) {
    hipLaunchKernelGGL((gptq_wush_block_kernel<FMT, G>), dim3(n_wg), dim3(256), 0, s, a, (int)b);
    const int64_t lo = b * G;
    if (lo == 0) continue;
    GemmF64Args u{};
    u.A = a.Wq + lo; u.sai = n; u.sak = 1;
    u.B = a.Xp + lo * n; u.sbk = n; u.sbj = 1;
    u.C = a.Y; u.ldc = n;
    u.M = a.d_out; u.N = lo; u.K = G;
    u.alpha = -1.0; u.beta = 1.0;
    gemm_f64(u, s);
  }
  // 4. Wq from the codes.
  const int64_t tot = a.d_out * n;
  hipLaunchKernelGGL((decode_kernel<FMT, G>), dim3((unsigned)((tot + 255) / 256)), dim3(256), 0, s, a);
  return hipGetLastError();
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

hipError_t launch_gptq_wush(int fmt, int G, const GptqWushArgs& a, hipStream_t s) {
  if (fmt == 0 && G == 32) return run_gptq_wush<0, 32>(a, s);
  if (fmt == 0) return run_gptq_wush<0, 16>(a, s);
  if (G == 32) return run_gptq_wush<2, 32>(a, s);
  return run_gptq_wush<2, 16>(a, s);
}

}  // namespace wush
