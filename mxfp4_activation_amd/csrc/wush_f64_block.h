// Float64 G x G block algebra shared by the transform builder
// (wush_build.hip) and GPTQ-WUSH (wush_gptq.hip): the normalized Sylvester
// Hadamard matrix and a one-sided (Hestenes) Jacobi SVD of a block held in
// LDS.  Device code only; not part of the public ABI.
#ifndef WUSH_F64_BLOCK_H_
#define WUSH_F64_BLOCK_H_

#include <hip/hip_runtime.h>

namespace wush {

// Entry (a, k) of the Sylvester Hadamard matrix of order G (H_1 = [1],
// H_2n = [[H_n, H_n], [H_n, -H_n]]) divided by sqrt(G).
template <int G>
__device__ __forceinline__ double hadamard_entry(int a, int k) {
  const double h = 1.0 / sqrt((double)G);
  return (__builtin_popcount((unsigned)(a & k)) & 1) ? -h : h;
}

// One-sided Jacobi on the columns of A (G x G in LDS, row stride G + 1),
// accumulating the rotations into V (which the caller initializes, usually
// to I).  On return the columns of A are mutually orthogonal to rounding
// level (A_in V = A_out), so the column norms of A_out are the singular
// values of A_in and V holds its right singular vectors.  Round r pairs
// column (r + k) % (G - 1) with (r - k) % (G - 1) for k = 1 .. G/2 - 1 and
// r % (G - 1) with G - 1 (k = 0), so a sweep of G - 1 rounds meets every
// pair once; pair k is handled by threads [k G/2, (k + 1) G/2), two rows
// each.  At most max_sweeps sweeps; it stops after the first sweep that
// rotates nothing.  Called by every thread of the workgroup (at least G²/4
// threads); starts and ends with a barrier.
template <int G>
__device__ void jacobi_columns(double (*A)[G + 1], double (*V)[G + 1], int* rotated, int max_sweeps) {
  const int t = threadIdx.x;
  constexpr int kTpp = G / 2;
  const int pk = t / kTpp, pl = t % kTpp;
  const bool in_pair = pk < G / 2;
  for (int sweep = 0; sweep < max_sweeps; ++sweep) {
    __syncthreads();
    if (t == 0) *rotated = 0;
    for (int r = 0; r < G - 1; ++r) {
      __syncthreads();
      if (in_pair) {
        int p, q;
        if (pk == 0) {
          p = r % (G - 1);
          q = G - 1;
        } else {
          p = (r + pk) % (G - 1);
          q = (r - pk + (G - 1)) % (G - 1);
        }
        const int r0 = 2 * pl, r1 = 2 * pl + 1;
        double al = A[r0][p] * A[r0][p] + A[r1][p] * A[r1][p];
        double be = A[r0][q] * A[r0][q] + A[r1][q] * A[r1][q];
        double ga = A[r0][p] * A[r0][q] + A[r1][p] * A[r1][q];
#pragma unroll
        for (int o = 1; o < kTpp; o <<= 1) {
          al += __shfl_xor(al, o, kTpp);
          be += __shfl_xor(be, o, kTpp);
          ga += __shfl_xor(ga, o, kTpp);
        }
        // Rotate when the pair is not orthogonal to rounding level.
        if (fabs(ga) > 1e-15 * sqrt(al * be) && ga != 0.0) {
          const double zeta = (be - al) / (2.0 * ga);
          const double tn = (zeta >= 0.0 ? 1.0 : -1.0) / (fabs(zeta) + sqrt(1.0 + zeta * zeta));
          const double cs = 1.0 / sqrt(1.0 + tn * tn), sn = cs * tn;
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const int rw = 2 * pl + h;
            const double xp = A[rw][p], xq = A[rw][q];
            A[rw][p] = cs * xp - sn * xq;
            A[rw][q] = sn * xp + cs * xq;
            const double vp = V[rw][p], vq = V[rw][q];
            V[rw][p] = cs * vp - sn * vq;
            V[rw][q] = sn * vp + cs * vq;
          }
          if (pl == 0) *rotated = 1;
        }
      }
    }
    __syncthreads();
    const int any = *rotated;
    if (!any) break;
  }
  __syncthreads();
}

}  // namespace wush

#endif  // WUSH_F64_BLOCK_H_
