// MXFP4 x MXFP4 GEMM for gfx950: the FP4 matrix multiplication that consumes
// the fused transform + quantization output.
//
// "WUSH: Near-Optimal Adaptive Transforms for LLM Quantization", deep dive,
// section 3.4.6 (Eq. 10): at inference each transformed, quantized
// activation block multiplies the pre-quantized transformed weight block,
// and the block contributions add up.  With both operands in MXFP4 (E2M1
// codes, one E8M0 scale per 32 elements along K) this is one GEMM:
//     C[m][n] = sum_k a[m][k] * b[n][k],
// a = decoded activations [M][K], b = decoded weights [N][K].
//
// v_mfma_scale_f32_32x32x64_f8f6f4 with E2M1 operands takes, in lane
// (i + 32h), the 16 code bytes of row i for k = 32h..32h+31 (element 2t in
// the low nibble of byte t) and that block's E8M0 scale byte, which is
// exactly the row-major layout the quantization kernel writes.
//
// Workgroup: a 128 x 128 tile of C, K in steps of 256 (128 code bytes per
// row), 8 waves in two groups of 4.  Group g takes the steps ks = g, g + 2,
// g + 4, ... (the K sum is split inside the workgroup), and the two partial
// tiles are added through LDS at the end.  The split puts two waves on
// every SIMD, so one wave's MFMAs cover the other's LDS latency, while the
// output tile, and with it the global traffic per FLOP, stays 128 x 128.
// Within a group, wave (wm, wn) owns a 64 x 64 quarter: 2 x 2 MFMA tiles of
// 32 x 32.
//
// Codes are staged through LDS with row-contiguous 16-byte loads (rows
// padded to 144 B, so the operand reads of 16 rows hit 16 distinct bank
// groups); each row's 8 scale bytes of a step are regrouped so that lane
// half h finds blocks h, h+2, h+4, h+6 in one word, and sub-step s selects
// byte s with the instruction's op_sel.  Each group double-buffers its LDS
// stage and keeps its global loads three of its steps ahead through two
// register sets.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "wush_gemm.h"

namespace wush {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int BM = 128, BN = 128;
constexpr int BK_BYTES = 128;            // code bytes per row per K step (256 elements)
constexpr int kRowB = BK_BYTES + 16;     // padded LDS row
constexpr int kGroups = 2;
constexpr int kThreads = 256 * kGroups;

struct GemmLds {
  uint8_t a[kGroups][2][BM * kRowB];
  uint8_t b[kGroups][2][BN * kRowB];
  uint32_t sa[kGroups][2][BM * 2];  // row r: word h = scale bytes of blocks h, h+2, h+4, h+6
  uint32_t sb[kGroups][2][BN * 2];
};
// The final exchange of partial tiles reuses the stage buffers: 8 waves x
// 2 tiles x 16 floats x 64 lanes.
static_assert(sizeof(((GemmLds*)0)->a) >= 8 * 2 * 16 * 64 * 4, "exchange does not fit");

__device__ __forceinline__ int lane_id() { return __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u)); }

// Eight scale bytes b0..b7 (blocks 0..7 of the step, b0 lowest) ->
// {b0 b2 b4 b6}, {b1 b3 b5 b7}.
__device__ __forceinline__ u32x2 regroup_scales(u32x2 v) {
  // v_perm_b32(src0, src1, sel): byte selectors 0..3 pick src1, 4..7 src0.
  const uint32_t even = __builtin_amdgcn_perm(v[1], v[0], 0x06040200u);
  const uint32_t odd = __builtin_amdgcn_perm(v[1], v[0], 0x07050301u);
  u32x2 r = {even, odd};
  return r;
}

template <int SUB>
__device__ __forceinline__ f32x16 mfma_fp4(u32x4 a, u32x4 b, f32x16 c, uint32_t sa, uint32_t sb) {
  const i32x8 a8 = {(int)a[0], (int)a[1], (int)a[2], (int)a[3], 0, 0, 0, 0};
  const i32x8 b8 = {(int)b[0], (int)b[1], (int)b[2], (int)b[3], 0, 0, 0, 0};
  // format 4 = E2M1 for both operands; op_sel SUB picks scale byte SUB.
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a8, b8, c, 4, 4, SUB, (int)sa, SUB, (int)sb);
}

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float x) {
  const uint32_t b = __float_as_uint(x);
  return (uint16_t)((b + 0x7FFFu + ((b >> 16) & 1u)) >> 16);
}

template <bool BF16_OUT>
__global__ __launch_bounds__(kThreads) void gemm_mxfp4_kernel(GemmArgs g) {
  __shared__ __attribute__((aligned(16))) GemmLds L;
  const int tid = threadIdx.x;
  const int lane = lane_id();
  const int wave = tid >> 6;
  const int grp = wave >> 2;      // K-split group
  const int gw = wave & 3;        // wave within the group
  const int gt = tid & 255;       // thread within the group
  const int wm = gw >> 1, wn = gw & 1;
  const int64_t m0 = (int64_t)blockIdx.y * BM, n0 = (int64_t)blockIdx.x * BN;
  const int64_t K = g.K, M = g.M, N = g.N;
  const int64_t row_bytes = K / 2, row_scales = K / 32;
  const int nk = (int)(K / 256);
  const int nj = (nk + 1) / 2;    // steps per group (group 1 idles on the last one when nk is odd)

  // Staging map (per group): thread t moves 16-byte chunk t % 8 of rows
  // t / 8 + 32 q (q = 0..3) of both tiles; threads 0..127 move A scale
  // rows, 128..255 B.
  const int c_chunk = gt & 7, c_row = gt >> 3;
  const uint8_t* a_src[4];
  const uint8_t* b_src[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    int64_t ra = m0 + c_row + 32 * q, rb = n0 + c_row + 32 * q;
    ra = ra < M ? ra : M - 1;  // rows past the edge reload the last row; never stored
    rb = rb < N ? rb : N - 1;
    a_src[q] = g.a_codes + ra * row_bytes + 16 * c_chunk;
    b_src[q] = g.b_codes + rb * row_bytes + 16 * c_chunk;
  }
  const bool scale_a = gt < 128;
  const int s_row = gt & 127;
  int64_t s_r = (scale_a ? m0 : n0) + s_row;
  const int64_t s_lim = scale_a ? M : N;
  s_r = s_r < s_lim ? s_r : s_lim - 1;
  const uint8_t* s_src = (scale_a ? g.a_scales : g.b_scales) + s_r * row_scales;

  // Group step j covers K step 2 j + grp.  Past the end the index is
  // clamped: the load repeats a valid step and nothing is computed from it.
  auto kstep = [&](int j) { return min(2 * j + grp, nk - 1); };

  // Two register sets carry global data two group steps ahead of its use:
  // step j stages set (j + 1) & 1 (the operands of step j + 1) into LDS and
  // then refills that set with step j + 3.
  struct Regs {
    u32x4 a[4], b[4];
    u32x2 s;
  };
  Regs R0, R1;
  auto load = [&](Regs& r, int j) {
    const int64_t off = (int64_t)kstep(j) * BK_BYTES;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      r.a[q] = *reinterpret_cast<const u32x4*>(a_src[q] + off);
      r.b[q] = *reinterpret_cast<const u32x4*>(b_src[q] + off);
    }
    r.s = *reinterpret_cast<const u32x2*>(s_src + (int64_t)kstep(j) * 8);
  };
  auto stage = [&](const Regs& r, int buf) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      *reinterpret_cast<u32x4*>(L.a[grp][buf] + (c_row + 32 * q) * kRowB + 16 * c_chunk) = r.a[q];
      *reinterpret_cast<u32x4*>(L.b[grp][buf] + (c_row + 32 * q) * kRowB + 16 * c_chunk) = r.b[q];
    }
    const u32x2 w = regroup_scales(r.s);
    uint32_t* dst = scale_a ? L.sa[grp][buf] : L.sb[grp][buf];
    *reinterpret_cast<u32x2*>(dst + 2 * s_row) = w;
  };

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x16{};

  const int li = lane & 31, lh = lane >> 5;
  auto compute = [&](int buf) {
    const uint8_t* la = L.a[grp][buf];
    const uint8_t* lb = L.b[grp][buf];
    uint32_t sa[2], sb[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      sa[t] = L.sa[grp][buf][2 * (64 * wm + 32 * t + li) + lh];
      sb[t] = L.sb[grp][buf][2 * (64 * wn + 32 * t + li) + lh];
    }
#define WUSH_GEMM_SUB(S)                                                                                   \
    {                                                                                                     \
      u32x4 av[2], bv[2];                                                                                 \
      _Pragma("unroll") for (int t = 0; t < 2; ++t) {                                                     \
        av[t] = *reinterpret_cast<const u32x4*>(la + (64 * wm + 32 * t + li) * kRowB + 32 * (S) + 16 * lh); \
        bv[t] = *reinterpret_cast<const u32x4*>(lb + (64 * wn + 32 * t + li) * kRowB + 32 * (S) + 16 * lh); \
      }                                                                                                   \
      _Pragma("unroll") for (int i = 0; i < 2; ++i) _Pragma("unroll") for (int j = 0; j < 2; ++j)         \
          acc[i][j] = mfma_fp4<S>(av[i], bv[j], acc[i][j], sa[i], sb[j]);                                \
    }
    WUSH_GEMM_SUB(0)
    WUSH_GEMM_SUB(1)
    WUSH_GEMM_SUB(2)
    WUSH_GEMM_SUB(3)
#undef WUSH_GEMM_SUB
  };

  // Group step j: barrier (this group's buffer j & 1 is complete and its
  // waves are done with buffer (j + 1) & 1), stage step j + 1, refill,
  // compute step j.  Loads and stages run unconditionally so the load
  // counter at every stage is the same on all paths.
  auto step = [&](int j, Regs& next) {
    __syncthreads();
    stage(next, (j + 1) & 1);
    load(next, j + 3);
    // Keep the refill ahead of this step's MFMAs; the scheduler would
    // otherwise sink it below them and halve the latency it hides.
    __builtin_amdgcn_sched_barrier(0);
    if (2 * j + grp < nk) compute(j & 1);
  };

  load(R0, 0);
  load(R1, 1);
  stage(R0, 0);
  load(R0, 2);
  int j = 0;
  for (; j + 1 < nj; j += 2) {
    step(j, R1);
    step(j + 1, R0);
  }
  if (j < nj) step(j, R1);

  // Add the two groups' partial tiles: group g finishes MFMA tile row
  // i == g of its quarter and hands tile row 1 - g to its partner wave.
  __syncthreads();
  float* xch = reinterpret_cast<float*>(&L.a[0][0][0]);
  const int partner = wave ^ 4;
  f32x16 give[2], fin[2];
#pragma unroll
  for (int jt = 0; jt < 2; ++jt) {  // constant indices keep acc in registers
    give[jt] = grp ? acc[0][jt] : acc[1][jt];
    fin[jt] = grp ? acc[1][jt] : acc[0][jt];
  }
#pragma unroll
  for (int jt = 0; jt < 2; ++jt)
#pragma unroll
    for (int r = 0; r < 16; ++r) xch[((wave * 2 + jt) * 16 + r) * 64 + lane] = give[jt][r];
  __syncthreads();
#pragma unroll
  for (int jt = 0; jt < 2; ++jt)
#pragma unroll
    for (int r = 0; r < 16; ++r) fin[jt][r] += xch[((partner * 2 + jt) * 16 + r) * 64 + lane];

  // Epilogue: lane (j + 32h) of MFMA tile (i, jt) holds C rows
  // 8 (r / 4) + 4 h + r % 4 of column j; a half-wave writes 32 consecutive
  // columns of one row.
#pragma unroll
  for (int jt = 0; jt < 2; ++jt) {
    const int64_t col = n0 + 64 * wn + 32 * jt + li;
    if (col >= N) continue;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int64_t row = m0 + 64 * wm + 32 * grp + 8 * (r / 4) + 4 * lh + (r % 4);
      if (row < M) {
        if (BF16_OUT)
          reinterpret_cast<uint16_t*>(g.C)[row * N + col] = f32_to_bf16_rne(fin[jt][r]);
        else
          reinterpret_cast<float*>(g.C)[row * N + col] = fin[jt][r];
      }
    }
  }
}

}  // namespace

hipError_t launch_gemm_mxfp4(const GemmArgs& g, bool bf16_out, hipStream_t s) {
  dim3 grid((unsigned)((g.N + BN - 1) / BN), (unsigned)((g.M + BM - 1) / BM)), block(kThreads);
  if (bf16_out) hipLaunchKernelGGL((gemm_mxfp4_kernel<true>), grid, block, 0, s, g);
  else hipLaunchKernelGGL((gemm_mxfp4_kernel<false>), grid, block, 0, s, g);
  return hipGetLastError();
}

}  // namespace wush
