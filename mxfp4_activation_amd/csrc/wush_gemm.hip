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
// Workgroup: a 64 TM x 64 TM tile of C (TM = 2: 128 x 128; TM = 1, for
// grids that would leave CUs idle: 64 x 64) and 8 waves in two groups of 4.
// K runs in steps of 256 elements (128 code bytes per row); group g takes
// the half-range [128 g, 128 g + 128) of every step (the K sum is split
// inside the workgroup) and the two partial tiles are added through LDS at
// the end.  Every SIMD holds one wave of each group.  Within a group, wave
// (wm, wn) owns a quarter: TM x TM MFMA tiles of 32 x 32.
//
// Operands go from global memory straight into LDS (global_load_lds, 16 B
// per lane, whole 128-byte rows), through a ring of step stages (4 at
// TM = 2, 8 at TM = 1), 2 or 4 steps ahead of the MFMAs.  No staging registers and no LDS write
// instructions are involved; each wave waits for its own loads with vmcnt
// and one barrier per step publishes them.
//
// LDS layout of a stage (BT = 64 TM rows): A codes [BT rows][128 B], B
// codes [BT][128 B], A scales [BT][8 B], B scales [BT][8 B].  A load instruction writes 1 KB
// contiguously (8 rows), so rows are not padded: the 16-byte chunk c of
// row r sits in slot c ^ ((r >> 1) & 7) instead, which gives the operand
// reads of 16 consecutive rows 16 distinct bank groups.  Sub-step s of a
// step gives lane (i + 32h) chunk 2 s + h of row i, i.e. K block 2 s + h,
// whose E8M0 scale is byte 2 s + h of the row's 8 scale bytes; the scale
// word is shifted right by 8 h so that op_sel 2 (s % 2) picks it for both
// lane halves.
//
// Fragment reads are inline-asm ds_read blocks that wait for their own
// results: plain LDS loads after a global_load_lds make the compiler wait
// for every outstanding global load, which would drain the ring.  Group 1
// runs its MFMAs before its reads in every step (on registers read in the
// step before), so that on each SIMD one wave reads LDS while the other
// keeps the matrix unit busy.
//
// The result goes through LDS once more, so that C is written with 16-byte
// row-contiguous stores.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "wush_gemm.h"

namespace wush {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kRowB = 128;                // code bytes per row per step (256 elements)
constexpr int kGroups = 2;
constexpr int kThreads = 256 * kGroups;
constexpr int kLdsB = 139264;             // 4 stages of 128-row tiles or 8 of 64-row tiles

// Tile geometry for TM MFMA tiles (of 32 x 32) per wave per dimension: the
// workgroup tile is 64 TM x 64 TM.  TM = 2 is the main shape; TM = 1 serves
// grids that would otherwise leave most CUs idle.
template <int TM>
struct Geo {
  static constexpr int BT = 64 * TM;                        // tile rows (= columns)
  static constexpr int kOffB = BT * kRowB;
  static constexpr int kOffSA = 2 * BT * kRowB;
  static constexpr int kOffSB = kOffSA + BT * 8;
  static constexpr int kStageB = kOffSB + BT * 8;
  static constexpr int kStages = kLdsB / kStageB;           // 4 or 8
  static constexpr int kAhead = TM == 2 ? 2 : 4;            // steps of loads in flight
  static constexpr int kLoadsPerStep = 2 * TM + 1;          // load instructions per wave per step
  static constexpr int kCRow = BT + 4;                      // padded fp32 row of the output tile
  static_assert(kStages * kStageB == kLdsB, "stages must fill the ring");
  static_assert(kStages >= kAhead + 1, "ring too short for the load distance");
  static_assert(kLdsB >= 8 * TM * TM * 8 * 64 * 4, "exchange does not fit");
  static_assert(kLdsB >= BT * kCRow * 4, "output tile does not fit");
};

__device__ __forceinline__ int lane_id() { return __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u)); }

template <int OPSEL>
__device__ __forceinline__ f32x16 mfma_fp4(u32x4 a, u32x4 b, f32x16 c, uint32_t sa, uint32_t sb) {
  const i32x8 a8 = {(int)a[0], (int)a[1], (int)a[2], (int)a[3], 0, 0, 0, 0};
  const i32x8 b8 = {(int)b[0], (int)b[1], (int)b[2], (int)b[3], 0, 0, 0, 0};
  // format 4 = E2M1 for both operands; op_sel picks the scale byte.
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a8, b8, c, 4, 4, OPSEL, (int)sa, OPSEL, (int)sb);
}

__device__ __forceinline__ uint32_t f32_to_bf16_rne(float x) {
  const uint32_t b = __float_as_uint(x);
  return (b + 0x7FFFu + ((b >> 16) & 1u)) >> 16;
}

// s_waitcnt vmcnt(N) followed by s_barrier, N spelled out.
template <int N>
__device__ __forceinline__ void wait_barrier() {
  asm volatile("s_waitcnt vmcnt(%0)\n s_barrier" ::"n"(N) : "memory");
}

typedef __attribute__((address_space(3))) uint8_t lds_u8;
typedef const __attribute__((address_space(1))) uint8_t glb_u8;

// Global-to-LDS copies of 16 and 4 bytes per lane.  Kept out of the kernel
// template: the builtin used directly in a template body makes the host pass
// drop the kernel's launch stub without a diagnostic.
__device__ __forceinline__ void dma16(glb_u8* src, lds_u8* dst) { __builtin_amdgcn_global_load_lds(src, dst, 16, 0, 0); }
__device__ __forceinline__ void dma4(glb_u8* src, lds_u8* dst) { __builtin_amdgcn_global_load_lds(src, dst, 4, 0, 0); }

template <int TM, bool BF16_OUT>
__global__ __launch_bounds__(kThreads) void gemm_mxfp4_kernel(GemmArgs g) {
  using Gm = Geo<TM>;
  constexpr int BT = Gm::BT;
  __shared__ __attribute__((aligned(1024))) uint8_t L[kLdsB];
  lds_u8* const Ls = (lds_u8*)L;
  const uint32_t lbase = (uint32_t)(uintptr_t)Ls;
  const int tid = threadIdx.x;
  const int lane = lane_id();
  const int wave = tid >> 6;
  const int grp = wave >> 2;      // K-split group
  const int gw = wave & 3;        // wave within the group
  const int wm = gw >> 1, wn = gw & 1;
  const int64_t m0 = (int64_t)blockIdx.y * BT, n0 = (int64_t)blockIdx.x * BT;
  const int64_t K = g.K, M = g.M, N = g.N;
  const int64_t row_bytes = K / 2, row_scales = K / 32;
  const int nk = (int)(K / 256);

  // Load map.  Code loads: wave w moves rows 8 (TM w + q) .. +7 (q < TM) of
  // both tiles; lane L takes row L / 8 of those 8 and stores LDS slot L % 8,
  // which holds chunk (L % 8) ^ ((row / 2) % 8).
  glb_u8* a_src[TM];
  glb_u8* b_src[TM];
#pragma unroll
  for (int q = 0; q < TM; ++q) {
    const int r = 8 * (TM * wave + q) + (lane >> 3);
    const int chunk = (lane & 7) ^ ((r >> 1) & 7);
    int64_t ra = m0 + r, rb = n0 + r;
    ra = ra < M ? ra : M - 1;  // rows past the edge reload the last row; never stored
    rb = rb < N ? rb : N - 1;
    a_src[q] = (glb_u8*)g.a_codes + ra * row_bytes + 16 * chunk;
    b_src[q] = (glb_u8*)g.b_codes + rb * row_bytes + 16 * chunk;
  }
  // Scale loads: waves 0..3 move A rows 16 TM w + L / 2, waves 4..7 B rows
  // 16 TM (w - 4) + L / 2, 4 bytes (half a row's 8) per lane; lanes from
  // 32 TM on stay idle.
  const bool s_is_a = wave < 4;
  const bool s_lane = lane < 32 * TM;
  int64_t s_row = (s_is_a ? m0 : n0) + 16 * TM * (wave & 3) + (lane >> 1);
  const int64_t s_lim = s_is_a ? M : N;
  s_row = s_row < s_lim ? s_row : s_lim - 1;
  glb_u8* s_src = (glb_u8*)(s_is_a ? g.a_scales : g.b_scales) + s_row * row_scales + 4 * (lane & 1);
  const int s_dst = (s_is_a ? Gm::kOffSA : Gm::kOffSB) + 128 * TM * (wave & 3);

  // Step ks lives in ring stage ks % kStages.
  auto issue = [&](int ks) {
    const int64_t kc = ks;
    lds_u8* st = Ls + (ks % Gm::kStages) * Gm::kStageB;
#pragma unroll
    for (int q = 0; q < TM; ++q) {
      dma16(a_src[q] + kc * kRowB, st + 1024 * (TM * wave + q));
      dma16(b_src[q] + kc * kRowB, st + Gm::kOffB + 1024 * (TM * wave + q));
    }
    if (s_lane) dma4(s_src + kc * 8, st + s_dst);
  };

  f32x16 acc[TM][TM];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TM; ++j) acc[i][j] = f32x16{};

  // Per-lane parts of the fragment addresses: group g runs sub-steps 2 g and
  // 2 g + 1, i.e. chunks 4 g + h and 4 g + 2 + h, and scale word g.
  const int li = lane & 31, lh = lane >> 5;
  const int sw = (li >> 1) & 7;
  const uint32_t fa0 = (32 * TM * wm + li) * kRowB + 16 * ((4 * grp + lh) ^ sw);
  const uint32_t fa1 = (32 * TM * wm + li) * kRowB + 16 * ((4 * grp + 2 + lh) ^ sw);
  const uint32_t fb0 = Gm::kOffB + (32 * TM * wn + li) * kRowB + 16 * ((4 * grp + lh) ^ sw);
  const uint32_t fb1 = Gm::kOffB + (32 * TM * wn + li) * kRowB + 16 * ((4 * grp + 2 + lh) ^ sw);
  const uint32_t fsa = Gm::kOffSA + 8 * (32 * TM * wm + li) + 4 * grp;
  const uint32_t fsb = Gm::kOffSB + 8 * (32 * TM * wn + li) + 4 * grp;
  const uint32_t shift = 8 * lh;

  struct Frag {
    u32x4 a[2][TM], b[2][TM];  // [sub-step][tile]
    uint32_t sa[TM], sb[TM];
  };
  auto read = [&](int ks, Frag& f) {
    const uint32_t st = lbase + (ks % Gm::kStages) * Gm::kStageB;
    // Tile row / column t = 1 is 32 rows further: 4096 B of codes, 256 B of scales.
    if constexpr (TM == 2) {
      asm volatile(
          "ds_read_b128 %0, %12\n"
          "ds_read_b128 %1, %12 offset:4096\n"
          "ds_read_b128 %2, %13\n"
          "ds_read_b128 %3, %13 offset:4096\n"
          "ds_read_b128 %4, %14\n"
          "ds_read_b128 %5, %14 offset:4096\n"
          "ds_read_b128 %6, %15\n"
          "ds_read_b128 %7, %15 offset:4096\n"
          "ds_read_b32 %8, %16\n"
          "ds_read_b32 %9, %16 offset:256\n"
          "ds_read_b32 %10, %17\n"
          "ds_read_b32 %11, %17 offset:256\n"
          "s_waitcnt lgkmcnt(0)"
          : "=&v"(f.a[0][0]), "=&v"(f.a[0][1]), "=&v"(f.a[1][0]), "=&v"(f.a[1][1]), "=&v"(f.b[0][0]),
            "=&v"(f.b[0][1]), "=&v"(f.b[1][0]), "=&v"(f.b[1][1]), "=&v"(f.sa[0]), "=&v"(f.sa[1]), "=&v"(f.sb[0]),
            "=&v"(f.sb[1])
          : "v"(st + fa0), "v"(st + fa1), "v"(st + fb0), "v"(st + fb1), "v"(st + fsa), "v"(st + fsb)
          : "memory");
    } else {
      asm volatile(
          "ds_read_b128 %0, %6\n"
          "ds_read_b128 %1, %7\n"
          "ds_read_b128 %2, %8\n"
          "ds_read_b128 %3, %9\n"
          "ds_read_b32 %4, %10\n"
          "ds_read_b32 %5, %11\n"
          "s_waitcnt lgkmcnt(0)"
          : "=&v"(f.a[0][0]), "=&v"(f.a[1][0]), "=&v"(f.b[0][0]), "=&v"(f.b[1][0]), "=&v"(f.sa[0]), "=&v"(f.sb[0])
          : "v"(st + fa0), "v"(st + fa1), "v"(st + fb0), "v"(st + fb1), "v"(st + fsa), "v"(st + fsb)
          : "memory");
    }
#pragma unroll
    for (int t = 0; t < TM; ++t) {
      f.sa[t] >>= shift;
      f.sb[t] >>= shift;
    }
  };
  auto mfma = [&](const Frag& f) {
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TM; ++j) acc[i][j] = mfma_fp4<0>(f.a[0][i], f.b[0][j], acc[i][j], f.sa[i], f.sb[j]);
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TM; ++j) acc[i][j] = mfma_fp4<2>(f.a[1][i], f.b[1][j], acc[i][j], f.sa[i], f.sb[j]);
  };

  // Step ks: wait for this wave's loads of step ks (those of the later
  // steps already issued may stay in flight), barrier (every wave's loads
  // of step ks have landed, and every wave is done with the stage step
  // ks - 1 used), refill that stage with step ks + kAhead if there is one.
  // Group 0 then reads step ks and runs its MFMAs; group 1 first runs the
  // MFMAs of step ks - 1 from registers and reads step ks last, so that on
  // each SIMD one wave reads LDS while the other keeps the matrix unit busy.
  constexpr int LPS = Gm::kLoadsPerStep;
  auto sync = [&](int ks) {
    const int later = min(Gm::kAhead - 1, nk - 1 - ks);  // steps issued after ks
    switch (later) {
      case 3: wait_barrier<3 * LPS>(); break;
      case 2: wait_barrier<2 * LPS>(); break;
      case 1: wait_barrier<LPS>(); break;
      default: wait_barrier<0>(); break;
    }
    if (ks + Gm::kAhead < nk) issue(ks + Gm::kAhead);
  };
  static_assert(Gm::kAhead <= 4, "sync() spells out the wait counts for up to four steps in flight");
  for (int p = 0; p < Gm::kAhead; ++p)
    if (p < nk) issue(p);
  Frag f;
  if (grp == 0) {
    for (int ks = 0; ks < nk; ++ks) {
      sync(ks);
      read(ks, f);
      mfma(f);
    }
  } else {
    for (int ks = 0; ks < nk; ++ks) {
      sync(ks);
      if (ks > 0) mfma(f);
      read(ks, f);
    }
    mfma(f);
  }
  wait_barrier<0>();

  // Add the two groups' partial tiles through LDS, then write the summed
  // tile to LDS as fp32 (rows padded): lane (j + 32h) of an MFMA tile holds
  // rows 8 (r / 4) + 4 h + r % 4 of column j in accumulator register r.
  f32x4* xch = reinterpret_cast<f32x4*>(L);
  float* ct = reinterpret_cast<float*>(L);
  const int partner = wave ^ 4;
  if constexpr (TM == 2) {
    // Group g finishes MFMA tile row g and hands tile row 1 - g to its
    // partner wave.
    f32x16 give[2], fin[2];
#pragma unroll
    for (int jt = 0; jt < 2; ++jt) {  // constant indices keep acc in registers
      give[jt] = grp ? acc[0][jt] : acc[1][jt];
      fin[jt] = grp ? acc[1][jt] : acc[0][jt];
    }
#pragma unroll
    for (int jt = 0; jt < 2; ++jt)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        f32x4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = give[jt][4 * q + e];
        xch[((wave * 2 + jt) * 4 + q) * 64 + lane] = v;
      }
    __syncthreads();
#pragma unroll
    for (int jt = 0; jt < 2; ++jt)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const f32x4 v = xch[((partner * 2 + jt) * 4 + q) * 64 + lane];
#pragma unroll
        for (int e = 0; e < 4; ++e) fin[jt][4 * q + e] += v[e];
      }
    __syncthreads();
#pragma unroll
    for (int jt = 0; jt < 2; ++jt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = 64 * wm + 32 * grp + 8 * (r / 4) + 4 * lh + (r % 4);
        ct[row * Gm::kCRow + 64 * wn + 32 * jt + li] = fin[jt][r];
      }
  } else {
    // Group g finishes accumulator registers 8 g .. 8 g + 7 and hands the
    // other eight to its partner.  The halves are picked once, by whole
    // vectors, so that every register index below is a constant: an index
    // that depends on the group compiles to a select over all 16 registers
    // for every element moved (about 1300 instructions, ~4 us per launch).
    f32x4 keep[2], hand[2];
#pragma unroll
    for (int q = 0; q < 2; ++q)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float lo = acc[0][0][4 * q + e], hi = acc[0][0][8 + 4 * q + e];
        keep[q][e] = grp ? hi : lo;
        hand[q][e] = grp ? lo : hi;
      }
#pragma unroll
    for (int q = 0; q < 2; ++q) xch[(wave * 2 + q) * 64 + lane] = hand[q];
    __syncthreads();
#pragma unroll
    for (int q = 0; q < 2; ++q) keep[q] += xch[(partner * 2 + q) * 64 + lane];
    __syncthreads();
    // keep[q][e] is register r = 8 g + 4 q + e: row 16 g + 8 q + 4 h + e.
#pragma unroll
    for (int q = 0; q < 2; ++q)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int row = 32 * wm + 16 * grp + 8 * q + 4 * lh + e;
        ct[row * Gm::kCRow + 32 * wn + li] = keep[q][e];
      }
  }
  __syncthreads();

  // Row-contiguous stores: each thread writes 4 (fp32) or 8 (bf16) columns
  // at a time, nontemporal (C is not read again by this kernel; every
  // workgroup stores at the same moment, and skipping the L2 allocation
  // measured 8-12% faster on the layer shapes).  Tiles cut by the matrix
  // edge, or rows that are not 16-byte aligned, store element by element.
  constexpr int kVec = BF16_OUT ? 8 : 4;
  constexpr int kVecPerRow = BT / kVec;
  const bool full = m0 + BT <= M && n0 + BT <= N && (N % kVec) == 0 && (reinterpret_cast<uintptr_t>(g.C) & 15) == 0;
  for (int v = tid; v < BT * kVecPerRow; v += kThreads) {
    const int row = v / kVecPerRow, c0 = (v % kVecPerRow) * kVec;
    const float* src = ct + row * Gm::kCRow + c0;
    const int64_t grow = m0 + row, gcol = n0 + c0;
    if (full) {
      if (BF16_OUT) {
        u32x4 o;
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] = f32_to_bf16_rne(src[2 * e]) | (f32_to_bf16_rne(src[2 * e + 1]) << 16);
        __builtin_nontemporal_store(o, reinterpret_cast<u32x4*>(reinterpret_cast<uint16_t*>(g.C) + grow * N + gcol));
      } else {
        const f32x4 o = {src[0], src[1], src[2], src[3]};
        __builtin_nontemporal_store(o, reinterpret_cast<f32x4*>(reinterpret_cast<float*>(g.C) + grow * N + gcol));
      }
    } else if (grow < M) {
      for (int e = 0; e < kVec && gcol + e < N; ++e) {
        if (BF16_OUT)
          reinterpret_cast<uint16_t*>(g.C)[grow * N + gcol + e] = (uint16_t)f32_to_bf16_rne(src[e]);
        else
          reinterpret_cast<float*>(g.C)[grow * N + gcol + e] = src[e];
      }
    }
  }
}

}  // namespace

hipError_t launch_gemm_mxfp4(const GemmArgs& g, bool bf16_out, hipStream_t s) {
  // 128 x 128 tiles unless that leaves more than a quarter of the 256 CUs
  // without a tile; then 64 x 64.
  const int64_t tiles128 = ((g.N + 127) / 128) * ((g.M + 127) / 128);
  const int bt = tiles128 >= 192 ? 128 : 64;
  const dim3 grid((unsigned)((g.N + bt - 1) / bt), (unsigned)((g.M + bt - 1) / bt)), block(kThreads);
  if (bt == 128) {
    if (bf16_out) hipLaunchKernelGGL((gemm_mxfp4_kernel<2, true>), grid, block, 0, s, g);
    else hipLaunchKernelGGL((gemm_mxfp4_kernel<2, false>), grid, block, 0, s, g);
  } else {
    if (bf16_out) hipLaunchKernelGGL((gemm_mxfp4_kernel<1, true>), grid, block, 0, s, g);
    else hipLaunchKernelGGL((gemm_mxfp4_kernel<1, false>), grid, block, 0, s, g);
  }
  return hipGetLastError();
}

}  // namespace wush
