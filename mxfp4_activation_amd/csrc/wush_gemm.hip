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
// TM = 2, 8 at TM = 1), 2 or 4 steps ahead of the MFMAs.  No staging
// registers and no LDS write instructions are involved; each wave waits for
// its own loads with vmcnt and one barrier per step publishes them.
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
// The global-to-LDS copies are issued from inline asm.  Issued through the
// compiler builtin, they make the compiler wait for every outstanding copy
// before any later LDS read (it cannot tell the ring stages apart), which
// drains the ring.  Issued from asm, they are invisible to that analysis;
// the per-step vmcnt waits below order them, and the fragment reads are
// plain LDS loads that the compiler schedules.  Each step is software
// pipelined within the wave: the fragments of step ks + 1 are read while
// the MFMAs of step ks run, from a second set of registers.
//
// At the end each K group writes its partial tile into its own fp32 region
// of LDS; the store pass adds the two and writes C with 16-byte
// row-contiguous stores.
//
// Packed B (PACKED_B): weights re-laid once, offline (pack_b_kernel), as
// the LDS image of every (128-row tile, K step): the B copies then read
// 1 KB (codes) and 256 B (scales) contiguously instead of 8 or 32 rows per
// instruction.  Everything after the copies is the same code, so the
// result is the same bit for bit.

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
constexpr int kPackStep = 128 * kRowB;    // packed B: code bytes of one 128-row tile per step
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
  static_assert(kStages >= kAhead + 2, "ring too short: the stage refilled must not be the one still being read");
  static_assert(kLdsB >= 2 * BT * kCRow * 4, "the two partial output tiles do not fit");
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

// Global-to-LDS copies of 16 and 4 bytes per lane to LDS address `dst`
// (wave-uniform; lane l writes at dst + l * size).  The copy takes its LDS
// base from M0.  M0 is declared clobbered; the compiler reserves M0 and
// warns that it does not preserve it across the statement, which is safe
// here because nothing else in these kernels uses M0 (the only M0 writes in
// their code are these).  The statements have no outputs, so no register
// can be overwritten by a copy in flight.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma16(glb_u8* src, uint32_t dst) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(src), "s"(dst) : "memory", "m0");
}
__device__ __forceinline__ void dma4(glb_u8* src, uint32_t dst) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dword %0, off" ::"v"(src), "s"(dst) : "memory", "m0");
}
#pragma clang diagnostic pop

template <int TM, bool BF16_OUT, bool PACKED_A, bool PACKED_B>
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
  const int64_t K = g.K, M = g.M, N = g.N, ldc = g.ldc;
  const int64_t row_bytes = K / 2, row_scales = K / 32;
  const int nk = (int)(K / 256);

  // Load map.  Code loads: wave w moves rows 8 (TM w + q) .. +7 (q < TM) of
  // both tiles; lane L takes row L / 8 of those 8 and stores LDS slot L % 8,
  // which holds chunk (L % 8) ^ ((row / 2) % 8).
  // Packed operands: 128-row tiles, each step kPackStep code bytes and 1 KB
  // of scales; a 64-row tile (TM = 1) is the second half of its 128-row
  // tile when its first row % 128 == 64.
  const int64_t pt_rows = (n0 / 128) * 128;  // first row of B's packed tile
  const int p_half = (int)((n0 % 128) / 64);
  const int64_t pa_rows = (m0 / 128) * 128;  // the same for A
  const int pa_half = (int)((m0 % 128) / 64);
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
    // Packed B: the tile's step already sits in its LDS image order, so
    // each copy reads 1 KB contiguously (see pack_b_kernel).
    if (PACKED_A)
      a_src[q] = (glb_u8*)g.a_codes + pa_rows * row_bytes + (kPackStep / 2) * pa_half + 1024 * (TM * wave + q) + 16 * lane;
    if (PACKED_B)
      b_src[q] = (glb_u8*)g.b_codes + pt_rows * row_bytes + (kPackStep / 2) * p_half + 1024 * (TM * wave + q) + 16 * lane;
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
  int64_t s_step = 8;  // scale bytes per step: 8 per row, or a packed tile's 1 KB
  if (PACKED_B && !s_is_a) {
    s_src = (glb_u8*)g.b_scales + pt_rows * row_scales + 512 * p_half + 128 * TM * (wave & 3) + 4 * lane;
    s_step = 8 * 128;
  }
  if (PACKED_A && s_is_a) {
    s_src = (glb_u8*)g.a_scales + pa_rows * row_scales + 512 * pa_half + 128 * TM * (wave & 3) + 4 * lane;
    s_step = 8 * 128;
  }
  const int s_dst = (s_is_a ? Gm::kOffSA : Gm::kOffSB) + 128 * TM * (wave & 3);
  // Both operands packed: a tile's scales for one step are 8 BT contiguous
  // bytes in global memory and in LDS, so one 16-byte-per-lane copy (lanes
  // below 32 TM) moves them.  Waves ks % 4 (A) and 4 + ks % 4 (B) take turns,
  // two copies per workgroup and step instead of eight 4-byte ones.
  constexpr bool kScale16 = PACKED_A && PACKED_B;
  glb_u8* const s16_src = kScale16 ? (glb_u8*)(s_is_a ? g.a_scales : g.b_scales) +
                                         (s_is_a ? pa_rows : pt_rows) * row_scales +
                                         512 * (s_is_a ? pa_half : p_half) + 16 * lane
                                   : nullptr;
  const int s16_dst = s_is_a ? Gm::kOffSA : Gm::kOffSB;

  // Step ks lives in ring stage ks % kStages.
  const uint32_t wave_u = (uint32_t)__builtin_amdgcn_readfirstlane(wave);
  auto issue = [&](int ks) {
    const int64_t kc = ks;
    const uint32_t st = (uint32_t)__builtin_amdgcn_readfirstlane((int)(lbase + (ks % Gm::kStages) * Gm::kStageB));
#pragma unroll
    for (int q = 0; q < TM; ++q) {
      dma16(a_src[q] + kc * (PACKED_A ? kPackStep : kRowB), st + 1024 * (TM * wave_u + q));
      dma16(b_src[q] + kc * (PACKED_B ? kPackStep : kRowB), st + Gm::kOffB + 1024 * (TM * wave_u + q));
    }
    if (kScale16) {
      if ((int)(wave_u & 3) == (ks & 3) && s_lane)
        dma16(s16_src + kc * 1024, st + (uint32_t)__builtin_amdgcn_readfirstlane(s16_dst));
    } else if (s_lane) {
      dma4(s_src + kc * s_step, st + (uint32_t)__builtin_amdgcn_readfirstlane(s_dst));
    }
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
  typedef const __attribute__((address_space(3))) u32x4 lds_v4;
  typedef const __attribute__((address_space(3))) uint32_t lds_u32;
  auto read = [&](int ks, Frag& f) {
    const uint32_t st = lbase + (ks % Gm::kStages) * Gm::kStageB;
    // Tile row / column t = 1 is 32 rows further: 4096 B of codes, 256 B of scales.
#pragma unroll
    for (int t = 0; t < TM; ++t) {
      f.a[0][t] = *(lds_v4*)(uintptr_t)(st + fa0 + 4096 * t);
      f.a[1][t] = *(lds_v4*)(uintptr_t)(st + fa1 + 4096 * t);
      f.b[0][t] = *(lds_v4*)(uintptr_t)(st + fb0 + 4096 * t);
      f.b[1][t] = *(lds_v4*)(uintptr_t)(st + fb1 + 4096 * t);
      f.sa[t] = *(lds_u32*)(uintptr_t)(st + fsa + 256 * t);
      f.sb[t] = *(lds_u32*)(uintptr_t)(st + fsb + 256 * t);
    }
  };
  auto mfma = [&](const Frag& f) {
    uint32_t sa[TM], sb[TM];
#pragma unroll
    for (int t = 0; t < TM; ++t) {
      sa[t] = f.sa[t] >> shift;
      sb[t] = f.sb[t] >> shift;
    }
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TM; ++j) acc[i][j] = mfma_fp4<0>(f.a[0][i], f.b[0][j], acc[i][j], sa[i], sb[j]);
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TM; ++j) acc[i][j] = mfma_fp4<2>(f.a[1][i], f.b[1][j], acc[i][j], sa[i], sb[j]);
    // The MFMAs are pure operations: without this the compiler sinks them
    // past the next step's barrier, which serializes the pipeline.
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TM; ++j) asm volatile("" : "+v"(acc[i][j]));
  };

  // sync(ks): wait for this wave's loads of step ks (those of the later
  // steps already issued may stay in flight), barrier (every wave's loads
  // of step ks have landed), then refill stage (ks + kAhead) % kStages.
  // That stage last held step ks + kAhead - kStages <= ks - 2, whose
  // fragments every wave read and consumed (in mfma) before this barrier;
  // only step ks - 1's reads may still be in flight when the barrier
  // passes, and its stage is a different one.
  // With kScale16 a wave issues a scale copy on one step in four; counting
  // only its 2 TM code copies per step waits for at most one later copy too.
  constexpr int LPS = kScale16 ? 2 * TM : Gm::kLoadsPerStep;
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
  // Software pipeline: the fragments of step ks + 1 are read while the
  // MFMAs of step ks run.  Unrolled by two so that the two fragment sets
  // keep fixed registers.
  Frag f0, f1;
  sync(0);
  read(0, f0);
  int ks = 0;
  for (; ks + 2 < nk; ks += 2) {
    sync(ks + 1);
    read(ks + 1, f1);
    mfma(f0);
    sync(ks + 2);
    read(ks + 2, f0);
    mfma(f1);
  }
  if (ks + 1 < nk) {
    sync(ks + 1);
    read(ks + 1, f1);
    mfma(f0);
    mfma(f1);
  } else {
    mfma(f0);
  }
  wait_barrier<0>();

  // Each K-split group writes its partial tile into its own fp32 region of
  // LDS (rows padded); the store pass adds the two.  Lane (j + 32h) of an
  // MFMA tile holds rows 8 (r / 4) + 4 h + r % 4 of column j in accumulator
  // register r.
  float* const ct0 = reinterpret_cast<float*>(L);
  float* const ct1 = ct0 + BT * Gm::kCRow;
  {
    float* ct = grp ? ct1 : ct0;
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TM; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = 32 * TM * wm + 32 * i + 8 * (r / 4) + 4 * lh + (r % 4);
          ct[row * Gm::kCRow + 32 * TM * wn + 32 * j + li] = acc[i][j][r];
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
  const bool full = m0 + BT <= M && n0 + BT <= N && (ldc % kVec) == 0 && (reinterpret_cast<uintptr_t>(g.C) & 15) == 0;
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  for (int v = tid; v < BT * kVecPerRow; v += kThreads) {
    const int row = v / kVecPerRow, c0 = (v % kVecPerRow) * kVec;
    float src[kVec];
#pragma unroll
    for (int q = 0; q < kVec / 4; ++q) {
      const f32x4 p0 = *reinterpret_cast<const f32x4*>(ct0 + row * Gm::kCRow + c0 + 4 * q);
      const f32x4 p1 = *reinterpret_cast<const f32x4*>(ct1 + row * Gm::kCRow + c0 + 4 * q);
#pragma unroll
      for (int e = 0; e < 4; ++e) src[4 * q + e] = p0[e] + p1[e];
    }
    const int64_t grow = m0 + row, gcol = n0 + c0;
    if (full) {
      if (BF16_OUT) {
        u32x4 o;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const f32x2 pr = {src[2 * e], src[2 * e + 1]};
          o[e] = __builtin_bit_cast(uint32_t, __builtin_convertvector(pr, bf16x2));
        }
        __builtin_nontemporal_store(o, reinterpret_cast<u32x4*>(reinterpret_cast<uint16_t*>(g.C) + grow * ldc + gcol));
      } else {
        const f32x4 o = {src[0], src[1], src[2], src[3]};
        __builtin_nontemporal_store(o, reinterpret_cast<f32x4*>(reinterpret_cast<float*>(g.C) + grow * ldc + gcol));
      }
    } else if (grow < M) {
      for (int e = 0; e < kVec && gcol + e < N; ++e) {
        if (BF16_OUT)
          reinterpret_cast<uint16_t*>(g.C)[grow * ldc + gcol + e] = (uint16_t)f32_to_bf16_rne(src[e]);
        else
          reinterpret_cast<float*>(g.C)[grow * ldc + gcol + e] = src[e];
      }
    }
  }
}

}  // namespace

template <int TM, bool BF16_OUT>
static void launch_tiles_out(const GemmArgs& g, int layout, hipStream_t s) {
  constexpr int bt = 64 * TM;
  const dim3 grid((unsigned)((g.N + bt - 1) / bt), (unsigned)((g.M + bt - 1) / bt)), block(kThreads);
  if (layout == kPackedAB) hipLaunchKernelGGL((gemm_mxfp4_kernel<TM, BF16_OUT, true, true>), grid, block, 0, s, g);
  else if (layout == kPackedB) hipLaunchKernelGGL((gemm_mxfp4_kernel<TM, BF16_OUT, false, true>), grid, block, 0, s, g);
  else hipLaunchKernelGGL((gemm_mxfp4_kernel<TM, BF16_OUT, false, false>), grid, block, 0, s, g);
}

template <int TM>
static void launch_tiles(const GemmArgs& g, bool bf16_out, int layout, hipStream_t s) {
  if (bf16_out) launch_tiles_out<TM, true>(g, layout, s);
  else launch_tiles_out<TM, false>(g, layout, s);
}

hipError_t launch_gemm_mxfp4(const GemmArgs& g, bool bf16_out, int layout, hipStream_t s) {
  // One workgroup per CU (by LDS), 256 CUs.  128 x 128 tiles unless that
  // leaves more than a quarter of the CUs without a tile; then 64 x 64.
  const int64_t mt = (g.M + 127) / 128, nt = (g.N + 127) / 128;
  const int64_t tiles128 = mt * nt;
  if (tiles128 < 192) {
    launch_tiles<1>(g, bf16_out, layout, s);
    return hipGetLastError();
  }
  // A last wave of 128 x 128 tiles that would occupy a quarter of the CUs
  // or fewer (Qwen3-14B's 5120-wide outputs: 320 tiles) runs as 64 x 64
  // tiles instead, four times as many, which fill that wave at about half
  // the time of a 128 x 128 wave: the columns of the whole waves go to one
  // launch, the remaining columns to a second on the same stream.  n1 is a
  // multiple of 128, so B's offset is the same in both layouts.
  const int64_t waves = tiles128 / 256, tail = tiles128 % 256;
  if (tail > 0 && 4 * tail <= 256 && (256 * waves) % mt == 0) {
    const int64_t n1 = (256 * waves / mt) * 128;
    if (n1 > 0 && n1 < g.N) {
      GemmArgs g1 = g, g2 = g;
      g1.N = n1;
      g2.N = g.N - n1;
      g2.b_codes = g.b_codes + n1 * (g.K / 2);
      g2.b_scales = g.b_scales + n1 * (g.K / 32);
      g2.C = static_cast<uint8_t*>(g.C) + n1 * (bf16_out ? 2 : 4);
      launch_tiles<2>(g1, bf16_out, layout, s);
      const hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
      launch_tiles<1>(g2, bf16_out, layout, s);
      return hipGetLastError();
    }
  }
  launch_tiles<2>(g, bf16_out, layout, s);
  return hipGetLastError();
}

// Packed B.  For each 128-row tile t of B and each K step ks (256
// elements), 16 KB of codes and 1 KB of scales, laid out exactly as the
// GEMM kernel stages that step in LDS: byte 1024 i + 16 L of the code
// block holds 16-byte chunk (L % 8) ^ ((r / 2) % 8) of row r = 8 i + L / 8,
// and the scale block holds the tile's 128 rows of 8 scale bytes.  Rows
// past N repeat row N - 1 (the kernel never stores their results).  One
// thread per 16 code bytes and per 8 scale bytes.
__global__ __launch_bounds__(256) void pack_b_kernel(const uint8_t* __restrict__ codes,
                                                     const uint8_t* __restrict__ scales, int64_t N, int64_t K,
                                                     uint8_t* __restrict__ pcodes, uint8_t* __restrict__ pscales,
                                                     int64_t n_code16, int64_t n_scale8) {
  const int64_t nk = K / 256;
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n_code16) {
    const int64_t tile = i / (nk * 1024), rem = i - tile * nk * 1024;
    const int64_t ks = rem / 1024;
    const int o = (int)(rem - ks * 1024), ins = o / 64, L = o % 64;
    const int r = 8 * ins + L / 8;
    const int chunk = (L % 8) ^ ((r >> 1) & 7);
    int64_t row = tile * 128 + r;
    row = row < N ? row : N - 1;
    const u32x4 v = *reinterpret_cast<const u32x4*>(codes + row * (K / 2) + ks * kRowB + 16 * chunk);
    *reinterpret_cast<u32x4*>(pcodes + 16 * i) = v;
  }
  if (i < n_scale8) {
    const int64_t tile = i / (nk * 128), rem = i - tile * nk * 128;
    const int64_t ks = rem / 128;
    const int r = (int)(rem - ks * 128);
    int64_t row = tile * 128 + r;
    row = row < N ? row : N - 1;
    const u32x2 v = *reinterpret_cast<const u32x2*>(scales + row * (K / 32) + ks * 8);
    *reinterpret_cast<u32x2*>(pscales + 8 * i) = v;
  }
}

hipError_t launch_pack_b(const uint8_t* codes, const uint8_t* scales, int64_t N, int64_t K, uint8_t* pcodes,
                         uint8_t* pscales, hipStream_t s) {
  const int64_t tiles = (N + 127) / 128, nk = K / 256;
  const int64_t n_code16 = tiles * nk * 1024, n_scale8 = tiles * nk * 128;
  const int64_t blocks = (n_code16 + 255) / 256;
  hipLaunchKernelGGL(pack_b_kernel, dim3((unsigned)blocks), dim3(256), 0, s, codes, scales, N, K, pcodes, pscales,
                     n_code16, n_scale8);
  return hipGetLastError();
}

}  // namespace wush
