// Fused WUSH transform + 4-bit quantization kernels for gfx950 (CDNA4).
//
// The computation follows "WUSH: Near-Optimal Adaptive Transforms for LLM
// Quantization".  Each G-channel block of a token row is multiplied by its
// own T_wush(c) (Eq. 8), then RTN AbsMax-quantized in groups of G (deep
// dive, sections 3.4.6 and 3.4.7; Eq. 10).  The pages' own kernel is a
// CUTLASS GEMM in which each thread block takes one block index c.  This
// design keeps only the idea that c is not a GEMM dimension.  The rest is
// laid out for wave64 matrix cores:
//
//  * Tile.  One wave owns a panel of 32 channels (one G=32 block, or two
//    G=16 blocks) for 32 tokens, and computes Y^T = T * X^T with two
//    v_mfma_f32_32x32x16_bf16.  The A operand is T, loaded once per wave
//    into VGPRs and reused across the wave's token tiles.  The B operand is
//    X.  MFMA k-slice kk takes channels 16kk..16kk+15 of the panel, so each of
//    the two 16-byte loads of a wave covers 32 contiguous bytes of 32 rows.
//  * Output rows of T are permuted when the A fragment is loaded.  After the
//    permutation, lane (n, h) holds outputs 16h..16h+15 of token n in
//    accumulator registers 0..15.  A 32-group's AbsMax is then an in-lane max
//    plus one exchange between lanes l and l^32.  A 16-group (NVFP4, with a
//    block-diagonal pair as A) is entirely in-lane.
//  * Exact scales.  A second MFMA pair bounds sum_j |T_ij||x_j| (MXFP4:
//    max|T| times the token's L1 norm; INT4 and NVFP4: the per-output sums
//    from |T| x |x|), which bounds how far the fp32 accumulation can be
//    from the exact sum.  If a group's scale decision is not constant over
//    [amax - d, amax + d], the outputs that can hold the group's maximum
//    are recomputed in float64 and rounded once to fp32, and the scale is
//    decided again on their maximum, the exactly rounded AbsMax.  The codes
//    keep the matrix-core values.
//
// Memory layout and ABI: see include/wush.h.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "wush_kernels.h"

namespace wush {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kWaves = kWavesPerGroup;  // waves per workgroup

__device__ __forceinline__ f32x16 mfma32(u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

__device__ __forceinline__ int lane_id() { return __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u)); }

// Output row held by A-operand row i, chosen so that D register r of lane
// half h is output 16h + r.  The 32x32 D layout puts row
// 8*(r/4) + 4*h + (r%4) in register r of half h.
__device__ __forceinline__ int permuted_row(int i) {
  return 16 * ((i >> 2) & 1) + 4 * (i >> 3) + (i & 3);
}

// max(v[l], v[l ^ 32]) for non-negative v.  v_permlane32_swap returns v[l]
// and v[l ^ 32] in its two results, in an order that depends on the lane
// half.  Non-negative floats order like their bit patterns.
__device__ __forceinline__ float max_halves(float v) {
  auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(p[0] > p[1] ? p[0] : p[1]);
}

// v[l] + v[l ^ 32], with the operands in the same order in both lanes of a
// pair, so both get the same rounded sum.
__device__ __forceinline__ double sum_halves(double v) {
  uint64_t b = __builtin_bit_cast(uint64_t, v);
  uint32_t lo = (uint32_t)b, hi = (uint32_t)(b >> 32);
  auto pl = __builtin_amdgcn_permlane32_swap(lo, lo, false, false);
  auto ph = __builtin_amdgcn_permlane32_swap(hi, hi, false, false);
  double a = __builtin_bit_cast(double, ((uint64_t)ph[0] << 32) | pl[0]);
  double c = __builtin_bit_cast(double, ((uint64_t)ph[1] << 32) | pl[1]);
  return a + c;
}

__device__ __forceinline__ float max_abs16(const f32x16& v) {
  float m = 0.0f;
#pragma unroll
  for (int r = 0; r < 16; ++r) m = fmaxf(m, fabsf(v[r]));
  return m;
}

__device__ __forceinline__ float max16(const f32x16& v) {
  float m = 0.0f;
#pragma unroll
  for (int r = 0; r < 16; ++r) m = fmaxf(m, v[r]);
  return m;
}

// ---------------------------------------------------------------- codecs

// E2M1 conversion of a pair: v_cvt_scalef32_pk_fp4_f32 divides both values
// by 2^(exponent field of `scale`), rounds to nearest even, saturates at +-6,
// keeps the sign of zero and writes a byte (first value in the low nibble)
// into byte BYTE of `old`.  With scale = 1.0 it is plain E2M1 rounding.
template <int BYTE>
__device__ __forceinline__ uint32_t cvt_e2m1x2(uint32_t old, float a, float b, float scale) {
  return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(old, a, b, scale, BYTE);
}

// OCP E4M3FN code of a non-negative finite x: nearest, ties to even, with
// saturation at 448 (code 126).
__device__ __forceinline__ uint32_t e4m3_code(float x) {
  if (x >= 448.0f) return 126u;
  if (x < 0.015625f) {  // below 2^-6: subnormal grid, step 2^-9
    return (uint32_t)__builtin_rintf(x * 512.0f);  // 0..8; 8 is 2^-6 = code 8
  }
  uint32_t b = __float_as_uint(x);
  b = b + 0x7FFFFu + ((b >> 20) & 1u);  // round mantissa to 3 bits, ties to even
  uint32_t c = (b >> 20) - (120u << 3);  // rebias exponent 127 -> 7
  return c > 126u ? 126u : c;
}

__device__ __forceinline__ float e4m3_value(uint32_t c) {
  uint32_t e = c >> 3, m = c & 7u;
  if (e == 0) return (float)m * 0.001953125f;  // m * 2^-9
  return __uint_as_float(((e + 120u) << 23) | (m << 20));
}

__device__ __forceinline__ uint32_t f16_bits(float x) {
  _Float16 h = (_Float16)x;  // v_cvt_f16_f32: round to nearest even
  return (uint32_t)__builtin_bit_cast(uint16_t, h);
}

__device__ __forceinline__ float f16_value(uint32_t b) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)b);
}

// fp32(x / 7), the correctly rounded quotient, for finite x >= 0: the
// product with fp32(1/7) and one FMA correction of its residual.  Equal to
// the IEEE quotient for every non-negative finite fp32 x, subnormals
// included (checked exhaustively on the host), at three instructions
// instead of the ten of a division.
__device__ __forceinline__ float div7(float x) {
  constexpr float r = 1.0f / 7.0f;
  const float q = x * r;
  return __builtin_fmaf(__builtin_fmaf(-q, 7.0f, x), r, q);
}

// fp32(1 / s) for s the value of a positive finite fp16 number: the
// hardware reciprocal with one FMA correction.  Equal to the IEEE quotient
// for every such s (checked exhaustively on the device against its own
// division and against the host's).
__device__ __forceinline__ float recip_f16_value(float s) {
  const float r0 = __builtin_amdgcn_rcpf(s);
  return __builtin_fmaf(__builtin_fmaf(-s, r0, 1.0f), r0, r0);
}

// ---------------------------------------------------------------- scale decisions
//
// Each decision is a monotone function of amax.  The checks report whether
// it could change anywhere in [amax - d, amax + d].  When it cannot, the
// decision at the top of the interval (returned through the reference) is
// the decision at amax itself, so the caller reuses it.

// INT4: q = fp32(amax / 7), the value the fp16 scale rounds; `bits` gets
// the fp16 scale.
__device__ __forceinline__ bool int4_unsure(float q, float d, uint32_t& bits) {
  float dq = d * 0.15f + q * 0x1p-21f;
  bits = f16_bits(q + dq);
  return f16_bits(fmaxf(q - dq, 0.0f)) != bits;
}

// NVFP4: the E4M3 code of fp32(fp32(amax / 6) / g) goes to `code`.
// The ratio is formed as amax * k6g with k6g = fp32(1 / fp32(6 g)): three
// roundings, against two in fp32(fp32(amax / 6) / g), so the two differ by
// at most about 5 * 2^-24 of the ratio.  The interval [ratio - dr,
// ratio + dr] covers that as well as d; when its two ends share an E4M3
// code, that code is the one of the exact chain for every amax in
// [amax - d, amax + d].  No division on this path.
__device__ __forceinline__ bool nv_unsure(float amax, float d, float g, float k6g, uint32_t& code) {
  code = 0u;
  if (!(g > 0.0f)) return false;  // every code is zero whatever amax is
  if (amax == 0.0f) return d > 0.0f && e4m3_code(d * k6g * (1.0f + 0x1p-20f)) != 0u;
  const float ratio = amax * k6g;
  // ratio scales linearly with amax; the relative slack covers roundings
  // (2^-20) and the ratio's own approximation (2^-21)
  const float dr = ratio * (d * __builtin_amdgcn_rcpf(amax)) * 1.01f + ratio * (0x1p-20f + 0x1p-21f);
  code = e4m3_code(ratio + dr);
  return e4m3_code(fmaxf(ratio - dr, 0.0f)) != code;
}

// ---------------------------------------------------------------- fragments

struct Frag {
  u32x4 t0, t1;  // T rows (permuted), k-slices 0 and 1 of this lane half
  u32x4 a0, a1;  // |T|
};

// Lane (i, h) of the A operand holds row permuted_row(i).  For k-slice kk
// its 8 values are columns 16kk + 8h .. 16kk + 8h + 7 of the panel.
// G == 32: panel p is block p.  G == 16: panel p is blocks 2p and 2p+1
// placed block-diagonally, so output rows 16kk..16kk+15 see only block
// 2p + kk through k-slice kk.
template <int G>
__device__ __forceinline__ Frag load_t(const uint16_t* __restrict__ T, int p, int C, int lane) {
  Frag f;
  const int i = lane & 31, h = lane >> 5;
  const int row = permuted_row(i);
  const u32x4 z = {0u, 0u, 0u, 0u};
  f.t0 = z;
  f.t1 = z;
  if (G == 32) {
    const uint16_t* src = T + ((size_t)p * 32 + row) * 32 + 8 * h;
    f.t0 = *reinterpret_cast<const u32x4*>(src);
    f.t1 = *reinterpret_cast<const u32x4*>(src + 16);
  } else {
    const int kk = row >> 4, blk = 2 * p + kk;
    if (blk < C) {
      u32x4 t = *reinterpret_cast<const u32x4*>(T + (size_t)blk * 256 + (row & 15) * 16 + 8 * h);
      if (kk == 0) f.t0 = t;
      else f.t1 = t;
    }
  }
  f.a0 = z;  // |T|: with_abs() fills it in where the bound needs it
  f.a1 = z;
  return f;
}

__device__ __forceinline__ void with_abs(Frag& f) {
  const u32x4 mask = {0x7FFF7FFFu, 0x7FFF7FFFu, 0x7FFF7FFFu, 0x7FFF7FFFu};
  f.a0 = f.t0 & mask;
  f.a1 = f.t1 & mask;
}

struct XTile {
  u32x4 b0, b1;
};

__device__ __forceinline__ u32x4 load16_nt(const uint16_t* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

typedef const __attribute__((address_space(3))) uint8_t lds_cu8;

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Recompute token `n`'s 32 outputs of the current panel in float64 and
// write them into the accumulator of lanes (n, 0) and (n, 1).  Lane (i, h)
// owns output row permuted_row(i): its T fragment (the MFMA A operand) is
// exactly its half-row of T, and it forms the half-h partial sum; lane
// l ^ 32 holds the other half.  Token n's channels of the panel come from
// the staged tile (LDS address `xtok`, its row at this panel; the same 16
// bytes for every lane of a half, a broadcast read).  The fragment is
// copied through an empty asm statement, so the compiler cannot hoist this
// rare path's float64 conversions of T out of the hot loop into registers
// that stay live.
__device__ __forceinline__ void exact_panel(uint32_t xtok, const Frag& f, f32x16& acc, float* lds, int n, int lane) {
  // Addresses below derive from an opaque copy of the lane id, so the
  // compiler keeps their arithmetic inside this rarely taken path.
  int lds_off = 0;
  asm volatile("" : "+v"(lane), "+v"(lds_off));
  lds += lds_off;
  const int i = lane & 31, h = lane >> 5;
  const int row = permuted_row(i);
  u32x4 tk[2] = {f.t0, f.t1};
  asm volatile("" : "+v"(tk[0]), "+v"(tk[1]));
  lds_cu8* xp = (lds_cu8*)(uintptr_t)(xtok + 16 * h);
  const u32x4 bk[2] = {*reinterpret_cast<const __attribute__((address_space(3))) u32x4*>(xp),
                       *reinterpret_cast<const __attribute__((address_space(3))) u32x4*>(xp + 32)};
  double s = 0.0;
#pragma unroll
  for (int kk = 0; kk < 2; ++kk) {
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const uint32_t xw = bk[kk][w];
      const uint32_t tw = tk[kk][w];
      s = __builtin_fma((double)bf16_lo(tw), (double)bf16_lo(xw), s);
      s = __builtin_fma((double)bf16_hi(tw), (double)bf16_hi(xw), s);
    }
  }
  const float y = (float)sum_halves(s);
  if (h == 0) lds[row] = y;
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  if (i == n) {
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[r] = lds[16 * h + r];
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// A-operand row that holds output k: the inverse of permuted_row.
__device__ __forceinline__ int row_of_output(int k) {
  return (k & 3) | (((k >> 4) & 1) << 2) | (((k >> 2) & 3) << 3);
}

// Exact value of output k of this lane's token, rounded once to fp32.
// Lane (n, h) multiplies its own 16 channels of the token (its B operand:
// k-slice 0 at LDS address xo, k-slice 1 at xo + 32) by the matching 16
// entries of T row k, which A-operand lane (row_of_output(k), h) holds;
// ds_bpermute fetches them.  Each product of two bf16 values is exact in
// float64; the two halves are summed with sum_halves, so lanes (n, 0) and
// (n, 1) get the same value when both ask for the same k.  Lanes may ask
// for different outputs (one per token), which makes the pass lane-parallel.
// The channels are read one word pair at a time through an opaque address:
// held in registers across the caller's loop they would cost 8 VGPRs, and
// their float64 conversions, hoisted, 32.
__device__ __forceinline__ float exact_output(const Frag& f, uint32_t xo, int k, int lane) {
  asm volatile("" : "+v"(xo));
  typedef const __attribute__((address_space(3))) uint32_t lds_u32;
  const int src = (row_of_output(k) + (lane & 32)) << 2;  // byte address of the source lane
  double s = 0.0;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const uint32_t x0 = *reinterpret_cast<lds_u32*>((lds_cu8*)(uintptr_t)(xo + 4 * w));
    const uint32_t x1 = *reinterpret_cast<lds_u32*>((lds_cu8*)(uintptr_t)(xo + 32 + 4 * w));
    const uint32_t t0 = (uint32_t)__builtin_amdgcn_ds_bpermute(src, (int)f.t0[w]);
    const uint32_t t1 = (uint32_t)__builtin_amdgcn_ds_bpermute(src, (int)f.t1[w]);
    s = __builtin_fma((double)bf16_lo(t0), (double)bf16_lo(x0), s);
    s = __builtin_fma((double)bf16_hi(t0), (double)bf16_hi(x0), s);
    s = __builtin_fma((double)bf16_lo(t1), (double)bf16_lo(x1), s);
    s = __builtin_fma((double)bf16_hi(t1), (double)bf16_hi(x1), s);
  }
  return (float)sum_halves(s);
}

// 16 values -> 16 E2M1 codes in two words, value r in nibble r.  `scale` is
// applied by the conversion as a division by 2^(its exponent field).
__device__ __forceinline__ u32x2 pack_e2m1(const f32x16& v, float scale) {
  // Each word's four bytes are all written below, so any initial value works.
  uint32_t w0 = __float_as_uint(scale), w1 = w0;
  w0 = cvt_e2m1x2<0>(w0, v[0], v[1], scale);
  w0 = cvt_e2m1x2<1>(w0, v[2], v[3], scale);
  w0 = cvt_e2m1x2<2>(w0, v[4], v[5], scale);
  w0 = cvt_e2m1x2<3>(w0, v[6], v[7], scale);
  w1 = cvt_e2m1x2<0>(w1, v[8], v[9], scale);
  w1 = cvt_e2m1x2<1>(w1, v[10], v[11], scale);
  w1 = cvt_e2m1x2<2>(w1, v[12], v[13], scale);
  w1 = cvt_e2m1x2<3>(w1, v[14], v[15], scale);
  u32x2 w = {w0, w1};
  return w;
}

// INT4 element: rne(clamp(y * r, -7, 7)) as a two's-complement nibble.  After
// adding 1.5 * 2^23, the low mantissa bits of the fp32 sum hold the rounded
// integer.  CLAMP = false skips the clamp where it cannot change the
// result (see quantize_panel).
template <bool CLAMP>
__device__ __forceinline__ uint32_t int4_bits(float y, float r) {
  float v = y * r;
  if (CLAMP) v = fminf(fmaxf(v, -7.0f), 7.0f);
  return __float_as_uint(v + 12582912.0f);
}

// Pack 16 INT4 values: v_perm_b32 gathers the low byte of four results into
// one word (even elements in one word, odd in the other).  Then the two words
// merge as nibble pairs.
template <bool CLAMP>
__device__ __forceinline__ uint32_t pack_int4x8(const f32x16& v, int base, float r) {
  uint32_t q[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) q[k] = int4_bits<CLAMP>(v[base + k], r);
  // bytes {q0, q2, q4, q6} and {q1, q3, q5, q7}
  uint32_t e01 = __builtin_amdgcn_perm(q[2], q[0], 0x0c0c0400u);  // [q0.b0, q2.b0, 0, 0]
  uint32_t e23 = __builtin_amdgcn_perm(q[6], q[4], 0x04000c0cu);  // [0, 0, q4.b0, q6.b0]
  uint32_t o01 = __builtin_amdgcn_perm(q[3], q[1], 0x0c0c0400u);
  uint32_t o23 = __builtin_amdgcn_perm(q[7], q[5], 0x04000c0cu);
  uint32_t ev = (e01 | e23) & 0x0F0F0F0Fu;
  uint32_t od = (o01 | o23) & 0x0F0F0F0Fu;
  return ev | (od << 4);
}

template <bool CLAMP>
__device__ __forceinline__ u32x2 pack_int4(const f32x16& v, float r) {
  u32x2 w = {pack_int4x8<CLAMP>(v, 0, r), pack_int4x8<CLAMP>(v, 8, r)};
  return w;
}

// Bound on |fp32 MFMA result - exact sum| for a group whose |T||x| sums
// peak at bound * bound_scale * 2^17.  The accumulation has at most 63
// roundings of partial sums bounded by that peak, each below 2^-23 relative
// (truncation is the worst case), so 2^-17 of the peak covers it; the
// caller folds 2^-17 into bound_scale.  A term of 2^-21 * amax covers the
// final rounding of y to fp32.  2^-120 covers products flushed at the
// bottom of the fp32 range.
__device__ __forceinline__ float err_bound(float bound, float bound_scale, float amax) {
  return __builtin_fmaf(bound, bound_scale, __builtin_fmaf(0x1p-21f, amax, 0x1p-120f));
}

// Workgroup -> (panel group, token group).  Workgroups are dispatched
// round-robin over the 8 XCDs.  When the count divides evenly, each XCD
// gets a contiguous range of the logical order:
// - panel-major (token_major == 0): an XCD covers a few panels over all
//   tokens, so its L2 fetches each T panel once.  When the whole grid is
//   resident at once, every T fetch competes with the first X loads, and
//   this order keeps them to 1/8 of T per XCD.
// - token-major (token_major != 0): an XCD covers whole token rows, so the
//   workgroups resident together read contiguous rows and complete each
//   row's scale line in one L2.  With several waves of workgroups the T
//   fetches are spread over the waves.
__device__ __forceinline__ void wg_coords(int n_pg, int n_tg, int token_major, int& pg, int& tg) {
  int b = blockIdx.x;
  int n = n_pg * n_tg;
  int logical = b;
  if ((n & 7) == 0) logical = (b & 7) * (n >> 3) + (b >> 3);
  if (token_major) {
    tg = logical / n_pg;
    pg = logical - tg * n_pg;
  } else {
    pg = logical / n_tg;
    tg = logical - pg * n_tg;
  }
}

// Per-group scale and code computation for one panel of one 32-token tile.
// Input: the panel's accumulators (lane (n, h) holds outputs 16h..16h+15 of
// token n) and `bound`, an upper bound on sum_j |T_kj x_j| over the lane's
// group.  Output: this lane's 16 codes (two words) and its scale bits.
// Groups whose scale decision falls within the accumulation error bound of
// a boundary first get their exact AbsMax, from the few outputs that can
// hold it.
template <int FMT>
__device__ __forceinline__ u32x2 quantize_panel(f32x16& acc, float bound, float bound_scale, const Frag& f,
                                                uint32_t tile, int tile_stride, float g, float k6g,
                                                const float* rtab, int lane, uint32_t& scale_bits,
                                                uint32_t& n_exact) {
  constexpr int G = (FMT == kNVFP4) ? 16 : 32;
  float amax = max_abs16(acc);
  if (G == 32) amax = max_halves(amax);
  const float d = err_bound(bound, bound_scale, amax);
  bool unsure;
  uint32_t sdec = 0u;  // INT4 / NVFP4: the settled scale bits
  if (FMT == kMXFP4) {
    // The E8M0 code depends only on the exponent field of amax.  It is
    // settled when amax - d and amax + d share sign and exponent field.
    unsure = (__float_as_uint(amax - d) ^ __float_as_uint(amax + d)) > 0x007FFFFFu;
  } else if (FMT == kINT4) {
    unsure = int4_unsure(div7(amax), d, sdec);
  } else {
    unsure = nv_unsure(amax, d, g, k6g, sdec);
  }
  uint64_t pending = __ballot(unsure);
  if (pending) {
    // The lane's own 16 channels of the token sit in the staged tile at
    // `xo` (k-slice 0) and xo + 32 (k-slice 1): its B operand.
    typedef const __attribute__((address_space(3))) u32x4 lds_u32x4;
    const int h = lane >> 5;
    const uint32_t xo = tile + (uint32_t)((lane & 31) * tile_stride + 16 * h);
    // MXFP4: a token whose channels in this panel are all zero (either
    // sign) has y = 0 exactly, and the matrix cores return exactly zero for
    // it, so it needs no recompute.  Zero-padded rows would otherwise all
    // land here: the bound's 2^-120 term leaves their interval across
    // several E8M0 codes.  (The INT4 and NVFP4 decisions are already
    // settled for them: fp16 and E4M3 both round that interval to 0.)
    // Such a token's group has amax = 0, so the check (an LDS re-read) runs
    // only when an unsure group has amax = 0; it cost about 0.24 us per
    // 4096 x 4096 launch when it ran in every recompute.
    if (FMT == kMXFP4 && __ballot(unsure && amax == 0.0f)) {
      const u32x4 q0 = *reinterpret_cast<lds_u32x4*>((lds_cu8*)(uintptr_t)xo);
      const u32x4 q1 = *reinterpret_cast<lds_u32x4*>((lds_cu8*)(uintptr_t)(xo + 32));
      const uint32_t any = (q0[0] | q0[1] | q0[2] | q0[3] | q1[0] | q1[1] | q1[2] | q1[3]) & 0x7FFF7FFFu;
      const uint64_t zl = __ballot(any == 0u);
      const uint64_t zt = zl & (zl >> 32) & 0xFFFFFFFFull;  // both halves of token n zero
      pending &= ~(zt | (zt << 32));
      unsure = unsure && !((zt >> (lane & 31)) & 1u);
    }
    n_exact += (uint32_t)__builtin_popcountll((pending | (pending >> 32)) & 0xFFFFFFFFull);  // wave-uniform
    // Candidates: every output's exact value is within d of its
    // matrix-core value, so the exact maximum is at least amax - d and the
    // output that holds it has |y^_k| >= amax - 2d.  The cut is taken at
    // amax - 2.25d: d >= 2^-21 amax, so the extra quarter covers the
    // rounding of the subtraction.  Only the candidates are recomputed, one
    // output per token per pass, all tokens of the tile at once; the
    // maximum over a group's candidates is its exact AbsMax.  The codes
    // keep the matrix-core values: with the exact scale they can differ
    // from the exactly rounded ones only within the accumulation bound of a
    // rounding midpoint.
    // Bit r of cand: |y^_r| > lo, the sign of lo - |y^_r| shifted in from
    // the top (v_alignbit).  The comparison is strict, which still keeps
    // the output holding the maximum: its |y^| >= amax - 2d > lo since
    // d > 0.  A settled group's cut is +inf: no candidates.
    const float lo = unsure ? amax - 2.25f * d : __builtin_inff();
    uint32_t cand = 0u;
#pragma unroll
    for (int r = 15; r >= 0; --r) cand = __builtin_amdgcn_alignbit(cand, __float_as_uint(lo - fabsf(acc[r])), 31);
    // Both lanes of a token see its 32 candidate bits, output k at bit k:
    // in both halves the swap's first result is the value of lane (n, 0),
    // the second that of lane (n, 1).
    // The wave takes as many passes as its token with the most candidates:
    // almost always one, at most 32 (32 near-equal outputs).  A pass costs
    // about what recomputing one token's whole panel does.
    const auto sw = __builtin_amdgcn_permlane32_swap(cand, cand, false, false);
    uint32_t m = sw[0] | (sw[1] << 16);
    if (__ballot(m != 0u)) {
      float ex = 0.0f;
      do {
        const int kk = m ? __builtin_ctz(m) : 0;
        const float yk = exact_output(f, xo, kk, lane);
        if (m && (G == 32 || (kk >> 4) == h)) ex = fmaxf(ex, fabsf(yk));
        m &= m - 1u;
      } while (__ballot(m != 0u));
      // An unsure group has a candidate (its largest |y^_k| is one); a
      // settled group keeps its amax.
      if (unsure) amax = ex;
    }
    // Decide again at the new amax (the same value for the settled groups).
    if (FMT == kINT4) sdec = f16_bits(div7(amax));
    if (FMT == kNVFP4 && g > 0.0f) sdec = e4m3_code((amax / 6.0f) / g);
  }
  if (FMT == kMXFP4) {
    // 2^e with e = floor(log2 amax) - 2, clamped at 2^-127 (code 0): the
    // exponent field minus 2.  Non-negative floats compare like integers.
    const int eb = (int)(__float_as_uint(amax) & 0x7F800000u) - (2 << 23);
    const uint32_t sc = (uint32_t)(eb > 0 ? eb : 0);
    scale_bits = sc >> 23;
    return pack_e2m1(acc, __uint_as_float(sc));
  } else if (FMT == kINT4) {
    const float s = f16_value(sdec);
    scale_bits = sdec;
    // fp32(1 / s); 0 for a zero or infinite scale
    const float r = (sdec & 0x7FFFu) != 0u && (sdec & 0x7C00u) != 0x7C00u ? recip_f16_value(s) : 0.0f;
    // With a normal fp16 scale, |y| <= amax and s >= fp32(amax / 7) (1 -
    // 2^-11) give |y r| <= 7.0035 after the roundings of r and of the
    // product: below 7.5, so rounding already lands in [-7, 7].  Zero and
    // subnormal scales (tiny amax) need the clamp; an infinite scale gives
    // r = 0.  The branch is taken per wave.
    if (__ballot((sdec & 0x7C00u) == 0u)) return pack_int4<true>(acc, r);
    return pack_int4<false>(acc, r);
  } else {
    const uint32_t code = sdec;  // 0 when g <= 0
    // fp32(1 / fp32(E4M3(code) g)), or 0: from the workgroup's table
    const float r = rtab[code];
    scale_bits = code;
    f32x16 v;
#pragma unroll
    for (int k = 0; k < 16; ++k) v[k] = acc[k] * r;
    return pack_e2m1(v, 1.0f);
  }
}

// max(v, v of the lane that DPP control CTRL selects), for non-negative v.
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_max(uint32_t v) {
  const uint32_t o = (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, CTRL, 0xF, 0xF, false);
  return v > o ? v : o;
}

// Largest |T| entry of the panel held by this wave, as a float (uniform).
// Non-negative bf16 values order like their 16-bit patterns, so the
// in-lane part is a packed 16-bit max.  Across lanes: quad swaps, half-row
// and row mirrors give every lane its 16-lane row maximum, then the four
// rows are read out to scalar registers.
__device__ __forceinline__ float panel_tmax(const Frag& f) {
  typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
  const uint32_t mask = 0x7FFF7FFFu;
  u16x2 m = __builtin_bit_cast(u16x2, f.t0[0] & mask);
#pragma unroll
  for (int e = 1; e < 4; ++e) m = __builtin_elementwise_max(m, __builtin_bit_cast(u16x2, f.t0[e] & mask));
#pragma unroll
  for (int e = 0; e < 4; ++e) m = __builtin_elementwise_max(m, __builtin_bit_cast(u16x2, f.t1[e] & mask));
  uint32_t r = m.x > m.y ? m.x : m.y;
  r = dpp_max<0xB1>(r);   // quad_perm [1,0,3,2]
  r = dpp_max<0x4E>(r);   // quad_perm [2,3,0,1]
  r = dpp_max<0x141>(r);  // row_half_mirror
  r = dpp_max<0x140>(r);  // row_mirror
  const uint32_t a = __builtin_amdgcn_readlane(r, 0), b = __builtin_amdgcn_readlane(r, 16);
  const uint32_t c = __builtin_amdgcn_readlane(r, 32), d = __builtin_amdgcn_readlane(r, 48);
  const uint32_t ab = a > b ? a : b, cd = c > d ? c : d;
  return __uint_as_float((ab > cd ? ab : cd) << 16);
}

}  // namespace

// ---------------------------------------------------------------- quant kernel
//
// Workgroup: 8 waves and a column of 256 channels (8 panels) over TPW
// consecutive 32-token tiles.  Wave w owns panel w and keeps its T fragment
// in VGPRs.
//
//  1. At entry each wave loads its T fragment, then every thread issues all
//     of its activation loads for the TPW tiles: 2 x 16 B per tile,
//     row-contiguous, so one wave instruction covers 2 rows x 512 B.
//  2. The tiles go to LDS (rows padded to 528 B, so the transposing
//     MFMA-operand reads are free of bank conflicts), then one barrier.
//  3. Each wave contracts and quantizes its panel of every tile.  It writes
//     the codes back in place over the first 16 B of its own panel in each
//     row (only this wave reads those bytes), and the scales into the row's
//     16-byte pad.  Then a second barrier.
//  4. The output leaves as whole rows: 32 rows x 128 B of codes and
//     32 rows x 8..16 B of scales per tile.
//
// One barrier per workgroup for the data, rather than one per tile: a
// barrier makes the whole workgroup wait for its slowest wave's loads, and
// with several workgroups resident per CU one workgroup's wait is covered
// by another's work.
// Rows past M are loaded from row M-1 and not stored.  Channels past K
// are not loaded; they are zero in LDS, and T is zero there too.

constexpr int kQWaves = kPanelsPerTile;  // waves per quant workgroup (one panel each)
constexpr int kPanels = kQWaves;         // panels (32 channels each) per tile
constexpr int kChunks = 4 * kPanels;     // 16-byte chunks per tile row
constexpr int kScaleOff = kPanels * 64;  // scales of a row start here
constexpr int kXRow = kScaleOff + 16;    // LDS bytes per row: the channels, then 16 B of scales

// LDS of one quant workgroup.
template <int TPW>
struct QuantLds {
  uint8_t xs[TPW][32 * kXRow];  // activation tiles; codes and scales in place
  float y[kQWaves][32];         // exact-recompute exchange, per wave
  uint32_t red[4][kQWaves];     // AbsMax pass: per-wave maxima of its reductions
  float rtab[256];              // NVFP4: fp32(1 / fp32(E4M3(c) g)) for every code c, or 0
};

// Contract and quantize panel `wave` of one staged tile; write its codes and
// scales back into the tile.  `row` is this lane's row of the tile.
//
// The accumulation bound: for MXFP4, whose scale boundaries are powers of
// two, a cheap bound max|T| * (L1 norm) suffices; an all-ones MFMA gives the
// L1 norms (of a token pair, see below); bscale is max|T| * 2^-17.  INT4 and NVFP4 scales have much denser
// boundaries, so they use the per-output bound max_k sum_j |T_kj x_j| from
// an |T| x |x| MFMA, with bscale = 2^-17.
template <int FMT>
__device__ __forceinline__ void panel_step(uint8_t* row, const Frag& f, const u32x4& ones, float bscale, float g,
                                           float k6g, const float* rtab, int wave, int lane, uint32_t& n_exact) {
  constexpr int G = (FMT == kNVFP4) ? 16 : 32;
  const int h = lane >> 5;
  const u32x4 mask = {0x7FFF7FFFu, 0x7FFF7FFFu, 0x7FFF7FFFu, 0x7FFF7FFFu};
  XTile x;
  x.b0 = *reinterpret_cast<const u32x4*>(row + wave * 64 + 16 * h);
  x.b1 = *reinterpret_cast<const u32x4*>(row + wave * 64 + 16 * h + 32);
  f32x16 zero = {};
  f32x16 acc = mfma32(f.t0, x.b0, zero);
  acc = mfma32(f.t1, x.b1, acc);
  float bound;
  if (FMT == kMXFP4) {
    // v_mfma_f32_16x16x32_bf16 on the same operand registers, at half the
    // cost of the 32x32x16 pair.  In its B layout, lane l supplies 8 values
    // of column l % 16 for k-slot l / 16, so column n sums |x| over lanes
    // n, n + 16, n + 32, n + 48: 16 channels of tokens n and n + 16.  With
    // both k-slices accumulated, every output of column n is
    // |x_n|_1 + |x_(n+16)|_1, an upper bound on token n's L1 norm (and on
    // token n + 16's), and lane l reads column l % 16.
    f32x4 z4 = {};
    f32x4 l1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, ones),
                                                       __builtin_bit_cast(bf16x8, x.b0 & mask), z4, 0, 0, 0);
    l1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, ones),
                                                 __builtin_bit_cast(bf16x8, x.b1 & mask), l1, 0, 0, 0);
    bound = l1[0];
  } else {
    f32x16 aab = mfma32(f.a0, x.b0 & mask, zero);
    aab = mfma32(f.a1, x.b1 & mask, aab);
    bound = max16(aab);
    if (G == 32) bound = max_halves(bound);
  }
  uint32_t sbits;
  // LDS address of row 0 of the staged tile at this wave's panel: the exact
  // recompute reads a token's channels there.
  const uint32_t tile = (uint32_t)(uintptr_t)(lds_cu8*)(row - (lane & 31) * kXRow + wave * 64);
  const u32x2 w = quantize_panel<FMT>(acc, bound, bscale, f, tile, kXRow, g, k6g, rtab, lane, sbits, n_exact);
  // Every lane of the wave has read its operands before any lane writes:
  // the reads above feed the MFMAs whose results the writes depend on.
  *reinterpret_cast<u32x2*>(row + wave * 64 + 8 * h) = w;
  if (FMT == kMXFP4) {
    if (h == 0) row[kScaleOff + wave] = (uint8_t)sbits;
  } else if (FMT == kINT4) {
    if (h == 0) *reinterpret_cast<uint16_t*>(row + kScaleOff + 2 * wave) = (uint16_t)sbits;
  } else {
    row[kScaleOff + 2 * wave + h] = (uint8_t)sbits;
  }
}

// Largest value of a non-negative float over the workgroup: wave maximum,
// then one LDS slot per wave.  Every thread gets the result.  Non-negative
// floats order like their bit patterns.  block_max3_nonneg does three at
// once, behind one barrier.
__device__ __forceinline__ float block_max_nonneg(float v, uint32_t* slots, int wave, int lane) {
  uint32_t b = __float_as_uint(v);
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    const uint32_t w = (uint32_t)__shfl_xor((int)b, o, 64);
    b = b > w ? b : w;
  }
  if (lane == 0) slots[wave] = b;
  __syncthreads();
  uint32_t r = slots[0];
#pragma unroll
  for (int i = 1; i < kQWaves; ++i) r = r > slots[i] ? r : slots[i];
  return __uint_as_float(r);
}

__device__ __forceinline__ uint32_t wave_max_bits(uint32_t b) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    const uint32_t w = (uint32_t)__shfl_xor((int)b, o, 64);
    b = b > w ? b : w;
  }
  return b;
}

__device__ __forceinline__ void block_max3_nonneg(float& v0, float& v1, float& v2, uint32_t (*slots)[kQWaves], int wave,
                                                  int lane) {
  const uint32_t b0 = wave_max_bits(__float_as_uint(v0));
  const uint32_t b1 = wave_max_bits(__float_as_uint(v1));
  const uint32_t b2 = wave_max_bits(__float_as_uint(v2));
  if (lane == 0) {
    slots[0][wave] = b0;
    slots[1][wave] = b1;
    slots[2][wave] = b2;
  }
  __syncthreads();
  uint32_t r0 = slots[0][0], r1 = slots[1][0], r2 = slots[2][0];
#pragma unroll
  for (int i = 1; i < kQWaves; ++i) {
    r0 = r0 > slots[0][i] ? r0 : slots[0][i];
    r1 = r1 > slots[1][i] ? r1 : slots[1][i];
    r2 = r2 > slots[2][i] ? r2 : slots[2][i];
  }
  v0 = __uint_as_float(r0);
  v1 = __uint_as_float(r1);
  v2 = __uint_as_float(r2);
}

// The exact max |y| over one run of staged tiles (the per-tensor AbsMax
// behind NVFP4's global scale), folded into *a.amax_bits.
//
// Pass 1 bounds every output: with A_k = sum_j |T_kj x_j| (an |T| x |x|
// MFMA), the fp32 matrix-core value differs from the exactly rounded y_k
// by at most d_k = 2^-17 A_k + 2^-21 |y^_k| (+ 2^-120 for flushed
// products), the bound the quantizer's scale guard uses.  Each lane keeps
// a lower bound on the largest |y| it holds, amax - D with D the largest
// d_k of the lane; the workgroup's largest lower bound `lo` is then a
// lower bound on the run's exact maximum.
// Pass 2 revisits only the tiles where some output's upper bound |y^_k| +
// d_k reaches lo.  Those outputs are the only ones that can hold the
// maximum; the tokens that own them are recomputed in float64 and rounded
// once to fp32 (exact_panel), and the maximum over the recomputed values is
// the run's exact maximum.  Outputs with A_k = 0 are exactly zero.
template <int FMT, int TPW, bool FULL>
__device__ __forceinline__ void amax_run(const QuantArgs& a, QuantLds<TPW>& L, Frag f, bool panel_ok, int n_tiles,
                                         int wave, int lane) {
  const u32x4 mask = {0x7FFF7FFFu, 0x7FFF7FFFu, 0x7FFF7FFFu, 0x7FFF7FFFu};
  with_abs(f);
  const int h = lane >> 5;
  float lo = 0.0f;
  float hi_t[TPW];
#pragma unroll
  for (int u = 0; u < TPW; ++u) hi_t[u] = -1.0f;
  if (panel_ok) {
    const uint8_t* row = L.xs[0] + (lane & 31) * kXRow + wave * 64 + 16 * h;
#pragma unroll
    for (int u = 0; u < TPW; ++u) {
      if (!FULL && u >= n_tiles) break;
      const u32x4 b0 = *reinterpret_cast<const u32x4*>(row + u * (32 * kXRow));
      const u32x4 b1 = *reinterpret_cast<const u32x4*>(row + u * (32 * kXRow) + 32);
      const f32x16 zero = {};
      f32x16 acc = mfma32(f.t0, b0, zero);
      acc = mfma32(f.t1, b1, acc);
      f32x16 aab = mfma32(f.a0, b0 & mask, zero);
      aab = mfma32(f.a1, b1 & mask, aab);
      const float am = max_abs16(acc);
      const float bnd = max16(aab);
      const float d = err_bound(bnd, 0x1p-17f, am);
      lo = fmaxf(lo, am - d);
      hi_t[u] = am + d;
    }
  }
  // The workgroup's largest lower bound, its largest upper bound, and the
  // largest exact maximum any workgroup has published so far (a relaxed
  // read; the stored value only grows).  If even the upper bound is below
  // a published maximum, nothing here can be the tensor's: stop.  The three
  // are reduced together, so every thread takes the same decision.
  float hi = 0.0f;
#pragma unroll
  for (int u = 0; u < TPW; ++u) hi = fmaxf(hi, hi_t[u]);
  float lo_wg = lo, hi_wg = hi;
  float cur = __uint_as_float(__hip_atomic_load(a.amax_bits, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
  block_max3_nonneg(lo_wg, hi_wg, cur, L.red, wave, lane);
  if (hi_wg < cur) return;

  float m = 0.0f;
  if (panel_ok) {
    const uint8_t* row = L.xs[0] + (lane & 31) * kXRow + wave * 64 + 16 * h;
#pragma unroll
    for (int u = 0; u < TPW; ++u) {
      if (!FULL && u >= n_tiles) break;
      if (!__ballot(hi_t[u] >= lo_wg)) continue;
      const u32x4 b0 = *reinterpret_cast<const u32x4*>(row + u * (32 * kXRow));
      const u32x4 b1 = *reinterpret_cast<const u32x4*>(row + u * (32 * kXRow) + 32);
      const f32x16 zero = {};
      f32x16 acc = mfma32(f.t0, b0, zero);
      acc = mfma32(f.t1, b1, acc);
      f32x16 aab = mfma32(f.a0, b0 & mask, zero);
      aab = mfma32(f.a1, b1 & mask, aab);
      bool cand = false;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float ak = fabsf(acc[r]);
        cand |= aab[r] > 0.0f && ak + err_bound(aab[r], 0x1p-17f, ak) >= lo_wg;
      }
      const uint64_t c = __ballot(cand);
      const uint32_t tokens = (uint32_t)c | (uint32_t)(c >> 32);  // token n: lane n or n + 32
      const uint32_t tile = (uint32_t)(uintptr_t)(lds_cu8*)(L.xs[u] + wave * 64);
      uint32_t pend = tokens;
      while (pend) {
        const int n = __builtin_ctz(pend);
        exact_panel(tile + n * kXRow, f, acc, L.y[wave], n, lane);
        pend &= pend - 1;
      }
      if ((tokens >> (lane & 31)) & 1u) m = fmaxf(m, max_abs16(acc));
    }
  }
  const float m_wg = block_max_nonneg(m, L.red[3], wave, lane);
  if (threadIdx.x == 0 && m_wg > 0.0f) {
    const uint32_t w = __float_as_uint(m_wg);
    // The stored value only grows, so a stale read just costs an atomic.
    if (w > __hip_atomic_load(a.amax_bits, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) atomicMax(a.amax_bits, w);
  }
}

// FULL: every row of the run is below M, K is a multiple of 256 and at most
// 2^26, so every tile is complete, every scale row segment is 8- or 16-byte
// aligned, and per-lane offsets fit in 32 bits.  Addresses are then a
// uniform per-tile base (scalar registers) plus a per-lane offset.
//
// AMAX: the same run computes only max |y| over its tiles (the NVFP4
// per-tensor AbsMax pre-pass) and folds it into *a.amax_bits.  Rows past M
// repeat row M - 1 and channels past K are zero on both sides, so they
// change no maximum.
template <int FMT, int TPW, bool FULL, bool AMAX = false, bool PACK = false>
__device__ __forceinline__ void quant_run(const QuantArgs& a, QuantLds<TPW>& L, int cg, int tg) {
  constexpr int G = (FMT == kNVFP4) ? 16 : 32;
  const int tid = threadIdx.x;
  const int lane = lane_id();
  const int wave = tid >> 6;
  const int64_t K = a.K, M = a.M;
  const int C = (int)(K / G);
  const int p0 = cg * kPanels;
  const int n_panels = FULL ? kPanels : ((a.n_panels - p0 < kPanels) ? a.n_panels - p0 : kPanels);
  const int64_t tile0 = (int64_t)tg * TPW;
  const int n_tiles = FULL ? TPW : (int)((a.n_tiles - tile0 < TPW) ? a.n_tiles - tile0 : TPW);

  // 1. T fragment first, then every activation load of the run.  The
  // memory counter retires in order, so the wave can use T while the
  // activations are still in flight.
  const bool panel_ok = wave < n_panels;
  Frag f;
  {
    const u32x4 z = {0u, 0u, 0u, 0u};
    f = panel_ok ? load_t<G>(a.T, p0 + wave, C, lane) : Frag{z, z, z, z};
  }
  // Thread t covers 16-byte chunk t%32 of rows t/32 and t/32 + 16 of each tile.
  const int chunk = tid % kChunks;
  const int row_a = tid / kChunks;  // 0..15
  const int64_t ch0 = (int64_t)p0 * 32 + 8 * chunk;
  const bool chunk_ok = FULL || ch0 < K;
  u32x4 v[TPW][2];
#pragma unroll
  for (int u = 0; u < TPW; ++u) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      if (FULL) {
        const uint16_t* base = a.X + (tile0 + u) * 32 * K + (int64_t)p0 * 32;  // uniform
        v[u][i] = load16_nt(base + (uint32_t)((row_a + 16 * i) * K + 8 * chunk));
      } else {
        const int64_t m = (tile0 + u) * 32 + row_a + 16 * i;
        const int64_t mc = m < M ? m : M - 1;
        const u32x4 z = {0u, 0u, 0u, 0u};
        v[u][i] = (chunk_ok && u < n_tiles) ? load16_nt(a.X + mc * K + ch0) : z;
      }
    }
  }
  const float bscale = (FMT == kMXFP4) ? panel_tmax(f) * 0x1p-17f : 0x1p-17f;
  if (FMT != kMXFP4) with_abs(f);  // |T| once per run, for the per-output bound
  u32x4 ones = {0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};  // bf16 1.0
  asm volatile("" : "+v"(ones));  // materialized once, kept in VGPRs
  float g = 0.0f;
  float k6g = 0.0f;
  if (FMT == kNVFP4 && !AMAX) {
    g = *a.global_scale;
    // The decision's ratio factor, and the reciprocals the codes are scaled
    // by: one IEEE division per thread here instead of one per lane and panel.
    k6g = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(g > 0.0f ? 1.0f / (6.0f * g) : 0.0f)));
    if (tid < 256) {
      const float eff = e4m3_value((uint32_t)tid) * g;
      L.rtab[tid] = (g > 0.0f && eff > 0.0f) ? 1.0f / eff : 0.0f;
    }
  }

  // 2. stage, in arrival order
#pragma unroll
  for (int u = 0; u < TPW; ++u) {
    *reinterpret_cast<u32x4*>(L.xs[u] + row_a * kXRow + 16 * chunk) = v[u][0];
    *reinterpret_cast<u32x4*>(L.xs[u] + (row_a + 16) * kXRow + 16 * chunk) = v[u][1];
  }
  __syncthreads();

  if (AMAX) {
    amax_run<FMT, TPW, FULL>(a, L, f, panel_ok, n_tiles, wave, lane);
    return;
  }

  // 3. contract and quantize
  uint32_t n_exact = 0;
  if (panel_ok) {
    uint8_t* row = L.xs[0] + (lane & 31) * kXRow;  // this lane's row; tiles at constant offsets
#pragma unroll
    for (int u = 0; u < TPW; ++u) {
      if (!FULL && u >= n_tiles) break;
      panel_step<FMT>(row + u * (32 * kXRow), f, ones, bscale, g, k6g, L.rtab, wave, lane, n_exact);
    }
  }
  __syncthreads();

  // 4. whole-row stores: thread t < 32 * kPanels stores 16 B of codes
  // (row t / kPanels, panel t % kPanels); the next 32 threads store one
  // row's scales each.
  const int s_elem = (FMT == kINT4) ? 2 : 1;
  const int64_t s_first = (G == 32) ? p0 : 2 * p0;  // first scale index of the tile in a row
  const int s_max = (G == 32) ? kPanels : 2 * kPanels;
  const int s_count = FULL ? s_max : (int)(((int64_t)C - s_first) < s_max ? (int64_t)C - s_first : s_max);
  const int64_t code_bytes_left = K / 2 - (int64_t)p0 * 16;
  const int code_row_bytes = FULL ? kPanels * 16 : (int)(code_bytes_left < kPanels * 16 ? code_bytes_left : kPanels * 16);
  constexpr int kCodeThreads = 32 * kPanels;
  const int c_row = tid / kPanels, c_panel = tid % kPanels;
  if constexpr (PACK) {
    // The MXFP4 GEMM's operand layout (wush_quant_mxfp4_packed): per
    // 128-row tile and 256-element K step (this workgroup's column), 16 KB
    // of codes in the order the GEMM kernel stages them (row r's 16-byte
    // chunk c at 1024 (r / 8) + 16 (8 (r % 8) + (c ^ ((r / 2) % 8)))) and
    // 1 KB of scales (row r at 8 r).  A tile's 32 rows are 4 KB and 256 B
    // of contiguous whole lines.  K is a multiple of 256 here.
    const int64_t nk = K / 256, ks = p0 / kPanels;
#pragma unroll
    for (int u = 0; u < TPW; ++u) {
      if (!FULL && u >= n_tiles) break;
      const int64_t m_t = (tile0 + u) * 32;  // first row of the tile
      const int r0 = (int)(m_t % 128);
      const uint8_t* xs = L.xs[u];
      if (tid < kCodeThreads) {
        const int r = r0 + c_row;
        if (FULL || m_t + c_row < M) {
          uint8_t* dst = a.codes + ((m_t / 128) * nk + ks) * 16384 + 1024 * (r >> 3) +
                         16 * (8 * (r & 7) + (c_panel ^ ((r >> 1) & 7)));
          *reinterpret_cast<u32x4*>(dst) = *reinterpret_cast<const u32x4*>(xs + c_row * kXRow + 64 * c_panel);
        }
      } else if (tid < kCodeThreads + 32) {
        const int rl = tid - kCodeThreads;
        if (FULL || m_t + rl < M) {
          uint8_t* dst = a.scales + ((m_t / 128) * nk + ks) * 1024 + 8 * (r0 + rl);
          *reinterpret_cast<u32x2*>(dst) = *reinterpret_cast<const u32x2*>(xs + rl * kXRow + kScaleOff);
        }
      }
    }
    if (a.n_exact && n_exact && lane == 0) atomicAdd(a.n_exact, n_exact);
    return;
  }
#pragma unroll
  for (int u = 0; u < TPW; ++u) {
    if (!FULL && u >= n_tiles) break;
    const int64_t t = tile0 + u;
    const uint8_t* xs = L.xs[u];
    if (FULL) {
      if (tid < kCodeThreads) {
        uint8_t* base = a.codes + (t * 32) * (K / 2) + (int64_t)p0 * 16;  // uniform
        const uint32_t off = (uint32_t)(c_row * (K / 2) + 16 * c_panel);
        *reinterpret_cast<u32x4*>(base + off) = *reinterpret_cast<const u32x4*>(xs + c_row * kXRow + 64 * c_panel);
      } else if (tid < kCodeThreads + 32) {
        const int r = tid - kCodeThreads;
        uint8_t* base = a.scales + ((t * 32) * C + s_first) * s_elem;  // uniform
        const uint32_t off = (uint32_t)(r * C * s_elem);
        const uint8_t* src = xs + r * kXRow + kScaleOff;
        if (s_max * s_elem == 4)
          *reinterpret_cast<uint32_t*>(base + off) = *reinterpret_cast<const uint32_t*>(src);
        else if (s_max * s_elem == 8)
          *reinterpret_cast<u32x2*>(base + off) = *reinterpret_cast<const u32x2*>(src);
        else
          *reinterpret_cast<u32x4*>(base + off) = *reinterpret_cast<const u32x4*>(src);
      }
    } else {
      if (tid < kCodeThreads) {
        const int64_t m = t * 32 + c_row;
        if (m < M && 16 * c_panel < code_row_bytes) {
          uint8_t* dst = a.codes + m * (K / 2) + (int64_t)p0 * 16 + 16 * c_panel;
          const u32x4 cv = *reinterpret_cast<const u32x4*>(xs + c_row * kXRow + 64 * c_panel);
          if (16 * c_panel + 16 <= code_row_bytes) {
            *reinterpret_cast<u32x4*>(dst) = cv;
          } else {  // a G=16 row ending half-way into the last panel
            u32x2 h8 = {cv[0], cv[1]};
            *reinterpret_cast<u32x2*>(dst) = h8;
          }
        }
      } else if (tid < kCodeThreads + 32) {
        const int r = tid - kCodeThreads;
        const int64_t m = t * 32 + r;
        if (m < M) {
          uint8_t* dst = a.scales + (m * C + s_first) * s_elem;
          const uint8_t* src = xs + r * kXRow + kScaleOff;
          const int nb = s_count * s_elem;
          for (int b = 0; b < nb; ++b) dst[b] = src[b];
        }
      }
    }
  }
  if (a.n_exact && n_exact && lane == 0) atomicAdd(a.n_exact, n_exact);
}

// 8 waves per SIMD (at most 64 VGPRs): with 35 KB of LDS per two-tile
// workgroup, four workgroups then share a CU.  Without the bound NVFP4 and
// INT4 took 68-70 VGPRs, which left room for three; four measured 6.6%
// faster on the 16384x4096 NVFP4 workload.  At this bound the NVFP4 edge
// path (quant_run<.., false>) keeps one register in scratch; the full-tile
// path spills nothing.  Three-tile runs (51 KB) fit three workgroups per CU
// by their LDS alone, so they ask for 6 waves per SIMD.
template <int FMT, int TPW, bool PACK = false>
__global__ __launch_bounds__(kQWaves * 64, TPW == 3 ? 6 : 8) void quant_kernel(QuantArgs a) {
  __shared__ __attribute__((aligned(16))) QuantLds<TPW> L;
  int cg, tg;
  wg_coords(a.n_pg, a.n_tg, a.token_major, cg, tg);
  const bool full = ((int64_t)(tg + 1) * TPW * 32 <= a.M) && (a.K % (kPanels * 32) == 0) && a.K <= (1 << 26);
  if (full) quant_run<FMT, TPW, true, false, PACK>(a, L, cg, tg);
  else quant_run<FMT, TPW, false, false, PACK>(a, L, cg, tg);
}

// The tensor AbsMax of the transformed activations (NVFP4's per-tensor
// scale), in the quant kernel's run structure: FMT kMXFP4 for G = 32,
// kNVFP4 for G = 16.
template <int FMT, int TPW>
__global__ __launch_bounds__(kQWaves * 64) void absmax_kernel(QuantArgs a) {
  __shared__ __attribute__((aligned(16))) QuantLds<TPW> L;
  int cg, tg;
  wg_coords(a.n_pg, a.n_tg, a.token_major, cg, tg);
  const bool full = ((int64_t)(tg + 1) * TPW * 32 <= a.M) && (a.K % (kPanels * 32) == 0) && a.K <= (1 << 26);
  if (full) quant_run<FMT, TPW, true, true>(a, L, cg, tg);
  else quant_run<FMT, TPW, false, true>(a, L, cg, tg);
}

// ---------------------------------------------------------------- transform

template <int G>
__global__ __launch_bounds__(kWaves * 64) void transform_kernel(TransformArgs a) {
  const int lane = lane_id();
  const int wave = threadIdx.x >> 6;
  int pg, tg;
  wg_coords(a.n_pg, a.n_tg, 0, pg, tg);
  const int p = pg * kWaves + wave;
  if (p >= a.n_panels) return;
  const int n = lane & 31, h = lane >> 5;
  const int C = (int)(a.K / G);
  const Frag f = load_t<G>(a.T, p, C, lane);
  const int c_in = 32 * p + 8 * h;
  const int d1 = ((G == 32) || (2 * p + 1 < C)) ? 16 : 0;
  const int out0 = 32 * p + 16 * h;  // first output channel held by this lane
  const bool group_ok = (G == 32) || (2 * p + h < C);
  const int64_t tile0 = (int64_t)tg * a.tiles_per_wave;
  const int64_t tile1 = (tile0 + a.tiles_per_wave < a.n_tiles) ? tile0 + a.tiles_per_wave : a.n_tiles;
  for (int64_t t = tile0; t < tile1; ++t) {
    const int64_t m = t * 32 + n;
    const uint16_t* src = a.X + (m < a.M ? m : a.M - 1) * a.K + c_in;
    XTile x;
    x.b0 = load16_nt(src);
    x.b1 = load16_nt(src + d1);
    f32x16 zero = {};
    f32x16 acc = mfma32(f.t0, x.b0, zero);
    acc = mfma32(f.t1, x.b1, acc);
    if (m >= a.M) continue;
    if (group_ok) {
      f32x4* dst = reinterpret_cast<f32x4*>(a.Y + m * a.K + out0);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        f32x4 v = {acc[4 * q], acc[4 * q + 1], acc[4 * q + 2], acc[4 * q + 3]};
        __builtin_nontemporal_store(v, &dst[q]);
      }
    }
  }
}

__global__ void fill_u32_kernel(uint32_t* p, uint32_t v) { *p = v; }

__global__ void global_scale_kernel(float* out) {
  // out holds the AbsMax bit pattern written by the absmax kernel
  float amax = __uint_as_float(*reinterpret_cast<uint32_t*>(out));
  *out = amax / 2688.0f;
}

// Element i is converted as part of the pair (2*(i/2), 2*(i/2)+1), exactly as
// the quantization kernels convert pairs, and written back one code per byte.
__global__ void e2m1_kernel(const float* __restrict__ v, int64_t n, uint8_t* __restrict__ out) {
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (; 2 * i < n; i += stride) {
    float a = v[2 * i];
    float b = (2 * i + 1 < n) ? v[2 * i + 1] : 0.0f;
    uint32_t w = cvt_e2m1x2<0>(0u, a, b, 1.0f);
    out[2 * i] = (uint8_t)(w & 0xFu);
    if (2 * i + 1 < n) out[2 * i + 1] = (uint8_t)((w >> 4) & 0xFu);
  }
}

// ---------------------------------------------------------------- launchers

template <int FMT, bool PACK = false>
static hipError_t launch_quant_fmt(const QuantArgs& a, int n_wg, hipStream_t s) {
  dim3 grid(n_wg), block(kQWaves * 64);
  switch (a.tiles_per_wave) {
    case 1: hipLaunchKernelGGL((quant_kernel<FMT, 1, PACK>), grid, block, 0, s, a); break;
    case 2: hipLaunchKernelGGL((quant_kernel<FMT, 2, PACK>), grid, block, 0, s, a); break;
    case 3: hipLaunchKernelGGL((quant_kernel<FMT, 3, PACK>), grid, block, 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_quant_mxfp4_packed(const QuantArgs& a, int n_wg, hipStream_t s) {
  return launch_quant_fmt<kMXFP4, true>(a, n_wg, s);
}

hipError_t launch_quant(int fmt, const QuantArgs& a, int n_wg, hipStream_t s) {
  switch (fmt) {
    case kMXFP4: return launch_quant_fmt<kMXFP4>(a, n_wg, s);
    case kNVFP4: return launch_quant_fmt<kNVFP4>(a, n_wg, s);
    case kINT4: return launch_quant_fmt<kINT4>(a, n_wg, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_transform(int G, const TransformArgs& a, int n_wg, hipStream_t s) {
  dim3 grid(n_wg), block(kWaves * 64);
  if (G == 32) hipLaunchKernelGGL((transform_kernel<32>), grid, block, 0, s, a);
  else hipLaunchKernelGGL((transform_kernel<16>), grid, block, 0, s, a);
  return hipGetLastError();
}

template <int FMT>
static void launch_absmax_fmt(const QuantArgs& a, int n_wg, hipStream_t s) {
  dim3 grid(n_wg), block(kQWaves * 64);
  switch (a.tiles_per_wave) {
    case 1: hipLaunchKernelGGL((absmax_kernel<FMT, 1>), grid, block, 0, s, a); break;
    case 2: hipLaunchKernelGGL((absmax_kernel<FMT, 2>), grid, block, 0, s, a); break;
    default: hipLaunchKernelGGL((absmax_kernel<FMT, 3>), grid, block, 0, s, a); break;
  }
}

hipError_t launch_absmax(int G, const QuantArgs& a, int n_wg, hipStream_t s) {
  if (a.tiles_per_wave < 1 || a.tiles_per_wave > 3) return hipErrorInvalidValue;
  hipLaunchKernelGGL(fill_u32_kernel, dim3(1), dim3(1), 0, s, a.amax_bits, 0u);
  if (n_wg == 0) return hipGetLastError();
  if (G == 32) launch_absmax_fmt<kMXFP4>(a, n_wg, s);
  else launch_absmax_fmt<kNVFP4>(a, n_wg, s);
  return hipGetLastError();
}

hipError_t launch_global_scale(float* out, hipStream_t s) {
  hipLaunchKernelGGL(global_scale_kernel, dim3(1), dim3(1), 0, s, out);
  return hipGetLastError();
}

hipError_t launch_e2m1(const float* v, int64_t n, uint8_t* out, hipStream_t s) {
  int64_t blocks = (n / 2 + 256) / 256;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(e2m1_kernel, dim3((unsigned)blocks), dim3(256), 0, s, v, n, out);
  return hipGetLastError();
}

}  // namespace wush
