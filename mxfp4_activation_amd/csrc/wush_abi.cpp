// C-ABI layer of the WUSH online path.  It validates arguments, checks the
// device, picks the launch shape and forwards to the kernels.
// Contract: include/wush.h.

#include <stdarg.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include <atomic>

#include <hip/hip_runtime.h>

#include "../../include/wush.h"
#include "wush_build.h"
#include "wush_dequant.h"
#include "wush_gemm.h"
#include "wush_gptq.h"
#include "wush_kernels.h"

namespace {

thread_local char g_last_error[512] = "";

wush_status fail(wush_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return st;
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Half-open byte ranges [p, p + n) overlap?
bool overlap(const void* p, uint64_t np, const void* q, uint64_t nq) {
  if (!p || !q || np == 0 || nq == 0) return false;
  uintptr_t a = reinterpret_cast<uintptr_t>(p), b = reinterpret_cast<uintptr_t>(q);
  return a < b + nq && b < a + np;
}

// Per-device "is gfx950" cache: 0 unknown, 1 yes, 2 no.
constexpr int kMaxDevices = 64;
std::atomic<int> g_dev_ok[kMaxDevices];

wush_status check_device() {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(WUSH_EHIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(WUSH_EUNSUPPORTED, "device index %d out of range", dev);
  int st = g_dev_ok[dev].load(std::memory_order_relaxed);
  if (st == 0) {
    hipDeviceProp_t prop;
    e = hipGetDeviceProperties(&prop, dev);
    if (e != hipSuccess) return fail(WUSH_EHIP, "hipGetDeviceProperties: %s", hipGetErrorString(e));
    st = (strncmp(prop.gcnArchName, "gfx950", 6) == 0) ? 1 : 2;
    g_dev_ok[dev].store(st, std::memory_order_relaxed);
  }
  if (st != 1) return fail(WUSH_EUNSUPPORTED, "device %d is not gfx950", dev);
  return WUSH_OK;
}

// Shape checks common to every entry point that reads X and T.
wush_status check_shape(const void* X, const void* T, int64_t M, int64_t K, int G) {
  if (G != 16 && G != 32) return fail(WUSH_EUNSUPPORTED, "G must be 16 or 32 (got %d)", G);
  if (M < 0) return fail(WUSH_EINVAL, "M must be >= 0 (got %lld)", (long long)M);
  if (K <= 0 || K % G != 0) return fail(WUSH_EINVAL, "K must be a positive multiple of %d (got %lld)", G, (long long)K);
  if (K > (int64_t)1 << 30) return fail(WUSH_EINVAL, "K too large (%lld)", (long long)K);
  if (M > (INT64_MAX / 4) / K) return fail(WUSH_EINVAL, "M*K overflows");
  if (M == 0) return WUSH_OK;
  if (!X || !T) return fail(WUSH_EINVAL, "null X or T");
  if (!aligned(X, 16) || !aligned(T, 16)) return fail(WUSH_EALIGN, "X and T must be 16-byte aligned");
  return WUSH_OK;
}

// Work split: each wave owns one 32-channel panel and walks a run of
// 32-token tiles.  Runs are sized so that the grid holds at least ~4
// workgroups per CU when the problem allows, and a wave reuses its T
// fragment over up to 8 tiles.
void plan(int64_t M, int64_t K, int64_t* n_tiles, int64_t* tpw, int* n_panels, int* n_pg, int* n_tg) {
  *n_tiles = (M + 31) / 32;
  *n_panels = (int)((K + 31) / 32);
  *n_pg = (*n_panels + wush::kWavesPerGroup - 1) / wush::kWavesPerGroup;
  const int64_t target_wg = 1024;  // 256 CUs x 4
  int64_t t = 8;
  while (t > 1 && (int64_t)(*n_pg) * ((*n_tiles + t - 1) / t) < target_wg) t >>= 1;
  *tpw = t;
  *n_tg = (int)((*n_tiles + t - 1) / t);
}

// Quant kernel split: a workgroup (8 waves) owns a 256-channel column of
// the input and a run of TPW 32-token tiles, all loaded at entry.  TPW is
// the longest run up to a per-format cap that still gives at least 1024
// workgroups, so that several workgroups share each CU and cover each
// other's waits.  Two-tile runs fit four workgroups per CU, three-tile runs
// three.  The caps, measured:
// - MXFP4: 3.  On 8192 x 14336, three-tile runs measured 2.6% faster than
//   two.  4096 x 4096 keeps two-tile runs, since three would leave fewer
//   than 1024 workgroups; forced, they measured 10% slower there.
// - NVFP4: 2.  Three-tile runs measured 1-2% slower on 16384 x 4096.
// - INT4: 3.  It does twice the vector work per tile and is compute-bound;
//   three-tile runs (with the exact recompute reading LDS) measured 10%
//   faster than four-tile runs, and four faster than two.
// WUSH_TILES_PER_WG (1, 2 or 3) overrides the choice for tuning.
//
// The workgroup order is panel-major while the whole grid fits on the chip
// at once (256 CUs x 4 workgroups, or x 3 for three-tile runs), and
// token-major beyond that.  On 8192 x 14336 MXFP4 (seven waves of
// workgroups) token-major measured 2.4% faster; on 4096 x 4096 (one wave)
// it measured 1% slower; on the NVFP4 and INT4 batches the two tie.
void plan_quant(int fmt, int64_t M, int64_t K, wush::QuantArgs& a) {
  a.n_tiles = (M + 31) / 32;
  a.n_panels = (int)((K + 31) / 32);
  a.n_pg = (a.n_panels + wush::kPanelsPerTile - 1) / wush::kPanelsPerTile;
  const int64_t target_wg = 8192 / wush::kPanelsPerTile;  // 1024 eight-wave workgroups
  int64_t t = fmt == wush::kNVFP4 ? 2 : 3;
  while (t > 1 && (int64_t)a.n_pg * ((a.n_tiles + t - 1) / t) < target_wg) --t;
  static const int64_t env = [] {
    const char* s = getenv("WUSH_TILES_PER_WG");
    return s ? (int64_t)atoll(s) : (int64_t)0;
  }();
  if (env >= 1 && env <= 3) t = env;
  a.tiles_per_wave = t;
  a.n_tg = (int)((a.n_tiles + t - 1) / t);
  const int64_t resident = 256 * (t == 3 ? 3 : 4);
  a.token_major = (int64_t)a.n_pg * a.n_tg > resident ? 1 : 0;
}

int64_t env_tpw() {
  static int64_t v = [] {
    const char* s = getenv("WUSH_TILES_PER_WAVE");
    return s ? (int64_t)atoll(s) : (int64_t)0;
  }();
  return v;
}

}  // namespace

extern "C" {

const char* wush_status_string(wush_status s) {
  switch (s) {
    case WUSH_OK: return "ok";
    case WUSH_EINVAL: return "invalid argument";
    case WUSH_EALIGN: return "misaligned pointer";
    case WUSH_EUNSUPPORTED: return "unsupported device or parameter";
    case WUSH_EHIP: return "HIP runtime error";
  }
  return "unknown status";
}

const char* wush_last_error(void) { return g_last_error; }

int wush_abi_version(void) { return WUSH_ABI_VERSION; }

wush_status wush_quant(int fmt, const void* X, const void* T, int64_t M, int64_t K,
                       const float* global_scale, void* codes, void* scales, uint32_t* n_exact,
                       hipStream_t stream) {
  g_last_error[0] = 0;
  if (fmt != wush::kMXFP4 && fmt != wush::kNVFP4 && fmt != wush::kINT4)
    return fail(WUSH_EUNSUPPORTED, "unknown format %d", fmt);
  const int G = (fmt == wush::kNVFP4) ? 16 : 32;
  wush_status st = check_shape(X, T, M, K, G);
  if (st != WUSH_OK || M == 0) return st;
  if (!codes || !scales) return fail(WUSH_EINVAL, "null codes or scales");
  if (fmt == wush::kNVFP4 && !global_scale) return fail(WUSH_EINVAL, "NVFP4 needs global_scale");
  // The kernels store codes in 16-byte vectors and each row's scales in
  // 8-byte (MXFP4) or 16-byte (NVFP4, INT4) vectors.
  if (!aligned(codes, 16)) return fail(WUSH_EALIGN, "codes must be 16-byte aligned");
  const int scale_bytes = (fmt == wush::kINT4) ? 2 : 1;
  const int scale_align = (fmt == wush::kMXFP4) ? 8 : 16;
  if (!aligned(scales, scale_align)) return fail(WUSH_EALIGN, "scales must be %d-byte aligned", scale_align);
  if (global_scale && fmt == wush::kNVFP4 && !aligned(global_scale, 4))
    return fail(WUSH_EALIGN, "global_scale must be 4-byte aligned");
  if (n_exact && !aligned(n_exact, 4)) return fail(WUSH_EALIGN, "n_exact must be 4-byte aligned");
  const uint64_t nx = (uint64_t)M * K * 2, nt = (uint64_t)K * G * 2;
  const uint64_t nc = (uint64_t)M * K / 2, ns = (uint64_t)M * (K / G) * scale_bytes;
  if (overlap(codes, nc, X, nx) || overlap(codes, nc, T, nt) || overlap(scales, ns, X, nx) ||
      overlap(scales, ns, T, nt) || overlap(codes, nc, scales, ns))
    return fail(WUSH_EINVAL, "output buffers overlap inputs or each other");
  st = check_device();
  if (st != WUSH_OK) return st;

  wush::QuantArgs a{};
  a.X = static_cast<const uint16_t*>(X);
  a.T = static_cast<const uint16_t*>(T);
  a.codes = static_cast<uint8_t*>(codes);
  a.scales = static_cast<uint8_t*>(scales);
  a.global_scale = global_scale;
  a.n_exact = n_exact;
  a.M = M;
  a.K = K;
  plan_quant(fmt, M, K, a);
  const int64_t n_wg = (int64_t)a.n_pg * a.n_tg;
  if (n_wg > 0x7FFFFFFF) return fail(WUSH_EINVAL, "problem too large for one launch");
  hipError_t e = wush::launch_quant(fmt, a, (int)n_wg, stream);
  if (e != hipSuccess) return fail(WUSH_EHIP, "launch: %s", hipGetErrorString(e));
  return WUSH_OK;
}

wush_status wush_quant_mxfp4(const void* X, const void* T, int64_t M, int64_t K, void* codes,
                             void* scales, hipStream_t stream) {
  return wush_quant(wush::kMXFP4, X, T, M, K, nullptr, codes, scales, nullptr, stream);
}

wush_status wush_quant_mxfp4_packed(const void* X, const void* T, int64_t M, int64_t K, void* packed_codes,
                                    void* packed_scales, hipStream_t stream) {
  g_last_error[0] = 0;
  wush_status st = check_shape(X, T, M, K, 32);
  if (st != WUSH_OK || M == 0) return st;
  if (K % 256 != 0) return fail(WUSH_EINVAL, "K must be a multiple of 256 for the packed layout (got %lld)", (long long)K);
  if (!packed_codes || !packed_scales) return fail(WUSH_EINVAL, "null codes or scales");
  if (!aligned(packed_codes, 16)) return fail(WUSH_EALIGN, "codes must be 16-byte aligned");
  if (!aligned(packed_scales, 8)) return fail(WUSH_EALIGN, "scales must be 8-byte aligned");
  const int64_t Mp = (M + 127) / 128 * 128;
  const uint64_t nx = (uint64_t)M * K * 2, nt = (uint64_t)K * 32 * 2;
  const uint64_t nc = (uint64_t)Mp * K / 2, ns = (uint64_t)Mp * K / 32;
  if (overlap(packed_codes, nc, X, nx) || overlap(packed_codes, nc, T, nt) || overlap(packed_scales, ns, X, nx) ||
      overlap(packed_scales, ns, T, nt) || overlap(packed_codes, nc, packed_scales, ns))
    return fail(WUSH_EINVAL, "output buffers overlap inputs or each other");
  st = check_device();
  if (st != WUSH_OK) return st;
  wush::QuantArgs a{};
  a.X = static_cast<const uint16_t*>(X);
  a.T = static_cast<const uint16_t*>(T);
  a.codes = static_cast<uint8_t*>(packed_codes);
  a.scales = static_cast<uint8_t*>(packed_scales);
  a.M = M;
  a.K = K;
  plan_quant(wush::kMXFP4, M, K, a);
  const int64_t n_wg = (int64_t)a.n_pg * a.n_tg;
  if (n_wg > 0x7FFFFFFF) return fail(WUSH_EINVAL, "problem too large for one launch");
  hipError_t e = wush::launch_quant_mxfp4_packed(a, (int)n_wg, stream);
  if (e != hipSuccess) return fail(WUSH_EHIP, "launch: %s", hipGetErrorString(e));
  return WUSH_OK;
}

wush_status wush_quant_nvfp4(const void* X, const void* T, int64_t M, int64_t K,
                             const float* global_scale, void* codes, void* scales,
                             hipStream_t stream) {
  return wush_quant(wush::kNVFP4, X, T, M, K, global_scale, codes, scales, nullptr, stream);
}

wush_status wush_quant_int4(const void* X, const void* T, int64_t M, int64_t K, void* codes,
                            void* scales, hipStream_t stream) {
  return wush_quant(wush::kINT4, X, T, M, K, nullptr, codes, scales, nullptr, stream);
}

static wush_status transform_common(const void* X, const void* T, int64_t M, int64_t K, int G,
                                    float* Y, hipStream_t stream) {
  wush::TransformArgs a{};
  a.X = static_cast<const uint16_t*>(X);
  a.T = static_cast<const uint16_t*>(T);
  a.Y = Y;
  a.M = M;
  a.K = K;
  plan(M, K, &a.n_tiles, &a.tiles_per_wave, &a.n_panels, &a.n_pg, &a.n_tg);
  const int64_t n_wg = (int64_t)a.n_pg * a.n_tg;
  if (n_wg > 0x7FFFFFFF) return fail(WUSH_EINVAL, "problem too large for one launch");
  hipError_t e = wush::launch_transform(G, a, (int)n_wg, stream);
  if (e != hipSuccess) return fail(WUSH_EHIP, "launch: %s", hipGetErrorString(e));
  return WUSH_OK;
}

wush_status wush_transform_f32(const void* X, const void* T, int64_t M, int64_t K, int G, float* Y,
                               hipStream_t stream) {
  g_last_error[0] = 0;
  wush_status st = check_shape(X, T, M, K, G);
  if (st != WUSH_OK || M == 0) return st;
  if (!Y) return fail(WUSH_EINVAL, "null Y");
  if (!aligned(Y, 16)) return fail(WUSH_EALIGN, "Y must be 16-byte aligned");
  if (overlap(Y, (uint64_t)M * K * 4, X, (uint64_t)M * K * 2) || overlap(Y, (uint64_t)M * K * 4, T, (uint64_t)K * G * 2))
    return fail(WUSH_EINVAL, "Y overlaps an input");
  st = check_device();
  if (st != WUSH_OK) return st;
  return transform_common(X, T, M, K, G, Y, stream);
}

// The AbsMax pre-pass runs the quant kernel's tiling (same planner), so it
// streams X in the same row-contiguous pattern.  M = 0 launches only the
// fill, which writes the empty tensor's AbsMax, 0.
static wush_status absmax_common(const void* X, const void* T, int64_t M, int64_t K, int G, float* out,
                                 hipStream_t stream) {
  wush_status st = check_shape(X, T, M, K, G);
  if (st != WUSH_OK) return st;
  if (!out) return fail(WUSH_EINVAL, "null output");
  if (!aligned(out, 4)) return fail(WUSH_EALIGN, "output must be 4-byte aligned");
  if (M > 0 && (overlap(out, 4, X, (uint64_t)M * K * 2) || overlap(out, 4, T, (uint64_t)K * G * 2)))
    return fail(WUSH_EINVAL, "output overlaps an input");
  st = check_device();
  if (st != WUSH_OK) return st;
  wush::QuantArgs a{};
  a.X = static_cast<const uint16_t*>(X);
  a.T = static_cast<const uint16_t*>(T);
  a.amax_bits = reinterpret_cast<uint32_t*>(out);
  a.M = M;
  a.K = K;
  int64_t n_wg = 0;
  if (M > 0) {
    // The pass does no quantization work, so it takes MXFP4's tile cap
    // for both G: on 16384 x 4096 with G = 16, three-tile runs measured
    // 34.3 against 40.5 us for the two-tile runs NVFP4 quantization uses.
    plan_quant(wush::kMXFP4, M, K, a);
    n_wg = (int64_t)a.n_pg * a.n_tg;
    if (n_wg > 0x7FFFFFFF) return fail(WUSH_EINVAL, "problem too large for one launch");
  } else {
    a.tiles_per_wave = 1;
  }
  hipError_t e = wush::launch_absmax(G, a, (int)n_wg, stream);
  if (e != hipSuccess) return fail(WUSH_EHIP, "launch: %s", hipGetErrorString(e));
  return WUSH_OK;
}

wush_status wush_absmax_transformed(const void* X, const void* T, int64_t M, int64_t K, int G,
                                    float* amax, hipStream_t stream) {
  g_last_error[0] = 0;
  return absmax_common(X, T, M, K, G, amax, stream);
}

wush_status wush_nvfp4_global_scale(const void* X, const void* T, int64_t M, int64_t K,
                                    float* global_scale, hipStream_t stream) {
  g_last_error[0] = 0;
  wush_status st = absmax_common(X, T, M, K, 16, global_scale, stream);
  if (st != WUSH_OK) return st;
  hipError_t e = wush::launch_global_scale(global_scale, stream);
  if (e != hipSuccess) return fail(WUSH_EHIP, "launch: %s", hipGetErrorString(e));
  return WUSH_OK;
}

static wush_status gemm_common(const void* a_codes, const void* a_scales, const void* b_codes, const void* b_scales,
                               int64_t M, int64_t N, int64_t K, void* C, int out_type, int layout,
                               hipStream_t stream) {
  if (out_type != WUSH_OUT_F32 && out_type != WUSH_OUT_BF16) return fail(WUSH_EINVAL, "unknown out_type %d", out_type);
  if (M < 0 || N < 0) return fail(WUSH_EINVAL, "M and N must be >= 0");
  if (K <= 0 || K % 256 != 0) return fail(WUSH_EINVAL, "K must be a positive multiple of 256 (got %lld)", (long long)K);
  if (K > ((int64_t)1 << 30)) return fail(WUSH_EINVAL, "K too large");
  if (M == 0 || N == 0) return WUSH_OK;
  if ((M + 127) / 128 > 65535) return fail(WUSH_EINVAL, "M too large for one launch");
  if ((N + 127) / 128 > 0x7FFFFFFF) return fail(WUSH_EINVAL, "N too large for one launch");
  if (M > (INT64_MAX / 8) / N || M > (INT64_MAX / 8) / K || N > (INT64_MAX / 8) / K)
    return fail(WUSH_EINVAL, "sizes overflow");
  if (!a_codes || !a_scales || !b_codes || !b_scales || !C) return fail(WUSH_EINVAL, "null pointer");
  if (!aligned(a_codes, 16) || !aligned(b_codes, 16)) return fail(WUSH_EALIGN, "codes must be 16-byte aligned");
  if (!aligned(a_scales, 8) || !aligned(b_scales, 8)) return fail(WUSH_EALIGN, "scales must be 8-byte aligned");
  if (!aligned(C, 4)) return fail(WUSH_EALIGN, "C must be 4-byte aligned");
  // Packed B covers N rounded up to a multiple of 128 rows.
  const int64_t nrows_b = layout != wush::kRowMajor ? (N + 127) / 128 * 128 : N;
  const int64_t nrows_a = layout == wush::kPackedAB ? (M + 127) / 128 * 128 : M;
  const uint64_t nc = (uint64_t)M * N * (out_type == WUSH_OUT_F32 ? 4 : 2);
  const uint64_t na = (uint64_t)nrows_a * K / 2, nb = (uint64_t)nrows_b * K / 2;
  const uint64_t nsa = (uint64_t)nrows_a * K / 32, nsb = (uint64_t)nrows_b * K / 32;
  if (overlap(C, nc, a_codes, na) || overlap(C, nc, b_codes, nb) || overlap(C, nc, a_scales, nsa) ||
      overlap(C, nc, b_scales, nsb))
    return fail(WUSH_EINVAL, "C overlaps an input");
  wush_status st = check_device();
  if (st != WUSH_OK) return st;
  wush::GemmArgs g{};
  g.a_codes = static_cast<const uint8_t*>(a_codes);
  g.a_scales = static_cast<const uint8_t*>(a_scales);
  g.b_codes = static_cast<const uint8_t*>(b_codes);
  g.b_scales = static_cast<const uint8_t*>(b_scales);
  g.C = C;
  g.M = M;
  g.N = N;
  g.K = K;
  g.ldc = N;
  hipError_t e = wush::launch_gemm_mxfp4(g, out_type == WUSH_OUT_BF16, layout, stream);
  if (e != hipSuccess) return fail(WUSH_EHIP, "launch: %s", hipGetErrorString(e));
  return WUSH_OK;
}

wush_status wush_gemm_mxfp4(const void* a_codes, const void* a_scales, const void* b_codes,
                            const void* b_scales, int64_t M, int64_t N, int64_t K, void* C, int out_type,
                            hipStream_t stream) {
  g_last_error[0] = 0;
  return gemm_common(a_codes, a_scales, b_codes, b_scales, M, N, K, C, out_type, wush::kRowMajor, stream);
}

wush_status wush_gemm_mxfp4_packed(const void* a_codes, const void* a_scales, int a_packed,
                                   const void* b_packed_codes, const void* b_packed_scales, int64_t M, int64_t N,
                                   int64_t K, void* C, int out_type, hipStream_t stream) {
  g_last_error[0] = 0;
  if (a_packed != 0 && a_packed != 1) return fail(WUSH_EINVAL, "a_packed must be 0 or 1 (got %d)", a_packed);
  return gemm_common(a_codes, a_scales, b_packed_codes, b_packed_scales, M, N, K, C, out_type,
                     a_packed ? wush::kPackedAB : wush::kPackedB, stream);
}

wush_status wush_gemm_pack_b(const void* b_codes, const void* b_scales, int64_t N, int64_t K, void* packed_codes,
                             void* packed_scales, hipStream_t stream) {
  g_last_error[0] = 0;
  if (N < 0) return fail(WUSH_EINVAL, "N must be >= 0");
  if (K <= 0 || K % 256 != 0) return fail(WUSH_EINVAL, "K must be a positive multiple of 256 (got %lld)", (long long)K);
  if (K > ((int64_t)1 << 30)) return fail(WUSH_EINVAL, "K too large");
  if (N == 0) return WUSH_OK;
  const int64_t nr = (N + 127) / 128 * 128;
  if (nr > (INT64_MAX / 8) / K || nr / 128 * (K / 256) * 1024 > 0x7FFFFFFFLL * 256)
    return fail(WUSH_EINVAL, "sizes overflow");
  if (!b_codes || !b_scales || !packed_codes || !packed_scales) return fail(WUSH_EINVAL, "null pointer");
  if (!aligned(b_codes, 16) || !aligned(packed_codes, 16)) return fail(WUSH_EALIGN, "codes must be 16-byte aligned");
  if (!aligned(b_scales, 8) || !aligned(packed_scales, 8)) return fail(WUSH_EALIGN, "scales must be 8-byte aligned");
  const uint64_t nb = (uint64_t)N * K / 2, nsb = (uint64_t)N * K / 32;
  const uint64_t npb = (uint64_t)nr * K / 2, npsb = (uint64_t)nr * K / 32;
  if (overlap(packed_codes, npb, b_codes, nb) || overlap(packed_codes, npb, b_scales, nsb) ||
      overlap(packed_scales, npsb, b_codes, nb) || overlap(packed_scales, npsb, b_scales, nsb) ||
      overlap(packed_codes, npb, packed_scales, npsb))
    return fail(WUSH_EINVAL, "packed outputs overlap an input or each other");
  wush_status st = check_device();
  if (st != WUSH_OK) return st;
  hipError_t e = wush::launch_pack_b(static_cast<const uint8_t*>(b_codes), static_cast<const uint8_t*>(b_scales), N, K,
                                     static_cast<uint8_t*>(packed_codes), static_cast<uint8_t*>(packed_scales), stream);
  if (e != hipSuccess) return fail(WUSH_EHIP, "launch: %s", hipGetErrorString(e));
  return WUSH_OK;
}

wush_status wush_dequant(int fmt, const void* codes, const void* scales, const float* global_scale, int64_t M,
                         int64_t K, float* out, hipStream_t stream) {
  g_last_error[0] = 0;
  if (fmt < 0 || fmt > 2) return fail(WUSH_EUNSUPPORTED, "unknown format %d", fmt);
  const int G = fmt == 1 ? 16 : 32;
  if (M < 0) return fail(WUSH_EINVAL, "M must be >= 0");
  if (K <= 0 || K % G != 0) return fail(WUSH_EINVAL, "K must be a positive multiple of %d (got %lld)", G, (long long)K);
  if (K > ((int64_t)1 << 30) || M > (INT64_MAX / 8) / K) return fail(WUSH_EINVAL, "sizes overflow");
  if (M == 0) return WUSH_OK;
  if ((M * (K / 16) + 255) / 256 > 0x7FFFFFFF) return fail(WUSH_EINVAL, "too large for one launch");
  if (!codes || !scales || !out || (fmt == 1 && !global_scale)) return fail(WUSH_EINVAL, "null pointer");
  if (!aligned(codes, 8)) return fail(WUSH_EALIGN, "codes must be 8-byte aligned");
  if (fmt == 2 && !aligned(scales, 2)) return fail(WUSH_EALIGN, "INT4 scales must be 2-byte aligned");
  if (fmt == 1 && !aligned(global_scale, 4)) return fail(WUSH_EALIGN, "global_scale must be 4-byte aligned");
  if (!aligned(out, 16)) return fail(WUSH_EALIGN, "out must be 16-byte aligned");
  const uint64_t no = (uint64_t)M * K * 4, nc = (uint64_t)M * K / 2, ns = (uint64_t)M * (K / G) * (fmt == 2 ? 2 : 1);
  if (overlap(out, no, codes, nc) || overlap(out, no, scales, ns) || (fmt == 1 && overlap(out, no, global_scale, 4)))
    return fail(WUSH_EINVAL, "out overlaps an input");
  wush_status st = check_device();
  if (st != WUSH_OK) return st;
  hipError_t e = wush::launch_dequant(fmt, static_cast<const uint8_t*>(codes), scales, global_scale, M, K, out, stream);
  if (e != hipSuccess) return fail(WUSH_EHIP, "launch: %s", hipGetErrorString(e));
  return WUSH_OK;
}

wush_status wush_build_transforms(const void* W, int64_t d_out, const void* Xcal, int64_t n_cal, int64_t d_in,
                                  int G, double damp, int use_hadamard, double* T_wush, double* T_xvsh,
                                  void* T_wush_bf16, void* T_xvsh_bf16, hipStream_t stream) {
  g_last_error[0] = 0;
  if (G != 16 && G != 32) return fail(WUSH_EUNSUPPORTED, "G must be 16 or 32 (got %d)", G);
  if (d_out < 1 || n_cal < 1) return fail(WUSH_EINVAL, "d_out and n_cal must be >= 1");
  if (d_in <= 0 || d_in % G != 0) return fail(WUSH_EINVAL, "d_in must be a positive multiple of G");
  if (d_in / G > 0x7FFFFFFF || d_out > (INT64_MAX / 2) / d_in || n_cal > (INT64_MAX / 2) / d_in)
    return fail(WUSH_EINVAL, "sizes overflow");
  if (!(damp >= 0.0)) return fail(WUSH_EINVAL, "damp must be >= 0");
  if (!W || !Xcal || !T_wush || !T_xvsh) return fail(WUSH_EINVAL, "null pointer");
  if (!aligned(W, 16) || !aligned(Xcal, 16)) return fail(WUSH_EALIGN, "W and Xcal must be 16-byte aligned");
  if (!aligned(T_wush, 8) || !aligned(T_xvsh, 8)) return fail(WUSH_EALIGN, "T_wush and T_xvsh must be 8-byte aligned");
  if ((T_wush_bf16 && !aligned(T_wush_bf16, 2)) || (T_xvsh_bf16 && !aligned(T_xvsh_bf16, 2)))
    return fail(WUSH_EALIGN, "bf16 outputs must be 2-byte aligned");
  const uint64_t nt = (uint64_t)d_in * G * 8, nb = (uint64_t)d_in * G * 2;
  const uint64_t nw = (uint64_t)d_out * d_in * 2, nx = (uint64_t)n_cal * d_in * 2;
  const void* outs[4] = {T_wush, T_xvsh, T_wush_bf16, T_xvsh_bf16};
  const uint64_t osz[4] = {nt, nt, nb, nb};
  for (int i = 0; i < 4; ++i) {
    if (!outs[i]) continue;
    if (overlap(outs[i], osz[i], W, nw) || overlap(outs[i], osz[i], Xcal, nx))
      return fail(WUSH_EINVAL, "an output overlaps an input");
    for (int j = 0; j < i; ++j)
      if (outs[j] && overlap(outs[i], osz[i], outs[j], osz[j])) return fail(WUSH_EINVAL, "outputs overlap");
  }
  wush_status st = check_device();
  if (st != WUSH_OK) return st;
  wush::BuildArgs a{};
  a.W = static_cast<const uint16_t*>(W);
  a.X = static_cast<const uint16_t*>(Xcal);
  a.d_out = d_out;
  a.n_cal = n_cal;
  a.d_in = d_in;
  a.damp = damp;
  a.use_hadamard = use_hadamard ? 1 : 0;
  a.T_wush = T_wush;
  a.T_xvsh = T_xvsh;
  a.T_wush_bf16 = static_cast<uint16_t*>(T_wush_bf16);
  a.T_xvsh_bf16 = static_cast<uint16_t*>(T_xvsh_bf16);
  hipError_t e = wush::launch_build(G, a, stream);
  if (e != hipSuccess) return fail(WUSH_EHIP, "launch: %s", hipGetErrorString(e));
  return WUSH_OK;
}

wush_status wush_gptq_block(int fmt, const double* Wbar, const double* R, int G, int64_t d_out, double* Q,
                            void* codes, int64_t codes_stride, void* scales, int64_t scales_stride,
                            hipStream_t stream) {
  g_last_error[0] = 0;
  if (fmt != 0 && fmt != 2) return fail(WUSH_EUNSUPPORTED, "GPTQ block supports MXFP4 (0) and INT4 (2), got %d", fmt);
  if (G != 16 && G != 32) return fail(WUSH_EUNSUPPORTED, "G must be 16 or 32 (got %d)", G);
  if (d_out < 0) return fail(WUSH_EINVAL, "d_out must be >= 0");
  if (d_out == 0) return WUSH_OK;
  if (d_out > ((int64_t)1 << 40) || codes_stride < G / 2 || scales_stride < 1 || codes_stride > ((int64_t)1 << 40) ||
      scales_stride > ((int64_t)1 << 40))
    return fail(WUSH_EINVAL, "bad size or stride");
  if (!Wbar || !R || !Q || !codes || !scales) return fail(WUSH_EINVAL, "null pointer");
  if (!aligned(Wbar, 8) || !aligned(R, 8) || !aligned(Q, 8)) return fail(WUSH_EALIGN, "Wbar, R and Q must be 8-byte aligned");
  if (!aligned(codes, 4) || codes_stride % 4 != 0) return fail(WUSH_EALIGN, "code rows must be 4-byte aligned");
  if (fmt == 2 && !aligned(scales, 2)) return fail(WUSH_EALIGN, "INT4 scales must be 2-byte aligned");
  const uint64_t nw = (uint64_t)G * d_out * 8, nr = (uint64_t)G * G * 8;
  const uint64_t nc = (uint64_t)(d_out - 1) * codes_stride + G / 2;
  const uint64_t ns = ((uint64_t)(d_out - 1) * scales_stride + 1) * (fmt == 2 ? 2 : 1);
  if (overlap(Q, nw, Wbar, nw) || overlap(Q, nw, R, nr) || overlap(codes, nc, Wbar, nw) || overlap(codes, nc, R, nr) ||
      overlap(scales, ns, Wbar, nw) || overlap(scales, ns, R, nr) || overlap(codes, nc, Q, nw) ||
      overlap(scales, ns, Q, nw))
    return fail(WUSH_EINVAL, "an output overlaps an input or another output");
  wush_status st = check_device();
  if (st != WUSH_OK) return st;
  wush::GptqArgs a{};
  a.Wbar = Wbar;
  a.R = R;
  a.d_out = d_out;
  a.Q = Q;
  a.codes = static_cast<uint8_t*>(codes);
  a.codes_stride = codes_stride;
  a.scales = scales;
  a.scales_stride = scales_stride;
  hipError_t e = wush::launch_gptq_block(fmt, G, a, stream);
  if (e != hipSuccess) return fail(WUSH_EHIP, "launch: %s", hipGetErrorString(e));
  return WUSH_OK;
}

wush_status wush_gptq_wush(int fmt, const double* W, const double* Xcal, int64_t d_out, int64_t n_cal, int64_t d_in,
                           int G, double damp, int use_gptq, double* Xp, double* Y, double* T_x, double* Wq,
                           void* codes, void* scales, hipStream_t stream) {
  g_last_error[0] = 0;
  if (fmt != 0 && fmt != 2) return fail(WUSH_EUNSUPPORTED, "GPTQ-WUSH supports MXFP4 (0) and INT4 (2), got %d", fmt);
  if (G != 16 && G != 32) return fail(WUSH_EUNSUPPORTED, "G must be 16 or 32 (got %d)", G);
  if (d_in <= 0 || d_in % G != 0) return fail(WUSH_EINVAL, "d_in must be a positive multiple of %d (got %lld)", G,
                                              (long long)d_in);
  if (d_out < G || n_cal <= 0) return fail(WUSH_EINVAL, "d_out must be >= G and n_cal >= 1");
  if (d_in > ((int64_t)1 << 16) || d_out > ((int64_t)1 << 24) || n_cal > ((int64_t)1 << 30) ||
      d_out * d_in > ((int64_t)1 << 31) || n_cal * d_in > ((int64_t)1 << 36))
    return fail(WUSH_EINVAL, "sizes too large");
  if (!(damp >= 0.0) || damp > 1e30) return fail(WUSH_EINVAL, "damp must be finite and >= 0");
  if (!W || !Xcal || !Xp || !Y || !T_x || !Wq || !codes || !scales) return fail(WUSH_EINVAL, "null pointer");
  if (!aligned(W, 8) || !aligned(Xcal, 8) || !aligned(Xp, 8) || !aligned(Y, 8) || !aligned(T_x, 8) || !aligned(Wq, 8))
    return fail(WUSH_EALIGN, "float64 arrays must be 8-byte aligned");
  if (!aligned(codes, 4)) return fail(WUSH_EALIGN, "codes must be 4-byte aligned");
  if (fmt == 2 && !aligned(scales, 2)) return fail(WUSH_EALIGN, "INT4 scales must be 2-byte aligned");
  const uint64_t nw = (uint64_t)d_out * d_in * 8, nx = (uint64_t)n_cal * d_in * 8, nh = (uint64_t)d_in * d_in * 8;
  const uint64_t nt = (uint64_t)d_in * G * 8, nc = (uint64_t)d_out * d_in / 2;
  const uint64_t ns = (uint64_t)d_out * (d_in / G) * (fmt == 2 ? 2 : 1);
  const void* outs[6] = {Xp, Y, T_x, Wq, codes, scales};
  const uint64_t nout[6] = {nh, nw, nt, nw, nc, ns};
  for (int i = 0; i < 6; ++i) {
    if (overlap(outs[i], nout[i], W, nw) || overlap(outs[i], nout[i], Xcal, nx))
      return fail(WUSH_EINVAL, "an output overlaps an input");
    for (int j = i + 1; j < 6; ++j)
      if (overlap(outs[i], nout[i], outs[j], nout[j])) return fail(WUSH_EINVAL, "two outputs overlap");
  }
  wush_status st = check_device();
  if (st != WUSH_OK) return st;
  wush::GptqWushArgs a{};
  a.W = W;
  a.Xcal = Xcal;
  a.d_out = d_out;
  a.n_cal = n_cal;
  a.d_in = d_in;
  a.damp = damp;
  a.use_gptq = use_gptq ? 1 : 0;
  a.Xp = Xp;
  a.Y = Y;
  a.T_x = T_x;
  a.Wq = Wq;
  a.codes = static_cast<uint8_t*>(codes);
  a.scales = scales;
  hipError_t e = wush::launch_gptq_wush(fmt, G, a, stream);
  if (e != hipSuccess) return fail(WUSH_EHIP, "launch: %s", hipGetErrorString(e));
  return WUSH_OK;
}

wush_status wush_fixed_transforms(int kind, int64_t C, int G, double* T, void* T_bf16, hipStream_t stream) {
  g_last_error[0] = 0;
  if (kind != 0 && kind != 1) return fail(WUSH_EINVAL, "kind must be 0 (identity) or 1 (Hadamard), got %d", kind);
  if (G != 16 && G != 32) return fail(WUSH_EUNSUPPORTED, "G must be 16 or 32 (got %d)", G);
  if (C < 0) return fail(WUSH_EINVAL, "C must be >= 0");
  if (C > ((int64_t)1 << 31) / (G * G)) return fail(WUSH_EINVAL, "C too large");
  if (!T && !T_bf16) return fail(WUSH_EINVAL, "both outputs are null");
  if (C == 0) return WUSH_OK;
  if (T && !aligned(T, 8)) return fail(WUSH_EALIGN, "T must be 8-byte aligned");
  if (T_bf16 && !aligned(T_bf16, 16)) return fail(WUSH_EALIGN, "T_bf16 must be 16-byte aligned");
  const uint64_t n = (uint64_t)C * G * G;
  if (T && T_bf16 && overlap(T, n * 8, T_bf16, n * 2)) return fail(WUSH_EINVAL, "outputs overlap");
  wush_status st = check_device();
  if (st != WUSH_OK) return st;
  hipError_t e = wush::launch_fixed(kind, C, G, T, static_cast<uint16_t*>(T_bf16), stream);
  if (e != hipSuccess) return fail(WUSH_EHIP, "launch: %s", hipGetErrorString(e));
  return WUSH_OK;
}

wush_status wush_f64_to_bf16(const double* src, int64_t n, void* dst, hipStream_t stream) {
  g_last_error[0] = 0;
  if (n < 0) return fail(WUSH_EINVAL, "n must be >= 0");
  if (n == 0) return WUSH_OK;
  if (n > ((int64_t)1 << 40)) return fail(WUSH_EINVAL, "n too large");
  if (!src || !dst) return fail(WUSH_EINVAL, "null pointer");
  if (!aligned(src, 8) || !aligned(dst, 2)) return fail(WUSH_EALIGN, "src must be 8-byte and dst 2-byte aligned");
  if (overlap(src, (uint64_t)n * 8, dst, (uint64_t)n * 2)) return fail(WUSH_EINVAL, "dst overlaps src");
  wush_status st = check_device();
  if (st != WUSH_OK) return st;
  hipError_t e = wush::launch_f64_to_bf16(src, n, static_cast<uint16_t*>(dst), stream);
  if (e != hipSuccess) return fail(WUSH_EHIP, "launch: %s", hipGetErrorString(e));
  return WUSH_OK;
}

wush_status wush_e2m1_encode(const float* v, int64_t n, uint8_t* codes, hipStream_t stream) {
  g_last_error[0] = 0;
  if (n < 0) return fail(WUSH_EINVAL, "n must be >= 0");
  if (n == 0) return WUSH_OK;
  if (!v || !codes) return fail(WUSH_EINVAL, "null pointer");
  if (!aligned(v, 4)) return fail(WUSH_EALIGN, "v must be 4-byte aligned");
  if (overlap(v, (uint64_t)n * 4, codes, (uint64_t)n)) return fail(WUSH_EINVAL, "codes overlaps v");
  wush_status st = check_device();
  if (st != WUSH_OK) return st;
  hipError_t e = wush::launch_e2m1(v, n, codes, stream);
  if (e != hipSuccess) return fail(WUSH_EHIP, "launch: %s", hipGetErrorString(e));
  return WUSH_OK;
}

}  // extern "C"
