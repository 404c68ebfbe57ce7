// Host-side checks of the C ABI (include/wush.h), built with the sanitizers
// against stubs.cpp.  It checks that:
//   * every malformed call returns its error code without making any HIP call
//     or launch (validation comes first);
//   * well-formed calls make exactly one launch (two for the global scale);
//   * the quantizer's launch plan covers every token tile and channel panel
//     exactly, for a sweep of shapes.
// Pointers are fake device addresses: nothing dereferences them.
#include <stdint.h>
#include <stdio.h>

#include "../../include/wush.h"
#include "stubs.h"

static int g_fail = 0;

#define EXPECT(cond, ...)                                   \
  do {                                                      \
    if (!(cond)) {                                          \
      ++g_fail;                                             \
      fprintf(stderr, "FAIL %s:%d: ", __FILE__, __LINE__);  \
      fprintf(stderr, __VA_ARGS__);                         \
      fprintf(stderr, "\n");                                \
    }                                                       \
  } while (0)

static void* P(uintptr_t a) { return reinterpret_cast<void*>(a); }
static const uintptr_t A = 1u << 20;  // 16-byte aligned, far from the others
static const uintptr_t B = A * 64;

// A malformed call: the expected status, no HIP call, no launch.
#define REJECT(expr, status)                                                                 \
  do {                                                                                       \
    const int h0 = g_hip_calls, l0 = g_launches;                                             \
    const wush_status st_ = (expr);                                                          \
    EXPECT(st_ == (status), "%s -> %d, want %d (%s)", #expr, (int)st_, (int)(status),       \
           wush_last_error());                                                               \
    EXPECT(g_hip_calls == h0 && g_launches == l0, "%s made a HIP call or launch", #expr);    \
    EXPECT(wush_last_error()[0] != 0, "%s left no error text", #expr);                       \
  } while (0)

// A well-formed call: OK and exactly n launches.
#define ACCEPT(expr, n)                                                                       \
  do {                                                                                        \
    const int l0 = g_launches;                                                                \
    const wush_status st_ = (expr);                                                           \
    EXPECT(st_ == WUSH_OK, "%s -> %d (%s)", #expr, (int)st_, wush_last_error());              \
    EXPECT(g_launches - l0 == (n), "%s launched %d times, want %d", #expr, g_launches - l0, (n)); \
  } while (0)

static void quant_validation() {
  for (int fmt = 0; fmt < 3; ++fmt) {
    const int G = fmt == 1 ? 16 : 32;
    const float* gs = static_cast<const float*>(P(3 * A));
    auto q = [&](uintptr_t X, uintptr_t T, int64_t M, int64_t K, uintptr_t c, uintptr_t s) {
      return wush_quant(fmt, P(X), P(T), M, K, gs, P(c), P(s), nullptr, nullptr);
    };
    ACCEPT(q(A, 2 * A, 0, 4 * G, 0, 0), 0);  // empty batch
    REJECT(q(A, 2 * A, -1, 4 * G, B, 2 * B), WUSH_EINVAL);
    REJECT(q(A, 2 * A, 8, G + 1, B, 2 * B), WUSH_EINVAL);
    REJECT(q(A, 2 * A, 8, 0, B, 2 * B), WUSH_EINVAL);
    REJECT(q(A, 2 * A, 8, (int64_t)1 << 31, B, 2 * B), WUSH_EINVAL);
    REJECT(q(A, 2 * A, INT64_MAX / 8, 1 << 20, B, 2 * B), WUSH_EINVAL);  // M*K overflows
    REJECT(q(0, 2 * A, 8, G, B, 2 * B), WUSH_EINVAL);
    REJECT(q(A, 0, 8, G, B, 2 * B), WUSH_EINVAL);
    REJECT(q(A, 2 * A, 8, G, 0, 2 * B), WUSH_EINVAL);
    REJECT(q(A, 2 * A, 8, G, B, 0), WUSH_EINVAL);
    REJECT(q(A + 2, 2 * A, 8, G, B, 2 * B), WUSH_EALIGN);
    REJECT(q(A, 2 * A + 8, 8, G, B, 2 * B), WUSH_EALIGN);
    REJECT(q(A, 2 * A, 8, G, B + 8, 2 * B), WUSH_EALIGN);  // codes need 16 bytes
    REJECT(q(A, 2 * A, 8, G, B, 2 * B + 4), WUSH_EALIGN);  // scales need 8 (MXFP4) or 16 bytes
    if (fmt != 0) REJECT(q(A, 2 * A, 8, G, B, 2 * B + 8), WUSH_EALIGN);
    else ACCEPT(q(A, 2 * A, 8, G, B, 2 * B + 8), 1);
    REJECT(q(A, 8 * A, 8, 4 * G, A + 64, 16 * A), WUSH_EINVAL);  // codes overlap X
    REJECT(q(A, 2 * A, 64, 4 * G, 2 * A, 16 * A), WUSH_EINVAL);  // codes overlap T
    REJECT(q(A, 2 * A, 64, 4 * G, B, B + 16), WUSH_EINVAL);      // codes overlap scales
    if (fmt == 1) {
      REJECT(wush_quant(fmt, P(A), P(2 * A), 8, G, nullptr, P(B), P(2 * B), nullptr, nullptr), WUSH_EINVAL);
      REJECT(wush_quant(fmt, P(A), P(2 * A), 8, G, static_cast<const float*>(P(3 * A + 2)), P(B), P(2 * B),
                        nullptr, nullptr),
             WUSH_EALIGN);
    }
    REJECT(wush_quant(fmt, P(A), P(2 * A), 8, G, gs, P(B), P(2 * B), static_cast<uint32_t*>(P(3 * B + 2)), nullptr),
           WUSH_EALIGN);
    ACCEPT(q(A, 2 * A, 8, G, B, 2 * B), 1);
  }
  REJECT(wush_quant(3, P(A), P(2 * A), 8, 32, nullptr, P(B), P(2 * B), nullptr, nullptr), WUSH_EUNSUPPORTED);
  REJECT(wush_quant(-1, P(A), P(2 * A), 8, 32, nullptr, P(B), P(2 * B), nullptr, nullptr), WUSH_EUNSUPPORTED);
  ACCEPT(wush_quant_mxfp4(P(A), P(2 * A), 8, 64, P(B), P(2 * B), nullptr), 1);
  ACCEPT(wush_quant_nvfp4(P(A), P(2 * A), 8, 64, static_cast<const float*>(P(3 * A)), P(B), P(2 * B), nullptr), 1);
  ACCEPT(wush_quant_int4(P(A), P(2 * A), 8, 64, P(B), P(2 * B), nullptr), 1);
}

// The quantizer's plan: every 32-token tile and every 256-channel column
// belongs to exactly one workgroup, runs are 1 to 3 tiles, and NVFP4 runs
// at most 2.
static void quant_plan() {
  const int64_t Ms[] = {1, 31, 32, 33, 64, 100, 1000, 4096, 4100, 8192, 8200, 16384, 65536};
  const int64_t Ks[] = {32, 64, 96, 256, 288, 4096, 4128, 8192, 14336};
  for (int fmt = 0; fmt < 3; ++fmt)
    for (int64_t M : Ms)
      for (int64_t K : Ks) {
        if (fmt == 1 && K % 16) continue;
        const int l0 = g_launches;
        const wush_status st = wush_quant(fmt, P(A), P(A + (uintptr_t)(M * K * 2 + 4096) / 16 * 16 + 4096), M, K,
                                          static_cast<const float*>(P(8)), P(B * 1024), P(B * 4096), nullptr,
                                          nullptr);
        EXPECT(st == WUSH_OK && g_launches == l0 + 1, "fmt %d M %lld K %lld: %s", fmt, (long long)M, (long long)K,
               wush_last_error());
        if (st != WUSH_OK) continue;
        const wush::QuantArgs& a = g_last_quant.args;
        const int64_t tiles = (M + 31) / 32, panels = (K + 31) / 32;
        EXPECT(a.n_tiles == tiles && a.n_panels == panels, "fmt %d M %lld K %lld: tiles/panels", fmt, (long long)M,
               (long long)K);
        EXPECT(a.tiles_per_wave >= 1 && a.tiles_per_wave <= (fmt == 1 ? 2 : 3), "fmt %d: run length %lld", fmt,
               (long long)a.tiles_per_wave);
        EXPECT((int64_t)a.n_pg * wush::kPanelsPerTile >= panels && (int64_t)(a.n_pg - 1) * wush::kPanelsPerTile < panels,
               "fmt %d M %lld K %lld: panel groups %d", fmt, (long long)M, (long long)K, a.n_pg);
        EXPECT((int64_t)a.n_tg * a.tiles_per_wave >= tiles && (int64_t)(a.n_tg - 1) * a.tiles_per_wave < tiles,
               "fmt %d M %lld K %lld: token groups %d x %lld", fmt, (long long)M, (long long)K, a.n_tg,
               (long long)a.tiles_per_wave);
        EXPECT((int64_t)g_last_quant.n_wg == (int64_t)a.n_pg * a.n_tg, "grid size");
      }
}

static void support_validation() {
  ACCEPT(wush_absmax_transformed(P(A), P(2 * A), 0, 64, 32, static_cast<float*>(P(B)), nullptr), 1);  // fills 0
  REJECT(wush_absmax_transformed(P(A), P(2 * A), 8, 64, 24, static_cast<float*>(P(B)), nullptr), WUSH_EUNSUPPORTED);
  REJECT(wush_absmax_transformed(P(A), P(2 * A), 8, 48, 32, static_cast<float*>(P(B)), nullptr), WUSH_EINVAL);
  REJECT(wush_absmax_transformed(P(A), P(2 * A), 8, 64, 32, nullptr, nullptr), WUSH_EINVAL);
  REJECT(wush_absmax_transformed(P(A), P(2 * A), 8, 64, 32, static_cast<float*>(P(B + 2)), nullptr), WUSH_EALIGN);
  REJECT(wush_absmax_transformed(P(A), P(2 * A), 8, 64, 32, static_cast<float*>(P(A + 16)), nullptr), WUSH_EINVAL);
  ACCEPT(wush_absmax_transformed(P(A), P(2 * A), 8, 64, 16, static_cast<float*>(P(B)), nullptr), 1);
  EXPECT(g_last_quant.fmt == -1 && g_last_quant.n_wg >= 1, "AbsMax plan");
  ACCEPT(wush_nvfp4_global_scale(P(A), P(2 * A), 8, 64, static_cast<float*>(P(B)), nullptr), 2);
  REJECT(wush_nvfp4_global_scale(P(A), P(2 * A), 8, 40, static_cast<float*>(P(B)), nullptr), WUSH_EINVAL);

  REJECT(wush_transform_f32(P(A), P(2 * A), 8, 64, 8, static_cast<float*>(P(B)), nullptr), WUSH_EUNSUPPORTED);
  REJECT(wush_transform_f32(P(A), P(2 * A), 8, 64, 32, nullptr, nullptr), WUSH_EINVAL);
  REJECT(wush_transform_f32(P(A), P(2 * A), 8, 64, 32, static_cast<float*>(P(B + 4)), nullptr), WUSH_EALIGN);
  REJECT(wush_transform_f32(P(A), P(2 * A), 8, 64, 32, static_cast<float*>(P(A + 512)), nullptr), WUSH_EINVAL);
  ACCEPT(wush_transform_f32(P(A), P(2 * A), 8, 64, 32, static_cast<float*>(P(B)), nullptr), 1);

  REJECT(wush_e2m1_encode(static_cast<const float*>(P(A)), -1, static_cast<uint8_t*>(P(B)), nullptr), WUSH_EINVAL);
  ACCEPT(wush_e2m1_encode(static_cast<const float*>(P(A)), 0, nullptr, nullptr), 0);
  REJECT(wush_e2m1_encode(static_cast<const float*>(P(A + 2)), 8, static_cast<uint8_t*>(P(B)), nullptr), WUSH_EALIGN);
  REJECT(wush_e2m1_encode(static_cast<const float*>(P(A)), 8, static_cast<uint8_t*>(P(A + 4)), nullptr), WUSH_EINVAL);
  ACCEPT(wush_e2m1_encode(static_cast<const float*>(P(A)), 8, static_cast<uint8_t*>(P(B)), nullptr), 1);

  REJECT(wush_fixed_transforms(2, 4, 32, static_cast<double*>(P(A)), nullptr, nullptr), WUSH_EINVAL);
  REJECT(wush_fixed_transforms(1, 4, 8, static_cast<double*>(P(A)), nullptr, nullptr), WUSH_EUNSUPPORTED);
  REJECT(wush_fixed_transforms(1, -1, 32, static_cast<double*>(P(A)), nullptr, nullptr), WUSH_EINVAL);
  REJECT(wush_fixed_transforms(1, 4, 32, nullptr, nullptr, nullptr), WUSH_EINVAL);
  REJECT(wush_fixed_transforms(1, 4, 32, static_cast<double*>(P(A + 4)), nullptr, nullptr), WUSH_EALIGN);
  REJECT(wush_fixed_transforms(1, 4, 32, nullptr, P(A + 8), nullptr), WUSH_EALIGN);
  REJECT(wush_fixed_transforms(1, 4, 32, static_cast<double*>(P(A)), P(A + 64), nullptr), WUSH_EINVAL);
  REJECT(wush_fixed_transforms(0, (int64_t)1 << 40, 32, static_cast<double*>(P(A)), nullptr, nullptr), WUSH_EINVAL);
  ACCEPT(wush_fixed_transforms(0, 0, 32, static_cast<double*>(P(A)), nullptr, nullptr), 0);
  ACCEPT(wush_fixed_transforms(1, 4, 16, static_cast<double*>(P(A)), P(B), nullptr), 1);

  REJECT(wush_f64_to_bf16(static_cast<const double*>(P(A)), -1, P(B), nullptr), WUSH_EINVAL);
  REJECT(wush_f64_to_bf16(static_cast<const double*>(P(A + 4)), 8, P(B), nullptr), WUSH_EALIGN);
  REJECT(wush_f64_to_bf16(static_cast<const double*>(P(A)), 8, P(B + 1), nullptr), WUSH_EALIGN);
  REJECT(wush_f64_to_bf16(static_cast<const double*>(P(A)), 8, P(A + 8), nullptr), WUSH_EINVAL);
  ACCEPT(wush_f64_to_bf16(static_cast<const double*>(P(A)), 0, nullptr, nullptr), 0);
  ACCEPT(wush_f64_to_bf16(static_cast<const double*>(P(A)), 8, P(B), nullptr), 1);
}

static void other_entries() {
  auto g = [](uintptr_t ac, uintptr_t as, uintptr_t bc, uintptr_t bs, int64_t M, int64_t N, int64_t K, uintptr_t C,
              int t) { return wush_gemm_mxfp4(P(ac), P(as), P(bc), P(bs), M, N, K, P(C), t, nullptr); };
  ACCEPT(g(A, 2 * A, 3 * A, 4 * A, 0, 16, 256, B, 0), 0);
  REJECT(g(A, 2 * A, 3 * A, 4 * A, 16, 16, 128, B, 0), WUSH_EINVAL);
  REJECT(g(A, 2 * A, 3 * A, 4 * A, 16, 16, 256, B, 2), WUSH_EINVAL);
  REJECT(g(A + 8, 2 * A, 3 * A, 4 * A, 16, 16, 256, B, 0), WUSH_EALIGN);
  REJECT(g(A, 2 * A + 4, 3 * A, 4 * A, 16, 16, 256, B, 0), WUSH_EALIGN);
  REJECT(g(A, 2 * A, 3 * A, 4 * A, 16, 16, 256, 3 * A + 64, 0), WUSH_EINVAL);
  REJECT(g(A, 2 * A, 3 * A, 4 * A, INT64_MAX / 2, INT64_MAX / 2, 256, B, 0), WUSH_EINVAL);
  ACCEPT(g(A, 2 * A, 3 * A, 4 * A, 16, 16, 256, B, 1), 1);

  auto gp = [](uintptr_t ac, uintptr_t as, int ap, uintptr_t bc, uintptr_t bs, int64_t M, int64_t N, int64_t K,
               uintptr_t C, int t) {
    return wush_gemm_mxfp4_packed(P(ac), P(as), ap, P(bc), P(bs), M, N, K, P(C), t, nullptr);
  };
  ACCEPT(gp(A, 2 * A, 1, 3 * A, 4 * A, 0, 16, 256, B, 0), 0);
  REJECT(gp(A, 2 * A, 2, 3 * A, 4 * A, 16, 16, 256, B, 0), WUSH_EINVAL);
  REJECT(gp(A, 2 * A, 1, 3 * A, 4 * A, 16, 16, 256, A + 4096, 0), WUSH_EINVAL);  // inside A's padded rows
  REJECT(gp(A, 2 * A, 0, 3 * A, 4 * A, 16, 16, 256, 3 * A + 4096, 0), WUSH_EINVAL);  // inside B's padded rows
  REJECT(gp(A, 2 * A, 0, 3 * A + 8, 4 * A, 16, 16, 256, B, 0), WUSH_EALIGN);
  ACCEPT(gp(A, 2 * A, 0, 3 * A, 4 * A, 16, 16, 256, B, 1), 1);
  ACCEPT(gp(A, 2 * A, 1, 3 * A, 4 * A, 16, 16, 256, B, 0), 1);

  auto pk = [](uintptr_t bc, uintptr_t bs, int64_t N, int64_t K, uintptr_t pc, uintptr_t ps) {
    return wush_gemm_pack_b(P(bc), P(bs), N, K, P(pc), P(ps), nullptr);
  };
  ACCEPT(pk(A, 2 * A, 0, 256, B, 2 * B), 0);
  REJECT(pk(A, 2 * A, -1, 256, B, 2 * B), WUSH_EINVAL);
  REJECT(pk(A, 2 * A, 16, 320, B, 2 * B), WUSH_EINVAL);
  REJECT(pk(A + 8, 2 * A, 16, 256, B, 2 * B), WUSH_EALIGN);
  REJECT(pk(A, 2 * A, 16, 256, B, 2 * B + 4), WUSH_EALIGN);
  REJECT(pk(A, 2 * A, 16, 256, A + 1024, 2 * B), WUSH_EINVAL);
  REJECT(pk(A, 2 * A, 16, 256, B, B + 8192), WUSH_EINVAL);
  REJECT(pk(A, 2 * A, INT64_MAX / 4, 256, B, 2 * B), WUSH_EINVAL);
  ACCEPT(pk(A, 2 * A, 16, 256, B, 2 * B), 1);

  auto qp = [](uintptr_t X, uintptr_t T, int64_t M, int64_t K, uintptr_t c, uintptr_t s) {
    return wush_quant_mxfp4_packed(P(X), P(T), M, K, P(c), P(s), nullptr);
  };
  ACCEPT(qp(A, 2 * A, 0, 256, B, 2 * B), 0);
  REJECT(qp(A, 2 * A, 4, 320, B, 2 * B), WUSH_EINVAL);
  REJECT(qp(A, 2 * A, 4, 256, 0, 2 * B), WUSH_EINVAL);
  REJECT(qp(A, 2 * A, 4, 256, B + 8, 2 * B), WUSH_EALIGN);
  REJECT(qp(A, 2 * A, 4, 256, B, 2 * B + 4), WUSH_EALIGN);
  REJECT(qp(A, 2 * A, 4, 256, B, B + 8192), WUSH_EINVAL);
  REJECT(qp(A, 2 * A, 4, 256, A + 1024, 2 * B), WUSH_EINVAL);
  ACCEPT(qp(A, 2 * A, 4, 256, B, 2 * B), 1);

  auto d = [](int fmt, uintptr_t c, uintptr_t s, uintptr_t gs, int64_t M, int64_t K, uintptr_t o) {
    return wush_dequant(fmt, P(c), P(s), static_cast<const float*>(P(gs)), M, K, static_cast<float*>(P(o)), nullptr);
  };
  ACCEPT(d(0, A, 2 * A, 0, 0, 64, B), 0);
  REJECT(d(3, A, 2 * A, 0, 4, 64, B), WUSH_EUNSUPPORTED);
  REJECT(d(1, A, 2 * A, 0, 4, 48, B), WUSH_EINVAL);
  REJECT(d(2, A, 2 * A + 1, 0, 4, 64, B), WUSH_EALIGN);
  REJECT(d(0, A, 2 * A, 0, 4, 64, A), WUSH_EINVAL);
  ACCEPT(d(1, A, 2 * A, 3 * A, 4, 48, B), 1);

  auto b = [](uintptr_t W, int64_t dout, uintptr_t X, int64_t nc, int64_t din, int G, double damp, uintptr_t tw,
              uintptr_t tx) {
    return wush_build_transforms(P(W), dout, P(X), nc, din, G, damp, 1, static_cast<double*>(P(tw)),
                                 static_cast<double*>(P(tx)), nullptr, nullptr, nullptr);
  };
  REJECT(b(A, 8, 2 * A, 8, 64, 24, 1e-6, B, 2 * B), WUSH_EUNSUPPORTED);
  REJECT(b(A, 0, 2 * A, 8, 64, 32, 1e-6, B, 2 * B), WUSH_EINVAL);
  REJECT(b(A, 8, 2 * A, 8, 64, 32, -1.0, B, 2 * B), WUSH_EINVAL);
  REJECT(b(A, 8, 2 * A, 8, 64, 32, 1e-6, B, B), WUSH_EINVAL);
  REJECT(b(A + 8, 8, 2 * A, 8, 64, 32, 1e-6, B, 2 * B), WUSH_EALIGN);
  ACCEPT(b(A, 8, 2 * A, 8, 64, 32, 1e-6, B, 2 * B), 1);

  auto q = [](int fmt, int G, int64_t dout, int64_t cs, uintptr_t c) {
    return wush_gptq_block(fmt, static_cast<const double*>(P(A)), static_cast<const double*>(P(2 * A)), G, dout,
                           static_cast<double*>(P(B)), P(c), cs, P(5 * B), 1, nullptr);
  };
  ACCEPT(q(0, 32, 0, 16, 3 * B), 0);
  REJECT(q(1, 32, 8, 16, 3 * B), WUSH_EUNSUPPORTED);
  REJECT(q(0, 32, 8, 8, 3 * B), WUSH_EINVAL);
  REJECT(q(0, 32, 8, 18, 3 * B), WUSH_EALIGN);
  REJECT(q(0, 32, 8, 16, B), WUSH_EINVAL);
  ACCEPT(q(2, 32, 8, 16, 3 * B), 1);

  // GPTQ-WUSH: W, Xcal inputs; Xp, Y, T_x, Wq, codes, scales outputs, each
  // far from the others.
  auto gw = [](int fmt, int G, int64_t dout, int64_t n, int64_t din, double damp, uintptr_t xp, uintptr_t cd,
               uintptr_t sc) {
    return wush_gptq_wush(fmt, static_cast<const double*>(P(A)), static_cast<const double*>(P(2 * A)), dout, n, din,
                          G, damp, 1, static_cast<double*>(P(xp)), static_cast<double*>(P(2 * B)),
                          static_cast<double*>(P(3 * B)), static_cast<double*>(P(4 * B)), P(cd), P(sc), nullptr);
  };
  REJECT(gw(1, 32, 40, 16, 64, 0.01, B, 5 * B, 6 * B), WUSH_EUNSUPPORTED);
  REJECT(gw(0, 24, 40, 16, 48, 0.01, B, 5 * B, 6 * B), WUSH_EUNSUPPORTED);
  REJECT(gw(0, 32, 40, 16, 48, 0.01, B, 5 * B, 6 * B), WUSH_EINVAL);
  REJECT(gw(0, 32, 0, 16, 64, 0.01, B, 5 * B, 6 * B), WUSH_EINVAL);
  REJECT(gw(0, 32, 31, 16, 64, 0.01, B, 5 * B, 6 * B), WUSH_EINVAL);  // d_out < G
  REJECT(gw(0, 32, 40, 0, 64, 0.01, B, 5 * B, 6 * B), WUSH_EINVAL);
  REJECT(gw(0, 32, 40, 16, 64, -1.0, B, 5 * B, 6 * B), WUSH_EINVAL);
  REJECT(gw(0, 32, 40, 16, 64, 0.01, B + 4, 5 * B, 6 * B), WUSH_EALIGN);
  REJECT(gw(0, 32, 40, 16, 64, 0.01, B, 5 * B + 2, 6 * B), WUSH_EALIGN);
  REJECT(gw(2, 32, 40, 16, 64, 0.01, B, 5 * B, 6 * B + 1), WUSH_EALIGN);
  REJECT(gw(0, 32, 40, 16, 64, 0.01, B, 2 * B, 6 * B), WUSH_EINVAL);  // codes over Y
  REJECT(gw(0, 32, 40, 16, 64, 0.01, A, 5 * B, 6 * B), WUSH_EINVAL);  // Xp over W
  ACCEPT(gw(0, 32, 40, 16, 64, 0.01, B, 5 * B, 6 * B), 1);
  ACCEPT(gw(2, 16, 16, 16, 64, 0.0, B, 5 * B, 6 * B), 1);
}

int main() {
  EXPECT(wush_abi_version() == WUSH_ABI_VERSION, "ABI version");
  for (int s = 0; s <= 4; ++s) EXPECT(wush_status_string(static_cast<wush_status>(s))[0], "status string %d", s);
  quant_validation();
  quant_plan();
  support_validation();
  other_entries();
  if (g_fail) {
    fprintf(stderr, "%d check(s) failed\n", g_fail);
    return 1;
  }
  printf("abi host checks passed (%d launches, %d HIP calls)\n", g_launches, g_hip_calls);
  return 0;
}
