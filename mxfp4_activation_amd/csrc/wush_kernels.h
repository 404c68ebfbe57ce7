// Internal interface between the C-ABI layer (wush_abi.cpp) and the device
// kernels (wush_kernels.hip).  Not part of the public ABI.
#ifndef WUSH_KERNELS_H_
#define WUSH_KERNELS_H_

#include <stdint.h>

#include <hip/hip_runtime_api.h>

namespace wush {

constexpr int kMXFP4 = 0;
constexpr int kNVFP4 = 1;
constexpr int kINT4 = 2;

constexpr int kWavesPerGroup = 4;   // waves per workgroup
#ifndef WUSH_QUANT_PANELS
#define WUSH_QUANT_PANELS 8
#endif
constexpr int kPanelsPerTile = WUSH_QUANT_PANELS;  // quant kernel: 32-channel panels (= waves) per workgroup

struct QuantArgs {
  const uint16_t* X;
  const uint16_t* T;
  uint8_t* codes;
  uint8_t* scales;
  const float* global_scale;
  uint32_t* n_exact;
  uint32_t* amax_bits;     // AbsMax kernel only: running max |y| as bits
  int64_t M;
  int64_t K;
  int64_t n_tiles;         // ceil(M / 32)
  int64_t tiles_per_wave;  // 32-token tiles each workgroup walks through
  int n_panels;            // ceil(K / 32)
  int n_pg;                // ceil(n_panels / kPanelsPerTile): tiles along K
  int n_tg;                // ceil(n_tiles / tiles_per_wave)
  int token_major;         // workgroup order: nonzero = token-major, 0 = panel-major
};

struct TransformArgs {
  const uint16_t* X;
  const uint16_t* T;
  float* Y;
  int64_t M;
  int64_t K;
  int64_t n_tiles;
  int64_t tiles_per_wave;
  int n_panels;
  int n_pg;
  int n_tg;
};

hipError_t launch_quant(int fmt, const QuantArgs& a, int n_wg, hipStream_t s);
// MXFP4 with codes and scales in the MXFP4 GEMM's packed operand layout
// (K a multiple of 256; a.codes / a.scales point at the packed buffers).
hipError_t launch_quant_mxfp4_packed(const QuantArgs& a, int n_wg, hipStream_t s);
hipError_t launch_transform(int G, const TransformArgs& a, int n_wg, hipStream_t s);
// Writes 0 to a.amax_bits, then folds max |T x| over the tensor into it.
hipError_t launch_absmax(int G, const QuantArgs& a, int n_wg, hipStream_t s);
hipError_t launch_global_scale(float* out, hipStream_t s);
hipError_t launch_e2m1(const float* v, int64_t n, uint8_t* out, hipStream_t s);

}  // namespace wush

#endif  // WUSH_KERNELS_H_
