// Host stand-ins for the HIP runtime calls and kernel launchers the C-ABI
// layer makes, so that its validation and launch planning can be built and
// run on a machine without a GPU (under AddressSanitizer and UBSan).
//
// Every stand-in counts its calls.  The device query reports one gfx950
// device, so a call that passes validation reaches its launcher, which
// records the launch shape and returns success.

#include <stdint.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "../../mxfp4_activation_amd/csrc/wush_build.h"
#include "../../mxfp4_activation_amd/csrc/wush_dequant.h"
#include "../../mxfp4_activation_amd/csrc/wush_gemm.h"
#include "../../mxfp4_activation_amd/csrc/wush_gptq.h"
#include "../../mxfp4_activation_amd/csrc/wush_kernels.h"
#include "stubs.h"

int g_hip_calls = 0;
int g_launches = 0;
StubQuant g_last_quant;

extern "C" {

hipError_t hipGetDevice(int* dev) {
  ++g_hip_calls;
  *dev = 0;
  return hipSuccess;
}

hipError_t hipGetDevicePropertiesR0600(hipDeviceProp_t* prop, int dev) {
  ++g_hip_calls;
  if (dev != 0) return hipErrorInvalidDevice;
  memset(prop, 0, sizeof(*prop));
  strcpy(prop->gcnArchName, "gfx950:sramecc+:xnack-");
  return hipSuccess;
}

const char* hipGetErrorString(hipError_t) { return "stub"; }

}  // extern "C"

namespace wush {

hipError_t launch_quant(int fmt, const QuantArgs& a, int n_wg, hipStream_t) {
  ++g_launches;
  g_last_quant.fmt = fmt;
  g_last_quant.args = a;
  g_last_quant.n_wg = n_wg;
  return hipSuccess;
}
hipError_t launch_quant_mxfp4_packed(const QuantArgs& a, int n_wg, hipStream_t) {
  ++g_launches;
  g_last_quant.fmt = 0;
  g_last_quant.args = a;
  g_last_quant.n_wg = n_wg;
  return hipSuccess;
}
hipError_t launch_transform(int, const TransformArgs&, int, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_absmax(int, const QuantArgs& a, int n_wg, hipStream_t) {
  ++g_launches;
  g_last_quant.fmt = -1;
  g_last_quant.args = a;
  g_last_quant.n_wg = n_wg;
  return hipSuccess;
}
hipError_t launch_global_scale(float*, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_e2m1(const float*, int64_t, uint8_t*, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_gemm_mxfp4(const GemmArgs&, bool, int, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_pack_b(const uint8_t*, const uint8_t*, int64_t, int64_t, uint8_t*, uint8_t*, hipStream_t) {
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_dequant(int, const uint8_t*, const void*, const float*, int64_t, int64_t, float*, hipStream_t) {
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_build(int, const BuildArgs&, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_fixed(int, int64_t, int, double*, uint16_t*, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_f64_to_bf16(const double*, int64_t, uint16_t*, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_gptq_block(int, int, const GptqArgs&, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_gptq_wush(int, int, const GptqWushArgs&, hipStream_t) { ++g_launches; return hipSuccess; }

}  // namespace wush
