// A C++ program that uses libwush through include/wush.h alone: plain HIP
// runtime calls for memory and streams, no Python and no torch in the
// process.  It quantizes one activation batch with the entry point of the
// requested format and writes the codes and scales to a file, which the
// GPU test compares with the oracle.
//
// Input file (little-endian):
//   char[8] "WUSHCLI1"; int32 fmt (0 MXFP4, 1 NVFP4, 2 INT4); int32 G;
//   int64 M; int64 K; float g (NVFP4: > 0 a static tensor scale, 0 = compute
//   it on the device with wush_nvfp4_global_scale);
//   X: bf16 bits [M][K]; T: bf16 bits [K/G][G][G].
// Output file:
//   char[8] "WUSHOUT1"; float g used (NVFP4, else 0);
//   codes [M][K/2] bytes; scales [M][K/G] x (1 byte, or 2 for INT4).
// Exit status 0 on success; 2 on a bad input file; 3 on a library or HIP
// error (the message goes to stderr).

#include <cstdint>
#include <cstdio>
#include <cstring>
#include <vector>

#include <hip/hip_runtime_api.h>

#include "wush.h"

namespace {

bool hip_ok(hipError_t e, const char* what) {
  if (e == hipSuccess) return true;
  std::fprintf(stderr, "%s: %s\n", what, hipGetErrorString(e));
  return false;
}

bool wush_ok(wush_status s, const char* what) {
  if (s == WUSH_OK) return true;
  std::fprintf(stderr, "%s: %s (%s)\n", what, wush_status_string(s), wush_last_error());
  return false;
}

template <typename V>
bool read_into(std::FILE* f, V* p, size_t n) {
  return std::fread(p, sizeof(V), n, f) == n;
}

}  // namespace

int main(int argc, char** argv) {
  if (argc != 3) {
    std::fprintf(stderr, "usage: %s in.bin out.bin\n", argv[0]);
    return 2;
  }
  if (wush_abi_version() != WUSH_ABI_VERSION) {
    std::fprintf(stderr, "library ABI %d, header %d\n", wush_abi_version(), WUSH_ABI_VERSION);
    return 3;
  }
  std::FILE* in = std::fopen(argv[1], "rb");
  if (!in) {
    std::fprintf(stderr, "cannot open %s\n", argv[1]);
    return 2;
  }
  char magic[8];
  int32_t fmt = 0, G = 0;
  int64_t M = 0, K = 0;
  float g_static = 0.0f;
  bool ok = read_into(in, magic, 8) && std::memcmp(magic, "WUSHCLI1", 8) == 0 && read_into(in, &fmt, 1) &&
            read_into(in, &G, 1) && read_into(in, &M, 1) && read_into(in, &K, 1) && read_into(in, &g_static, 1);
  ok = ok && (fmt == 0 || fmt == 1 || fmt == 2) && (G == (fmt == 1 ? 16 : 32)) && M >= 0 && K > 0 && K % G == 0 &&
       M <= (int64_t)1 << 24 && K <= (int64_t)1 << 20;
  if (!ok) {
    std::fprintf(stderr, "bad input header\n");
    std::fclose(in);
    return 2;
  }
  const size_t nx = (size_t)M * (size_t)K, nt = (size_t)(K / G) * G * G;
  const size_t n_codes = nx / 2, s_bytes = (fmt == 2) ? 2 : 1, n_scales = (size_t)M * (size_t)(K / G) * s_bytes;
  std::vector<uint16_t> x(nx), t(nt);
  ok = read_into(in, x.data(), nx) && read_into(in, t.data(), nt);
  std::fclose(in);
  if (!ok) {
    std::fprintf(stderr, "short input file\n");
    return 2;
  }

  void *dX = nullptr, *dT = nullptr, *dC = nullptr, *dS = nullptr;
  float* dG = nullptr;
  hipStream_t s = nullptr;
  std::vector<uint8_t> codes(n_codes), scales(n_scales);
  float g_used = 0.0f;
  int rc = 3;
  // hipMalloc of 0 bytes returns a null pointer; allocate at least one byte
  // so that every buffer is a real device address.
  if (hip_ok(hipMalloc(&dX, nx * 2 + 1), "hipMalloc X") && hip_ok(hipMalloc(&dT, nt * 2), "hipMalloc T") &&
      hip_ok(hipMalloc(&dC, n_codes + 1), "hipMalloc codes") && hip_ok(hipMalloc(&dS, n_scales + 1), "hipMalloc scales") &&
      hip_ok(hipMalloc((void**)&dG, sizeof(float)), "hipMalloc g") && hip_ok(hipStreamCreate(&s), "hipStreamCreate") &&
      hip_ok(hipMemcpy(dX, x.data(), nx * 2, hipMemcpyHostToDevice), "copy X") &&
      hip_ok(hipMemcpy(dT, t.data(), nt * 2, hipMemcpyHostToDevice), "copy T") &&
      hip_ok(hipMemcpy(dG, &g_static, sizeof(float), hipMemcpyHostToDevice), "copy g")) {
    bool launched = false;
    if (fmt == 0) {
      launched = wush_ok(wush_quant_mxfp4(dX, dT, M, K, dC, dS, s), "wush_quant_mxfp4");
    } else if (fmt == 1) {
      launched = (g_static > 0.0f || wush_ok(wush_nvfp4_global_scale(dX, dT, M, K, dG, s), "wush_nvfp4_global_scale")) &&
                 wush_ok(wush_quant_nvfp4(dX, dT, M, K, dG, dC, dS, s), "wush_quant_nvfp4");
    } else {
      launched = wush_ok(wush_quant_int4(dX, dT, M, K, dC, dS, s), "wush_quant_int4");
    }
    if (launched && hip_ok(hipStreamSynchronize(s), "hipStreamSynchronize") &&
        hip_ok(hipMemcpy(codes.data(), dC, n_codes, hipMemcpyDeviceToHost), "copy codes") &&
        hip_ok(hipMemcpy(scales.data(), dS, n_scales, hipMemcpyDeviceToHost), "copy scales") &&
        hip_ok(hipMemcpy(&g_used, dG, sizeof(float), hipMemcpyDeviceToHost), "copy g"))
      rc = 0;
  }
  if (s) (void)hipStreamDestroy(s);
  (void)hipFree(dX);
  (void)hipFree(dT);
  (void)hipFree(dC);
  (void)hipFree(dS);
  (void)hipFree(dG);
  if (rc != 0) return rc;

  std::FILE* out = std::fopen(argv[2], "wb");
  if (!out) {
    std::fprintf(stderr, "cannot write %s\n", argv[2]);
    return 2;
  }
  if (fmt != 1) g_used = 0.0f;
  ok = std::fwrite("WUSHOUT1", 1, 8, out) == 8 && std::fwrite(&g_used, sizeof(float), 1, out) == 1 &&
       std::fwrite(codes.data(), 1, n_codes, out) == n_codes && std::fwrite(scales.data(), 1, n_scales, out) == n_scales;
  ok = (std::fclose(out) == 0) && ok;
  if (!ok) {
    std::fprintf(stderr, "write failed\n");
    return 2;
  }
  return 0;
}
