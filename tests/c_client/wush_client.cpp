// A C++ program that uses libwush through include/wush.h alone: plain HIP
// runtime calls for memory and streams, no Python and no torch in the
// process.  It quantizes one activation batch with the entry point of the
// requested format and writes the codes and scales to a file, which the
// GPU test compares with the oracle.
//
// With a "WUSHGEM1" input it runs the whole Eq. 10 forward instead:
// quantize X into the GEMM's packed operand layout, pack the MXFP4 weights
// once, multiply, and write C.
//
// Input file (little-endian):
//   char[8] "WUSHCLI1"; int32 fmt (0 MXFP4, 1 NVFP4, 2 INT4); int32 G;
//   int64 M; int64 K; float g (NVFP4: > 0 a static tensor scale, 0 = compute
//   it on the device with wush_nvfp4_global_scale);
//   X: bf16 bits [M][K]; T: bf16 bits [K/G][G][G].
// Output file:
//   char[8] "WUSHOUT1"; float g used (NVFP4, else 0);
//   codes [M][K/2] bytes; scales [M][K/G] x (1 byte, or 2 for INT4).
// GEMM input: char[8] "WUSHGEM1"; int64 M, N, K; X bf16 bits [M][K];
//   T bf16 bits [K/32][32][32]; weight codes [N][K/2]; weight E8M0 scales
//   [N][K/32].  GEMM output: char[8] "WUSHOUTG"; C fp32 [M][N].
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

// The Eq. 10 forward: wush_quant_mxfp4_packed, wush_gemm_pack_b,
// wush_gemm_mxfp4_packed.  `in` is positioned after the magic.
int run_gemm(std::FILE* in, const char* out_path) {
  int64_t M = 0, N = 0, K = 0;
  bool ok = read_into(in, &M, 1) && read_into(in, &N, 1) && read_into(in, &K, 1);
  ok = ok && M > 0 && N > 0 && K > 0 && K % 256 == 0 && M <= (int64_t)1 << 20 && N <= (int64_t)1 << 20 &&
       K <= (int64_t)1 << 16;
  if (!ok) {
    std::fprintf(stderr, "bad input header\n");
    std::fclose(in);
    return 2;
  }
  const size_t nx = (size_t)M * K, nt = (size_t)K * 32, nwc = (size_t)N * K / 2, nws = (size_t)N * K / 32;
  const int64_t Mp = (M + 127) / 128 * 128, Np = (N + 127) / 128 * 128;
  std::vector<uint16_t> x(nx), t(nt);
  std::vector<uint8_t> wc(nwc), ws(nws);
  ok = read_into(in, x.data(), nx) && read_into(in, t.data(), nt) && read_into(in, wc.data(), nwc) &&
       read_into(in, ws.data(), nws);
  std::fclose(in);
  if (!ok) {
    std::fprintf(stderr, "short input file\n");
    return 2;
  }
  void *dX = nullptr, *dT = nullptr, *dWc = nullptr, *dWs = nullptr, *dAc = nullptr, *dAs = nullptr, *dBc = nullptr,
       *dBs = nullptr, *dC = nullptr;
  hipStream_t s = nullptr;
  std::vector<float> c((size_t)M * N);
  int rc = 3;
  if (hip_ok(hipMalloc(&dX, nx * 2), "hipMalloc X") && hip_ok(hipMalloc(&dT, nt * 2), "hipMalloc T") &&
      hip_ok(hipMalloc(&dWc, nwc), "hipMalloc W codes") && hip_ok(hipMalloc(&dWs, nws), "hipMalloc W scales") &&
      hip_ok(hipMalloc(&dAc, (size_t)Mp * K / 2), "hipMalloc packed A") &&
      hip_ok(hipMalloc(&dAs, (size_t)Mp * K / 32), "hipMalloc packed A scales") &&
      hip_ok(hipMalloc(&dBc, (size_t)Np * K / 2), "hipMalloc packed B") &&
      hip_ok(hipMalloc(&dBs, (size_t)Np * K / 32), "hipMalloc packed B scales") &&
      hip_ok(hipMalloc(&dC, c.size() * sizeof(float)), "hipMalloc C") && hip_ok(hipStreamCreate(&s), "hipStreamCreate") &&
      hip_ok(hipMemcpy(dX, x.data(), nx * 2, hipMemcpyHostToDevice), "copy X") &&
      hip_ok(hipMemcpy(dT, t.data(), nt * 2, hipMemcpyHostToDevice), "copy T") &&
      hip_ok(hipMemcpy(dWc, wc.data(), nwc, hipMemcpyHostToDevice), "copy W codes") &&
      hip_ok(hipMemcpy(dWs, ws.data(), nws, hipMemcpyHostToDevice), "copy W scales") &&
      wush_ok(wush_gemm_pack_b(dWc, dWs, N, K, dBc, dBs, s), "wush_gemm_pack_b") &&
      wush_ok(wush_quant_mxfp4_packed(dX, dT, M, K, dAc, dAs, s), "wush_quant_mxfp4_packed") &&
      wush_ok(wush_gemm_mxfp4_packed(dAc, dAs, 1, dBc, dBs, M, N, K, dC, WUSH_OUT_F32, s), "wush_gemm_mxfp4_packed") &&
      hip_ok(hipStreamSynchronize(s), "hipStreamSynchronize") &&
      hip_ok(hipMemcpy(c.data(), dC, c.size() * sizeof(float), hipMemcpyDeviceToHost), "copy C"))
    rc = 0;
  if (s) (void)hipStreamDestroy(s);
  for (void* p : {dX, dT, dWc, dWs, dAc, dAs, dBc, dBs, dC}) (void)hipFree(p);
  if (rc != 0) return rc;
  std::FILE* out = std::fopen(out_path, "wb");
  if (!out) {
    std::fprintf(stderr, "cannot write %s\n", out_path);
    return 2;
  }
  ok = std::fwrite("WUSHOUTG", 1, 8, out) == 8 && std::fwrite(c.data(), sizeof(float), c.size(), out) == c.size();
  ok = (std::fclose(out) == 0) && ok;
  if (!ok) {
    std::fprintf(stderr, "write failed\n");
    return 2;
  }
  return 0;
}

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
  char magic[8] = {};
  const bool got_magic = read_into(in, magic, 8);
  if (got_magic && std::memcmp(magic, "WUSHGEM1", 8) == 0) return run_gemm(in, argv[2]);
  int32_t fmt = 0, G = 0;
  int64_t M = 0, K = 0;
  float g_static = 0.0f;
  bool ok = got_magic && std::memcmp(magic, "WUSHCLI1", 8) == 0 && read_into(in, &fmt, 1) &&
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
