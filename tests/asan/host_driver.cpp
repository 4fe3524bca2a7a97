// Host-side driver for the AddressSanitizer build (tests/test_asan_host.py):
// the host format converters over every input class, and every device entry
// point's argument validation in dry-run mode (valid and invalid calls), in a
// binary built with -fsanitize=address.  Launchers are stubs that abort: a
// dry run must never reach one.  Exit status 0 and no sanitizer report is a
// pass.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "mxfp8.h"

struct ihipStream_t;
typedef ihipStream_t* hipStream_t;

#define STUB(...)                                                        \
  {                                                                      \
    std::fprintf(stderr, "a launcher was reached in dry-run mode\n");   \
    std::abort();                                                        \
  }

namespace mx {
mx_status launch_quant(const void*, const int64_t*, const void*, const void*, int64_t, int64_t, int32_t, int32_t,
                       int32_t, int32_t, int32_t, int32_t, uint8_t*, uint8_t*, hipStream_t) STUB()
mx_status launch_bmm(const uint8_t*, const uint8_t*, int32_t, const uint8_t*, const uint8_t*, void*, int64_t, int32_t,
                     int32_t, int32_t, hipStream_t) STUB()
mx_status launch_gemm_mx32(const uint8_t*, const uint8_t*, const uint8_t*, const uint8_t*, void*, int64_t, int64_t,
                           int64_t, hipStream_t) STUB()
bool launch_linear_mx32_fused(const void*, const uint8_t*, const uint8_t*, void*, int64_t, int64_t, int64_t,
                              hipStream_t, mx_status*) STUB()
bool launch_gemm_mx32_wres(const uint8_t*, const uint8_t*, const uint8_t*, const uint8_t*, void*, int64_t, int64_t,
                           int64_t, hipStream_t, mx_status*) STUB()
mx_status launch_gemm_bf16(const void*, const void*, void*, int64_t, int64_t, int64_t, hipStream_t) STUB()
mx_status launch_dequant(const uint8_t*, const uint8_t*, void*, int64_t, int64_t, int32_t, hipStream_t) STUB()
mx_status launch_f32_to_e8m0(const float*, uint8_t*, int64_t, int32_t*, hipStream_t) STUB()
mx_status launch_f32_to_e4m3(const float*, uint8_t*, int64_t, int32_t, hipStream_t) STUB()
mx_status launch_rope_bf16(const void*, const int64_t*, const void*, const void*, int64_t, int64_t, int32_t, int32_t,
                           int32_t, int32_t, void*, hipStream_t) STUB()
mx_status launch_bmm_bf16(const void*, const void*, void*, int64_t, int32_t, int32_t, int32_t, hipStream_t) STUB()
mx_status launch_expand_scales(const void*, int32_t, int32_t, int32_t, int32_t, int32_t, uint8_t*, int32_t*,
                               hipStream_t) STUB()
mx_status launch_woa_fused(const void*, const int64_t*, const void*, const void*, int64_t, int64_t, int32_t, int32_t,
                           int32_t, int32_t, const uint8_t*, const uint8_t*, void*, int32_t, int32_t,
                           hipStream_t) STUB()
mx_status launch_stream_read(const void*, int64_t, uint32_t*, hipStream_t) STUB()
}  // namespace mx

static int failures = 0;
#define EXPECT(cond)                                                             \
  do {                                                                           \
    if (!(cond)) {                                                               \
      std::fprintf(stderr, "%s:%d: expectation failed: %s\n", __FILE__, __LINE__, #cond); \
      ++failures;                                                                \
    }                                                                            \
  } while (0)

int main() {
  // ---- host converters over every BF16 pattern times a range of powers of two
  std::vector<float> in;
  for (int e = -140; e <= 10; e += 5)
    for (uint32_t b = 0; b < 0x10000; ++b) {
      uint32_t u = b << 16;
      float f;
      std::memcpy(&f, &u, 4);
      in.push_back(std::ldexp(f, e));
    }
  std::vector<uint8_t> codes(in.size());
  EXPECT(mx_f32_to_e4m3_ocp(in.data(), codes.data(), static_cast<int64_t>(in.size())) == MX_OK);
  EXPECT(mx_f32_to_e4m3_fnuz(in.data(), codes.data(), static_cast<int64_t>(in.size())) == MX_OK);
  EXPECT(mx_f32_to_e4m3_ocp(nullptr, nullptr, 0) == MX_OK);
  EXPECT(mx_f32_to_e4m3_ocp(nullptr, codes.data(), 4) == MX_ERR_INVALID_ARG);
  std::vector<uint8_t> all(256);
  for (int i = 0; i < 256; ++i) all[i] = static_cast<uint8_t>(i);
  std::vector<float> back(256);
  EXPECT(mx_e4m3_to_f32(all.data(), back.data(), 256, MX_FP8_E4M3_OCP) == MX_OK);
  EXPECT(mx_e4m3_to_f32(all.data(), back.data(), 256, MX_FP8_E4M3_FNUZ) == MX_OK);
  EXPECT(mx_e4m3_to_f32(all.data(), back.data(), 256, 7) == MX_ERR_INVALID_ARG);
  EXPECT(mx_e8m0_to_f32(all.data(), back.data(), 256) == MX_OK);
  std::vector<float> pw;
  for (int e = -150; e <= 130; ++e) pw.push_back(std::ldexp(1.0f, e));
  pw.push_back(0.0f); pw.push_back(-1.0f); pw.push_back(3.0f); pw.push_back(NAN); pw.push_back(INFINITY);
  std::vector<uint8_t> eb(pw.size());
  EXPECT(mx_f32_pow2_to_e8m0(pw.data(), eb.data(), static_cast<int64_t>(pw.size())) == MX_ERR_NOT_LOSSLESS);
  EXPECT(mx_f32_pow2_to_e8m0(pw.data() + 23, eb.data(), 255) == MX_OK);        // 2^-127 .. 2^127
  for (int s = -1; s <= 6; ++s) EXPECT(std::strlen(mx_status_string(s)) > 0);

  // ---- dry-run validation of every device entry point
  mx_set_dry_run(1);
  alignas(64) static unsigned char dummy[1 << 16];
  void* P = dummy;
  const int64_t* pos = reinterpret_cast<const int64_t*>(dummy);
  EXPECT(mx_inv_rope_group_quant(P, pos, P, P, 100, 16, 4, 128, 64, 0, 128, 0, dummy, dummy, nullptr) == MX_OK);
  EXPECT(mx_inv_rope_group_quant(P, pos, P, P, 100, 16, 4, 128, 63, 0, 128, 0, dummy, dummy, nullptr) ==
         MX_ERR_INVALID_ARG);
  EXPECT(mx_inv_rope_group_quant(dummy + 1, pos, P, P, 100, 16, 4, 128, 64, 0, 128, 0, dummy, dummy, nullptr) ==
         MX_ERR_INVALID_ARG);
  EXPECT(std::strlen(mx_last_error()) > 0);
  EXPECT(mx_bmm_a8w8_mxscale(dummy, dummy, 0, dummy, dummy, P, 16, 2, 128, 256, nullptr) == MX_OK);
  EXPECT(mx_bmm_a8w8_mxscale(dummy, dummy, 0, dummy, dummy, P, 16, 2, 128, 200, nullptr) == MX_ERR_INVALID_ARG);
  EXPECT(mx_wo_a_fused(P, pos, P, P, 100, 16, 4, 128, 64, 0, dummy, dummy, P, 2, 128, nullptr) == MX_OK);
  EXPECT(mx_wo_a_fused(P, pos, P, P, 100, 16, 4, 128, 128, 0, dummy, dummy, P, 2, 128, nullptr) ==
         MX_ERR_UNSUPPORTED);
  EXPECT(mx_inv_rope_bf16(P, pos, P, P, 100, 16, 4, 128, 64, 0, dummy + 32768, nullptr) == MX_OK);
  EXPECT(mx_bmm_bf16(P, P, P, 16, 2, 128, 256, nullptr) == MX_OK);
  EXPECT(mx_dequant_mxfp8_to_bf16(dummy, dummy, P, 64, 576, 32, nullptr) == MX_OK);
  EXPECT(mx_dequant_mxfp8_to_bf16(dummy, dummy, P, 64, 576, 128, nullptr) == MX_ERR_INVALID_ARG);
  const size_t ws = mx_linear_workspace_bytes(64, 4096, 576, 1);
  EXPECT(ws == static_cast<size_t>(4096) * 576 * 2);
  EXPECT(mx_linear(P, 64, 576, P, dummy, 1, 4096, P, P, ws, nullptr) == MX_OK);
  EXPECT(mx_linear(P, 64, 576, P, dummy, 1, 4096, P, P, ws - 1, nullptr) == MX_ERR_INVALID_ARG);
  EXPECT(mx_linear(P, 8192, 2304, P, dummy, 1, 5120, P, P, mx_linear_workspace_bytes(8192, 5120, 2304, 1),
                   nullptr) == MX_OK);
  EXPECT(mx_linear(P, 1, int64_t(1) << 31, P, dummy, 2, 16, P, nullptr, 0, nullptr) == MX_ERR_INVALID_ARG);
  EXPECT(mx_linear_noalloc(P, 64, 1152, P, dummy, 1, 4096, P, nullptr) == MX_OK);
  EXPECT(mx_linear_noalloc(P, 1, 1056, P, dummy, 1, 16384, P, nullptr) == MX_ERR_INVALID_ARG);
  EXPECT(mx_stream_read(P, 1 << 20, reinterpret_cast<uint32_t*>(dummy), nullptr) == MX_OK);
  EXPECT(mx_stream_read(P, 24, reinterpret_cast<uint32_t*>(dummy), nullptr) == MX_ERR_INVALID_ARG);
  EXPECT(mx_woa_expand_scales(dummy, 0, 128, 2, 256, 512, dummy, nullptr, nullptr) == MX_OK);
  EXPECT(mx_woa_expand_scales(dummy, 1, 7, 2, 256, 512, dummy, nullptr, nullptr) == MX_ERR_INVALID_ARG);
  EXPECT(mx_f32_pow2_to_e8m0_device(reinterpret_cast<const float*>(dummy), dummy, 16, nullptr, nullptr) == MX_OK);
  EXPECT(mx_f32_to_e4m3_device(reinterpret_cast<const float*>(dummy), dummy, 16, 0, nullptr) == MX_OK);
  uint64_t counters[MX_NUM_COUNTERS + 4];
  EXPECT(mx_get_counters(counters, MX_NUM_COUNTERS + 4) == MX_NUM_COUNTERS);
  mx_set_dry_run(0);
  if (failures) return 1;
  std::printf("host driver: all checks passed\n");
  return 0;
}
