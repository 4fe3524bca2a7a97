// C ABI of libmxfp8: argument validation, the gfx950 probe, status and error
// text, launch counters, and dispatch to the kernels.  Every entry point
// checks its arguments before touching the GPU and never throws.
#include <algorithm>
#include <atomic>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>

#include "common.hpp"

namespace mx {

mx_status launch_quant(const void* x, const int64_t* positions, const void* cos, const void* sin, int64_t max_pos,
                       int64_t T, int32_t H, int32_t D, int32_t rope_dim, int32_t style, int32_t group, int32_t fmt,
                       uint8_t* q, uint8_t* scale, hipStream_t stream);
mx_status launch_bmm(const uint8_t* a, const uint8_t* sa, int32_t a_fmt, const uint8_t* w, const uint8_t* sw,
                     void* out, int64_t T, int32_t G, int32_t N, int32_t K, hipStream_t stream);
mx_status launch_gemm_mx32(const uint8_t* xq, const uint8_t* xs, const uint8_t* w, const uint8_t* sw, void* out,
                           int64_t M, int64_t N, int64_t K, hipStream_t stream);
bool launch_linear_mx32_fused(const void* x, const uint8_t* w, const uint8_t* sw, void* out, int64_t M, int64_t N,
                              int64_t K, hipStream_t stream, mx_status* st);
bool launch_gemm_mx32_wres(const uint8_t* xq, const uint8_t* xs, const uint8_t* w, const uint8_t* sw, void* out,
                           int64_t M, int64_t N, int64_t K, hipStream_t stream, mx_status* st);
mx_status launch_gemm_bf16(const void* x, const void* w, void* out, int64_t M, int64_t N, int64_t K,
                           hipStream_t stream);
mx_status launch_dequant(const uint8_t* w, const uint8_t* w_scale, void* out, int64_t N, int64_t K, int32_t block,
                         hipStream_t stream);
mx_status launch_f32_to_e8m0(const float* in, uint8_t* out, int64_t n, int32_t* reject_count, hipStream_t stream);
mx_status launch_f32_to_e4m3(const float* in, uint8_t* out, int64_t n, int32_t fmt, hipStream_t stream);
mx_status launch_rope_bf16(const void* x, const int64_t* positions, const void* cos, const void* sin,
                           int64_t max_pos, int64_t T, int32_t H, int32_t D, int32_t rope_dim, int32_t style,
                           void* out, hipStream_t stream);
mx_status launch_bmm_bf16(const void* x, const void* w, void* out, int64_t T, int32_t G, int32_t N, int32_t K,
                          hipStream_t stream);
mx_status launch_expand_scales(const void* in, int32_t kind, int32_t block_n, int32_t G, int32_t N, int32_t K,
                               uint8_t* out, int32_t* reject_count, hipStream_t stream);
mx_status launch_stream_read(const void* src, int64_t bytes, uint32_t* sink, hipStream_t stream);
mx_status launch_woa_fused(const void* x, const int64_t* positions, const void* cos, const void* sin,
                           int64_t max_pos, int64_t T, int32_t H, int32_t D, int32_t rope_dim, int32_t style,
                           const uint8_t* w, const uint8_t* w_scale, void* out, int32_t G, int32_t N,
                           hipStream_t stream);

namespace {

thread_local char g_err[512] = "";
std::atomic<int> g_dry_run{0};
std::atomic<uint64_t> g_counters[MX_NUM_COUNTERS];

constexpr int kMaxDevices = 64;
std::atomic<int> g_probe[kMaxDevices];   // 0 unknown, 1 ok, 2 unsupported
std::once_flag g_log_once[kMaxDevices];

bool log_enabled() {
  const char* v = std::getenv("MX_LOG");
  return v && v[0] == '1';
}

}  // namespace

mx_status fail(mx_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return st;
}

void clear_error() { g_err[0] = 0; }
bool dry_run() { return g_dry_run.load(std::memory_order_relaxed) != 0; }
void count(Counter c) { g_counters[c].fetch_add(1, std::memory_order_relaxed); }

mx_status launch_status(const char* what) {
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(MX_ERR_HIP, "%s: launch failed: %s", what, hipGetErrorString(e));
  return MX_OK;
}

static std::atomic<int> g_cus[kMaxDevices];

int device_cu_count() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 0;
  return g_cus[dev].load(std::memory_order_relaxed);
}

static mx_status probe_device(int dev) {
  if (dev < 0 || dev >= kMaxDevices) return fail(MX_ERR_INVALID_ARG, "mx_probe: device %d out of range", dev);
  int state = g_probe[dev].load(std::memory_order_acquire);
  char arch[64] = "";
  if (state == 0) {
    hipDeviceProp_t prop;
    const hipError_t e = hipGetDeviceProperties(&prop, dev);
    if (e != hipSuccess) {
      std::snprintf(arch, sizeof(arch), "(no device: %s)", hipGetErrorString(e));
      state = 2;
    } else {
      std::snprintf(arch, sizeof(arch), "%s", prop.gcnArchName);
      state = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
      g_cus[dev].store(prop.multiProcessorCount, std::memory_order_relaxed);
    }
    g_probe[dev].store(state, std::memory_order_release);
    if (log_enabled()) {
      std::call_once(g_log_once[dev], [&] {
        std::fprintf(stderr, "[mxfp8] device %d arch %s: %s\n", dev, arch,
                     state == 1 ? "FP8 wo_a path enabled" : "unsupported, callers fall back");
      });
    }
  }
  if (state != 1) return fail(MX_ERR_UNSUPPORTED, "device %d is not a gfx950 GPU (or no HIP device is present)", dev);
  return MX_OK;
}

mx_status require_gfx950() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) {
    (void)hipGetLastError();
    return fail(MX_ERR_UNSUPPORTED, "no HIP device is present");
  }
  return probe_device(dev);
}

}  // namespace mx

using namespace mx;

#define MX_CHECK(cond, ...)                                       \
  do {                                                            \
    if (!(cond)) return fail(MX_ERR_INVALID_ARG, __VA_ARGS__);    \
  } while (0)

// Validation done, dry-run honoured, device checked: the common preamble.
#define MX_PREAMBLE()                                   \
  do {                                                  \
    if (dry_run()) { clear_error(); return MX_OK; }     \
    const mx_status st_ = require_gfx950();             \
    if (st_ != MX_OK) return st_;                       \
  } while (0)

extern "C" {

const char* mx_status_string(int s) {
  switch (s) {
    case MX_OK: return "MX_OK";
    case MX_ERR_INVALID_ARG: return "MX_ERR_INVALID_ARG";
    case MX_ERR_UNSUPPORTED: return "MX_ERR_UNSUPPORTED";
    case MX_ERR_NOT_LOSSLESS: return "MX_ERR_NOT_LOSSLESS";
    case MX_ERR_HIP: return "MX_ERR_HIP";
    default: return "MX_ERR_UNKNOWN";
  }
}

const char* mx_last_error(void) { return g_err; }
const char* mx_version(void) { return "mxfp8 0.1 (gfx950)"; }
void mx_set_dry_run(int on) { g_dry_run.store(on ? 1 : 0); }

mx_status mx_probe(int device) {
  const mx_status st = probe_device(device);
  if (st == MX_OK) clear_error();
  return st;
}

int mx_get_counters(uint64_t* out, int n) {
  for (int i = 0; out && i < std::min(n, MX_NUM_COUNTERS); ++i) out[i] = g_counters[i].load();
  return MX_NUM_COUNTERS;
}

void mx_reset_counters(void) {
  for (auto& c : g_counters) c.store(0);
}

mx_status mx_inv_rope_group_quant(const void* x, const int64_t* positions, const void* cos, const void* sin,
                                  int64_t max_pos, int64_t T, int32_t H, int32_t D, int32_t rope_dim,
                                  int32_t rope_style, int32_t group, int32_t fmt, uint8_t* q, uint8_t* scale,
                                  void* stream) {
  const char* fn = "mx_inv_rope_group_quant";
  MX_CHECK(T >= 0, "%s: T = %lld < 0", fn, (long long)T);
  MX_CHECK(H > 0 && D > 0, "%s: H = %d and D = %d must be positive", fn, H, D);
  MX_CHECK(D % 8 == 0, "%s: D = %d must be a multiple of 8", fn, D);
  MX_CHECK(group == 128 || group == 32, "%s: group = %d (128 or 32)", fn, group);
  const int64_t L = static_cast<int64_t>(H) * D;
  MX_CHECK(L % group == 0, "%s: H*D = %lld is not a multiple of the group %d", fn, (long long)L, group);
  MX_CHECK(L / 8 < (int64_t(1) << 30), "%s: H*D = %lld is too large", fn, (long long)L);
  MX_CHECK(rope_dim >= 0 && rope_dim <= D && rope_dim % 16 == 0, "%s: rope_dim = %d (multiple of 16, <= D = %d)",
           fn, rope_dim, D);
  MX_CHECK(rope_style == MX_ROPE_INTERLEAVED || rope_style == MX_ROPE_NEOX, "%s: unknown rope style %d", fn,
           rope_style);
  MX_CHECK(fmt == MX_FP8_E4M3_OCP || fmt == MX_FP8_E4M3_FNUZ, "%s: unknown FP8 format %d", fn, fmt);
  if (T == 0) { clear_error(); return MX_OK; }
  MX_CHECK(x && q && scale, "%s: null tensor pointer", fn);
  MX_CHECK(aligned(x, 16) && aligned(q, 16), "%s: x and q must be 16-byte aligned", fn);
  if (rope_dim > 0) {
    MX_CHECK(positions && cos && sin, "%s: rope_dim > 0 needs positions, cos and sin", fn);
    MX_CHECK(max_pos >= 1, "%s: max_pos = %lld", fn, (long long)max_pos);
    const uintptr_t ta = rope_style == MX_ROPE_NEOX ? 16 : 8;
    MX_CHECK(aligned(cos, ta) && aligned(sin, ta) && aligned(positions, 8), "%s: cos/sin must be %d-byte aligned",
             fn, (int)ta);
  }
  MX_PREAMBLE();
  count(C_QUANT);
  const mx_status st = launch_quant(x, positions, cos, sin, max_pos, T, H, D, rope_dim, rope_style, group, fmt, q,
                                    scale, static_cast<hipStream_t>(stream));
  if (st == MX_OK) clear_error();
  return st;
}

mx_status mx_bmm_a8w8_mxscale(const uint8_t* a, const uint8_t* a_scale, int32_t a_fmt, const uint8_t* w,
                              const uint8_t* w_scale, void* out, int64_t T, int32_t G, int32_t N, int32_t K,
                              void* stream) {
  const char* fn = "mx_bmm_a8w8_mxscale";
  MX_CHECK(T >= 0 && T < (int64_t(1) << 31), "%s: T = %lld out of range", fn, (long long)T);
  MX_CHECK(G >= 1 && N >= 1 && K >= 1, "%s: G = %d, N = %d, K = %d must be positive", fn, G, N, K);
  MX_CHECK(K % MX_WOA_GROUP == 0, "%s: K = %d is not a multiple of 128 (group-128 layout required)", fn, K);
  MX_CHECK(N % 16 == 0, "%s: N = %d is not a multiple of 16", fn, N);
  MX_CHECK(static_cast<int64_t>(G) * K < (int64_t(1) << 31) && static_cast<int64_t>(N) * K < (int64_t(1) << 31),
           "%s: G*K or N*K too large", fn);
  MX_CHECK(static_cast<int64_t>(256) * G * K < (int64_t(1) << 32), "%s: G*K too large for 32-bit tile offsets",
           fn);
  MX_CHECK(a_fmt == MX_FP8_E4M3_OCP || a_fmt == MX_FP8_E4M3_FNUZ, "%s: unknown FP8 format %d", fn, a_fmt);
  if (T == 0) { clear_error(); return MX_OK; }
  MX_CHECK(a && a_scale && w && w_scale && out, "%s: null tensor pointer", fn);
  MX_CHECK(aligned(a, 16) && aligned(w, 16), "%s: a and w must be 16-byte aligned", fn);
  MX_CHECK(aligned(out, 16), "%s: out must be 16-byte aligned", fn);
  MX_PREAMBLE();
  const mx_status st = launch_bmm(a, a_scale, a_fmt, w, w_scale, out, T, G, N, K, static_cast<hipStream_t>(stream));
  if (st == MX_OK) clear_error();
  return st;
}

mx_status mx_wo_a_fused(const void* x, const int64_t* positions, const void* cos, const void* sin, int64_t max_pos,
                        int64_t T, int32_t H, int32_t D, int32_t rope_dim, int32_t rope_style, const uint8_t* w,
                        const uint8_t* w_scale, void* out, int32_t G, int32_t N, void* stream) {
  const char* fn = "mx_wo_a_fused";
  MX_CHECK(T >= 0 && T < (int64_t(1) << 31), "%s: T = %lld out of range", fn, (long long)T);
  MX_CHECK(H > 0 && D > 0 && G >= 1 && N >= 1, "%s: H = %d, D = %d, G = %d, N = %d must be positive", fn, H, D, G,
           N);
  const int64_t L = static_cast<int64_t>(H) * D;
  MX_CHECK(L % G == 0, "%s: H*D = %lld is not a multiple of G = %d", fn, (long long)L, G);
  MX_CHECK(L < (int64_t(1) << 23), "%s: H*D = %lld is too large", fn, (long long)L);
  const int64_t K = L / G;
  MX_CHECK(K % MX_WOA_GROUP == 0, "%s: K = %lld is not a multiple of 128", fn, (long long)K);
  MX_CHECK(N % 16 == 0, "%s: N = %d is not a multiple of 16", fn, N);
  MX_CHECK(rope_dim >= 0 && rope_dim <= D && rope_dim % 16 == 0, "%s: rope_dim = %d (multiple of 16, <= D = %d)",
           fn, rope_dim, D);
  MX_CHECK(rope_style == MX_ROPE_INTERLEAVED || rope_style == MX_ROPE_NEOX, "%s: unknown rope style %d", fn,
           rope_style);
  // shapes the one-kernel path does not take: the two calls serve them
  if (K > 4096 || D % 128 != 0 || rope_dim > 64 ||
      (rope_style == MX_ROPE_NEOX && rope_dim > 0 && (rope_dim & (rope_dim - 1)) != 0) ||
      (rope_dim > 0 && max_pos > (int64_t(0x7FFFFFFF) / rope_dim)))
    return fail(MX_ERR_UNSUPPORTED,
                "%s: K = %lld, D = %d, rope_dim = %d (style %d), max_pos = %lld not served in one kernel; use "
                "mx_inv_rope_group_quant then mx_bmm_a8w8_mxscale",
                fn, (long long)K, D, rope_dim, rope_style, (long long)max_pos);
  if (T == 0) { clear_error(); return MX_OK; }
  MX_CHECK(x && w && w_scale && out, "%s: null tensor pointer", fn);
  MX_CHECK(aligned(x, 16) && aligned(w, 16) && aligned(out, 16), "%s: x, w and out must be 16-byte aligned", fn);
  if (rope_dim > 0) {
    MX_CHECK(positions && cos && sin, "%s: rope_dim > 0 needs positions, cos and sin", fn);
    MX_CHECK(max_pos >= 1, "%s: max_pos = %lld", fn, (long long)max_pos);
    // the table rows are read in 16-byte pieces
    MX_CHECK(aligned(cos, 16) && aligned(sin, 16) && aligned(positions, 8),
             "%s: cos/sin must be 16-byte aligned, positions 8-byte aligned", fn);
  }
  MX_PREAMBLE();
  count(C_WOA_FUSED);
  const mx_status st = launch_woa_fused(x, positions, cos, sin, max_pos, T, H, D, rope_dim, rope_style, w, w_scale,
                                        out, G, N, static_cast<hipStream_t>(stream));
  if (st == MX_OK) clear_error();
  return st;
}

mx_status mx_inv_rope_bf16(const void* x, const int64_t* positions, const void* cos, const void* sin,
                           int64_t max_pos, int64_t T, int32_t H, int32_t D, int32_t rope_dim, int32_t rope_style,
                           void* out, void* stream) {
  const char* fn = "mx_inv_rope_bf16";
  MX_CHECK(T >= 0, "%s: T = %lld < 0", fn, (long long)T);
  MX_CHECK(H > 0 && D > 0, "%s: H = %d and D = %d must be positive", fn, H, D);
  MX_CHECK(D % 8 == 0, "%s: D = %d must be a multiple of 8", fn, D);
  const int64_t L = static_cast<int64_t>(H) * D;
  MX_CHECK(L / 8 < (int64_t(1) << 30), "%s: H*D = %lld is too large", fn, (long long)L);
  MX_CHECK(rope_dim >= 0 && rope_dim <= D && rope_dim % 16 == 0, "%s: rope_dim = %d (multiple of 16, <= D = %d)",
           fn, rope_dim, D);
  MX_CHECK(rope_style == MX_ROPE_INTERLEAVED || rope_style == MX_ROPE_NEOX, "%s: unknown rope style %d", fn,
           rope_style);
  if (T == 0) { clear_error(); return MX_OK; }
  MX_CHECK(x && out, "%s: null tensor pointer", fn);
  MX_CHECK(aligned(x, 16) && aligned(out, 16), "%s: x and out must be 16-byte aligned", fn);
  const uintptr_t xb = reinterpret_cast<uintptr_t>(x), ob = reinterpret_cast<uintptr_t>(out);
  const uintptr_t bytes = static_cast<uintptr_t>(T * L * 2);
  MX_CHECK(xb == ob || xb + bytes <= ob || ob + bytes <= xb, "%s: out overlaps x without being x", fn);
  if (rope_dim > 0) {
    MX_CHECK(positions && cos && sin, "%s: rope_dim > 0 needs positions, cos and sin", fn);
    MX_CHECK(max_pos >= 1, "%s: max_pos = %lld", fn, (long long)max_pos);
    MX_CHECK(aligned(cos, 16) && aligned(sin, 16) && aligned(positions, 8),
             "%s: cos/sin must be 16-byte aligned, positions 8-byte aligned", fn);
  }
  MX_PREAMBLE();
  count(C_ROPE_BF16);
  const mx_status st = launch_rope_bf16(x, positions, cos, sin, max_pos, T, H, D, rope_dim, rope_style, out,
                                        static_cast<hipStream_t>(stream));
  if (st == MX_OK) clear_error();
  return st;
}

mx_status mx_bmm_bf16(const void* x, const void* w, void* out, int64_t T, int32_t G, int32_t N, int32_t K,
                      void* stream) {
  const char* fn = "mx_bmm_bf16";
  MX_CHECK(T >= 0 && T < (int64_t(1) << 31), "%s: T = %lld out of range", fn, (long long)T);
  MX_CHECK(G >= 1 && N >= 1 && K >= 1, "%s: G = %d, N = %d, K = %d must be positive", fn, G, N, K);
  MX_CHECK(K % 128 == 0, "%s: K = %d is not a multiple of 128", fn, K);
  MX_CHECK(N % 16 == 0, "%s: N = %d is not a multiple of 16", fn, N);
  MX_CHECK(static_cast<int64_t>(256) * G * K * 2 < (int64_t(1) << 32) &&
               static_cast<int64_t>(N) * K < (int64_t(1) << 31),
           "%s: G*K or N*K too large for 32-bit tile offsets", fn);
  if (T == 0) { clear_error(); return MX_OK; }
  MX_CHECK(x && w && out, "%s: null tensor pointer", fn);
  MX_CHECK(aligned(x, 16) && aligned(w, 16) && aligned(out, 16), "%s: x, w and out must be 16-byte aligned", fn);
  MX_PREAMBLE();
  const mx_status st = launch_bmm_bf16(x, w, out, T, G, N, K, static_cast<hipStream_t>(stream));
  if (st == MX_OK) clear_error();
  return st;
}

mx_status mx_dequant_mxfp8_to_bf16(const uint8_t* w, const uint8_t* w_scale, void* out, int64_t N, int64_t K,
                                   int32_t block, void* stream) {
  const char* fn = "mx_dequant_mxfp8_to_bf16";
  MX_CHECK(N >= 0 && K >= 0, "%s: N = %lld, K = %lld", fn, (long long)N, (long long)K);
  MX_CHECK(block == 32 || block == 128, "%s: block = %d (32 or 128)", fn, block);
  MX_CHECK(K % block == 0, "%s: K = %lld is not a multiple of the block %d", fn, (long long)K, block);
  if (N == 0 || K == 0) { clear_error(); return MX_OK; }
  MX_CHECK(w && w_scale && out, "%s: null tensor pointer", fn);
  MX_CHECK(aligned(w, 16) && aligned(out, 16), "%s: w and out must be 16-byte aligned", fn);
  MX_PREAMBLE();
  count(C_DEQUANT);
  const mx_status st = launch_dequant(w, w_scale, out, N, K, block, static_cast<hipStream_t>(stream));
  if (st == MX_OK) clear_error();
  return st;
}

mx_status mx_stream_read(const void* src, int64_t bytes, uint32_t* sink, void* stream) {
  const char* fn = "mx_stream_read";
  MX_CHECK(bytes >= 0 && bytes % 16 == 0, "%s: bytes = %lld is not a non-negative multiple of 16", fn,
           (long long)bytes);
  if (bytes == 0) { clear_error(); return MX_OK; }
  MX_CHECK(src && sink, "%s: null pointer", fn);
  MX_CHECK(aligned(src, 16) && aligned(sink, 4), "%s: src must be 16-byte and sink 4-byte aligned", fn);
  MX_PREAMBLE();
  const mx_status st = launch_stream_read(src, bytes, sink, static_cast<hipStream_t>(stream));
  if (st == MX_OK) clear_error();
  return st;
}

int mx_linear_dequant_at_load(int64_t K) { return K % MX_LINEAR_K_ALIGN != 0 ? 1 : 0; }

size_t mx_linear_workspace_bytes(int64_t M, int64_t N, int64_t K, int32_t w_elem_bytes) {
  if (M < 0 || N < 0 || K <= 0 || K % MX_LINEAR_BLOCK != 0) return 0;
  if (w_elem_bytes == 2) return 0;
  if (K % MX_LINEAR_K_ALIGN != 0) return static_cast<size_t>(N) * K * 2;
  // x codes [M, K] then x scales [M, K/32], the scales 16-byte aligned
  const size_t codes = (static_cast<size_t>(M) * K + 15) / 16 * 16;
  return codes + static_cast<size_t>(M) * (K / MX_LINEAR_BLOCK);
}

}  // extern "C"

namespace {

// Argument checks shared by mx_linear and mx_linear_noalloc (everything but
// the workspace).
mx_status linear_check(const char* fn, const void* x, int64_t M, int64_t K, const void* w, const uint8_t* w_scale,
                       int32_t w_elem_bytes, int64_t N, void* out) {
  MX_CHECK(M >= 0 && N >= 0 && K > 0, "%s: M = %lld, N = %lld, K = %lld", fn, (long long)M, (long long)N,
           (long long)K);
  MX_CHECK(K % MX_LINEAR_BLOCK == 0, "%s: K = %lld is not a multiple of %d", fn, (long long)K, MX_LINEAR_BLOCK);
  MX_CHECK(N % 16 == 0, "%s: N = %lld is not a multiple of 16", fn, (long long)N);
  MX_CHECK(w_elem_bytes == 1 || w_elem_bytes == 2, "%s: w_elem_bytes = %d (1 = FP8, 2 = BF16)", fn, w_elem_bytes);
  // the kernels index K, M*K, N*K and M*N with 32-bit and 40-bit offsets,
  // and take N as a 32-bit value
  MX_CHECK(M <= (int64_t(1) << 30) && N < (int64_t(1) << 31) && K < (int64_t(1) << 31) &&
               N * K < (int64_t(1) << 40) && M * K < (int64_t(1) << 40) && M * N < (int64_t(1) << 40),
           "%s: shape too large (M = %lld, N = %lld, K = %lld)", fn, (long long)M, (long long)N, (long long)K);
  if (M == 0 || N == 0) return MX_OK;
  MX_CHECK(x && w && out, "%s: null tensor pointer", fn);
  MX_CHECK(w_elem_bytes == 2 || w_scale, "%s: an FP8 weight needs w_scale", fn);
  MX_CHECK(aligned(x, 16) && aligned(w, 16) && aligned(out, 8), "%s: x and w must be 16-byte aligned", fn);
  return MX_OK;
}

// The three branches of the linear, on a checked call; `workspace` holds at
// least mx_linear_workspace_bytes(M, N, K, w_elem_bytes), 16-byte aligned.
mx_status linear_run(const void* x, int64_t M, int64_t K, const void* w, const uint8_t* w_scale,
                     int32_t w_elem_bytes, int64_t N, void* out, void* workspace, hipStream_t s) {
  mx_status st;
  if (w_elem_bytes == 2) {
    // weight already BF16 (dequantised once at load)
    count(C_LINEAR_BF16);
    st = launch_gemm_bf16(x, w, out, M, N, K, s);
  } else if (K % MX_LINEAR_K_ALIGN == 0) {
    // x -> MXFP8 (OCP, block 32, no rotation) into the workspace, then the
    // block-scaled FP8 GEMM (up to 16 rows and K <= 4096 both in one kernel)
    count(C_LINEAR_FP8);
    const uint8_t* w8 = static_cast<const uint8_t*>(w);
    if (M > 16 || !launch_linear_mx32_fused(x, w8, w_scale, out, M, N, K, s, &st)) {
      uint8_t* xq = static_cast<uint8_t*>(workspace);
      uint8_t* xs = xq + (static_cast<size_t>(M) * K + 15) / 16 * 16;
      st = launch_quant(x, nullptr, nullptr, nullptr, 0, M, 1, static_cast<int32_t>(K), 0, MX_ROPE_INTERLEAVED,
                        MX_LINEAR_BLOCK, MX_FP8_E4M3_OCP, xq, xs, s);
      if (st == MX_OK && (M > 64 || !launch_gemm_mx32_wres(xq, xs, w8, w_scale, out, M, N, K, s, &st)))
        st = launch_gemm_mx32(xq, xs, w8, w_scale, out, M, N, K, s);
    }
  } else {
    // an FP8 weight with K % 128 != 0 that was not prepared at load: dequantise
    // it into the workspace on this call; it never reaches the scaled GEMM
    count(C_LINEAR_PERCALL);
    st = launch_dequant(static_cast<const uint8_t*>(w), w_scale, workspace, N, K, MX_LINEAR_BLOCK, s);
    if (st == MX_OK) st = launch_gemm_bf16(x, workspace, out, M, N, K, s);
  }
  return st;
}

// Scratch of mx_linear_noalloc: one copy per GPU, in the code object, held
// until the process ends.  In host code `scratch` names a host-side stand-in,
// not the device array; its device address comes from hipGetSymbolAddress,
// once per device (scratch_on_current_device).
constexpr size_t kScratchBytes = size_t(MX_LINEAR_NOALLOC_SCRATCH_BYTES);
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

mx_status scratch_on_current_device(void** ptr) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) {
    (void)hipGetLastError();
    return fail(MX_ERR_UNSUPPORTED, "no HIP device is present");
  }
  if (dev < 0 || dev >= kMaxDevices) return fail(MX_ERR_INVALID_ARG, "device %d out of range", dev);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(MX_ERR_HIP, "mx_linear_noalloc: hipGetSymbolAddress of the scratch array failed on device %d: %s",
                  dev, hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return MX_OK;
}

}  // namespace

extern "C" {

mx_status mx_linear(const void* x, int64_t M, int64_t K, const void* w, const uint8_t* w_scale, int32_t w_elem_bytes,
                    int64_t N, void* out, void* workspace, size_t workspace_bytes, void* stream) {
  const char* fn = "mx_linear";
  mx_status st = linear_check(fn, x, M, K, w, w_scale, w_elem_bytes, N, out);
  if (st != MX_OK) return st;
  if (M == 0 || N == 0) { clear_error(); return MX_OK; }
  const size_t need = mx_linear_workspace_bytes(M, N, K, w_elem_bytes);
  MX_CHECK(need == 0 || (workspace && workspace_bytes >= need && aligned(workspace, 16)),
           "%s: this call needs a 16-byte aligned workspace of %zu bytes (got %zu)", fn, need, workspace_bytes);
  MX_PREAMBLE();
  st = linear_run(x, M, K, w, w_scale, w_elem_bytes, N, out, workspace, static_cast<hipStream_t>(stream));
  if (st == MX_OK) clear_error();
  return st;
}

mx_status mx_linear_noalloc(const void* x, int64_t M, int64_t K, const void* w, const uint8_t* w_scale,
                            int32_t w_elem_bytes, int64_t N, void* out, void* stream) {
  const char* fn = "mx_linear_noalloc";
  mx_status st = linear_check(fn, x, M, K, w, w_scale, w_elem_bytes, N, out);
  if (st != MX_OK) return st;
  if (M == 0 || N == 0) { clear_error(); return MX_OK; }
  const size_t need = mx_linear_workspace_bytes(M, N, K, w_elem_bytes);
  if (need > kScratchBytes)
    return fail(MX_ERR_INVALID_ARG,
                "%s: this call needs %zu bytes of scratch, more than the library's %zu (M = %lld, N = %lld, "
                "K = %lld); use mx_linear with a workspace",
                fn, need, kScratchBytes, (long long)M, (long long)N, (long long)K);
  MX_PREAMBLE();
  void* ws = nullptr;
  if (need) {
    st = scratch_on_current_device(&ws);
    if (st != MX_OK) return st;
  }
  st = linear_run(x, M, K, w, w_scale, w_elem_bytes, N, out, ws, static_cast<hipStream_t>(stream));
  if (st == MX_OK) clear_error();
  return st;
}

mx_status mx_woa_expand_scales(const void* scale, int32_t scale_kind, int32_t block_n, int32_t G, int32_t N,
                               int32_t K, uint8_t* out, int32_t* reject_count, void* stream) {
  const char* fn = "mx_woa_expand_scales";
  MX_CHECK(scale_kind == MX_SCALE_E8M0 || scale_kind == MX_SCALE_F32, "%s: unknown scale kind %d", fn, scale_kind);
  MX_CHECK(block_n == 1 || block_n == 128, "%s: block_n = %d (1 or 128)", fn, block_n);
  MX_CHECK(G >= 1 && N >= 1 && K >= 128, "%s: G = %d, N = %d, K = %d", fn, G, N, K);
  MX_CHECK(K % MX_WOA_GROUP == 0, "%s: K = %d is not a multiple of 128 (group-128 layout required)", fn, K);
  MX_CHECK(static_cast<int64_t>(G) * N * (K / 128) < (int64_t(1) << 31), "%s: G*N*K/128 too large", fn);
  MX_CHECK(scale && out, "%s: null pointer", fn);
  MX_CHECK(scale_kind == MX_SCALE_E8M0 || aligned(scale, 4), "%s: FP32 scales must be 4-byte aligned", fn);
  MX_CHECK(!reject_count || aligned(reject_count, 4), "%s: reject_count must be 4-byte aligned", fn);
  MX_PREAMBLE();
  count(C_EXPAND_SCALES);
  const mx_status st = launch_expand_scales(scale, scale_kind, block_n, G, N, K, out, reject_count,
                                            static_cast<hipStream_t>(stream));
  if (st == MX_OK) clear_error();
  return st;
}

mx_status mx_f32_pow2_to_e8m0_device(const float* in, uint8_t* out, int64_t n, int32_t* reject_count, void* stream) {
  const char* fn = "mx_f32_pow2_to_e8m0_device";
  MX_CHECK(n >= 0, "%s: n = %lld", fn, (long long)n);
  if (n == 0) { clear_error(); return MX_OK; }
  MX_CHECK(in && out, "%s: null pointer", fn);
  MX_CHECK(aligned(in, 4), "%s: in must be 4-byte aligned", fn);
  MX_PREAMBLE();
  count(C_E8M0_DEVICE);
  const mx_status st = launch_f32_to_e8m0(in, out, n, reject_count, static_cast<hipStream_t>(stream));
  if (st == MX_OK) clear_error();
  return st;
}

mx_status mx_f32_to_e4m3_device(const float* in, uint8_t* out, int64_t n, int32_t fmt, void* stream) {
  const char* fn = "mx_f32_to_e4m3_device";
  MX_CHECK(n >= 0, "%s: n = %lld", fn, (long long)n);
  MX_CHECK(fmt == MX_FP8_E4M3_OCP || fmt == MX_FP8_E4M3_FNUZ, "%s: unknown FP8 format %d", fn, fmt);
  if (n == 0) { clear_error(); return MX_OK; }
  MX_CHECK(in && out, "%s: null pointer", fn);
  MX_CHECK(aligned(in, 4), "%s: in must be 4-byte aligned", fn);
  MX_PREAMBLE();
  count(C_E4M3_DEVICE);
  const mx_status st = launch_f32_to_e4m3(in, out, n, fmt, static_cast<hipStream_t>(stream));
  if (st == MX_OK) clear_error();
  return st;
}

}  // extern "C"
