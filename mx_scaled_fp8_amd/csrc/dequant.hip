// One-pass MXFP8 -> BF16 weight dequantisation, and the device format
// converters (gfx950).
//
// "[ROCm][DSv4.1][Perf] Dequantize the MXFP8 weight once when dot_scaled
// cannot be used" (Purpose; "Why it is worth a patch"): out[n,k] =
// bf16(decode(w[n,k]) * 2^(s[n,k/block]-127)).  The page's version chains
// pointwise kernels through an FP32 intermediate; here every lane reads 16
// codes (16 bytes) and one scale byte and writes 16 BF16 (32 bytes), so the
// pass moves 1 + 1/block + 2 bytes per element and nothing else.  Each pair
// of codes is one v_cvt_scalef32_pk_bf16_fp8 (product, then nearest-even
// BF16).
#include "common.hpp"

namespace mx {

namespace {

constexpr int kThreads = 256;

typedef __bf16 v2bf __attribute__((ext_vector_type(2)));

// Two OCP codes (low or high 16 bits of `codes`) -> two BF16 = bf16(code * 2^e):
// v_cvt_scalef32_pk_bf16_fp8 reads the E8M0 scale from the FP32 exponent field
// (`sbits`); it was checked exact against the oracle for every code and
// 2^-127 <= 2^e <= 2^120.
template <bool HI_WORD>
__device__ __forceinline__ uint32_t dq_pair(uint32_t codes, float sbits, bool nan_scale) {
  const v2bf r = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(static_cast<int>(codes), sbits, HI_WORD);
  return nan_scale ? 0x7FC07FC0u : __builtin_bit_cast(uint32_t, r);
}

__global__ __launch_bounds__(kThreads) void dequant_kernel(const uint4* __restrict__ w, const uint8_t* __restrict__ sc,
                                                           uint4* __restrict__ out, uint64_t chunks,
                                                           uint32_t chunks_per_block_shift) {
  const uint64_t c = static_cast<uint64_t>(blockIdx.x) * kThreads + threadIdx.x;
  if (c >= chunks) return;
  const uint4 v = w[c];
  const uint32_t s = sc[c >> chunks_per_block_shift];
  const float sbits = __uint_as_float(s << 23);
  const bool nan_scale = s == 0xFFu;
  uint4 o0, o1;
  o0.x = dq_pair<false>(v.x, sbits, nan_scale);
  o0.y = dq_pair<true>(v.x, sbits, nan_scale);
  o0.z = dq_pair<false>(v.y, sbits, nan_scale);
  o0.w = dq_pair<true>(v.y, sbits, nan_scale);
  o1.x = dq_pair<false>(v.z, sbits, nan_scale);
  o1.y = dq_pair<true>(v.z, sbits, nan_scale);
  o1.z = dq_pair<false>(v.w, sbits, nan_scale);
  o1.w = dq_pair<true>(v.w, sbits, nan_scale);
  out[2 * c] = o0;
  out[2 * c + 1] = o1;
}

// FP32 power of two 2^n, -127 <= n <= 127 -> byte n + 127; else 0xFF and counted.
__global__ __launch_bounds__(kThreads) void f32_to_e8m0_kernel(const float* __restrict__ in, uint8_t* __restrict__ out,
                                                               uint64_t n, int32_t* reject_count) {
  const uint64_t i = static_cast<uint64_t>(blockIdx.x) * kThreads + threadIdx.x;
  if (i >= n) return;
  const uint32_t u = __float_as_uint(in[i]);
  const uint32_t ef = (u >> 23) & 0xFFu;
  int b;
  if (u == 0x00400000u) b = 0;
  else if ((u >> 31) != 0 || (u & 0x7FFFFFu) != 0 || ef == 0 || ef == 0xFFu) b = -1;
  else b = static_cast<int>(ef);
  if (b < 0) {
    out[i] = 0xFF;
    if (reject_count) atomicAdd(reject_count, 1);
  } else {
    out[i] = static_cast<uint8_t>(b);
  }
}

// Checkpoint weight scales -> the [G, N, K/128] E8M0 layout the wo_a GEMM
// reads.  Output byte i = (g, n, kb) takes source (g, n / block_n, kb) of a
// [G, ceil(N/block_n), K/128] tensor: E8M0 bytes are copied, FP32 scales go
// through the lossless power-of-two rule above (0xFF where rejected).  A
// rejected source scale is counted once, by the thread of its block's first row.
template <bool F32>
__global__ __launch_bounds__(kThreads) void expand_scales_kernel(const void* __restrict__ in, uint8_t* __restrict__ out,
                                                                 uint32_t total, uint32_t N, uint32_t KB,
                                                                 uint32_t block_n, int32_t* reject_count) {
  const uint32_t i = blockIdx.x * kThreads + threadIdx.x;
  if (i >= total) return;
  const uint32_t row = i / KB;                   // g * N + n
  const uint32_t kb = i - row * KB;
  const uint32_t g = row / N;
  const uint32_t n = row - g * N;
  const uint32_t nb = (N + block_n - 1) / block_n;
  const uint32_t src = (g * nb + n / block_n) * KB + kb;
  if constexpr (!F32) {
    out[i] = static_cast<const uint8_t*>(in)[src];
  } else {
    const uint32_t u = __float_as_uint(static_cast<const float*>(in)[src]);
    const uint32_t ef = (u >> 23) & 0xFFu;
    int b;
    if (u == 0x00400000u) b = 0;
    else if ((u >> 31) != 0 || (u & 0x7FFFFFu) != 0 || ef == 0 || ef == 0xFFu) b = -1;
    else b = static_cast<int>(ef);
    out[i] = b < 0 ? uint8_t(0xFF) : static_cast<uint8_t>(b);
    if (b < 0 && reject_count && n % block_n == 0) atomicAdd(reject_count, 1);
  }
}

// FP32 -> e4m3, nearest even, saturating.  The FNUZ code of v is the OCP
// code of 2v (the FNUZ grid is the OCP grid halved, 224 = 448 / 2) with -0
// mapped to 0x00.
template <int FMT>
__global__ __launch_bounds__(kThreads) void f32_to_e4m3_kernel(const float* __restrict__ in, uint8_t* __restrict__ out,
                                                               uint64_t n) {
  const uint64_t i = static_cast<uint64_t>(blockIdx.x) * kThreads + threadIdx.x;
  if (i >= n) return;
  float v = in[i];
  uint32_t code;
  if (__builtin_isnan(v)) {
    code = FMT == MX_FP8_E4M3_OCP ? 0x7Fu : 0x80u;
  } else {
    if (FMT == MX_FP8_E4M3_FNUZ) v = ldexpf(v, 1);     // exact, or +-Inf
    v = fminf(fmaxf(v, -448.0f), 448.0f);                // saturate (Inf included)
    code = static_cast<uint32_t>(cvt_fp8x2<false>(v, v, 0)) & 0xFFu;
    if (FMT == MX_FP8_E4M3_FNUZ && code == 0x80u) code = 0;
  }
  out[i] = static_cast<uint8_t>(code);
}

}  // namespace

mx_status launch_dequant(const uint8_t* w, const uint8_t* w_scale, void* out, int64_t N, int64_t K, int32_t block,
                         hipStream_t stream) {
  const uint64_t chunks = static_cast<uint64_t>(N) * static_cast<uint64_t>(K) / 16;
  if (chunks == 0) return MX_OK;
  const uint32_t shift = block == 32 ? 1 : 3;   // 16-code chunks per scale block: 2 or 8
  const uint64_t blocks = (chunks + kThreads - 1) / kThreads;
  dequant_kernel<<<static_cast<uint32_t>(blocks), kThreads, 0, stream>>>(
      reinterpret_cast<const uint4*>(w), w_scale, reinterpret_cast<uint4*>(out), chunks, shift);
  return launch_status("mx_dequant_mxfp8_to_bf16");
}

mx_status launch_f32_to_e8m0(const float* in, uint8_t* out, int64_t n, int32_t* reject_count, hipStream_t stream) {
  if (n == 0) return MX_OK;
  const uint64_t blocks = (static_cast<uint64_t>(n) + kThreads - 1) / kThreads;
  f32_to_e8m0_kernel<<<static_cast<uint32_t>(blocks), kThreads, 0, stream>>>(in, out, n, reject_count);
  return launch_status("mx_f32_pow2_to_e8m0_device");
}

mx_status launch_f32_to_e4m3(const float* in, uint8_t* out, int64_t n, int32_t fmt, hipStream_t stream) {
  if (n == 0) return MX_OK;
  const uint64_t blocks = (static_cast<uint64_t>(n) + kThreads - 1) / kThreads;
  if (fmt == MX_FP8_E4M3_OCP)
    f32_to_e4m3_kernel<MX_FP8_E4M3_OCP><<<static_cast<uint32_t>(blocks), kThreads, 0, stream>>>(in, out, n);
  else
    f32_to_e4m3_kernel<MX_FP8_E4M3_FNUZ><<<static_cast<uint32_t>(blocks), kThreads, 0, stream>>>(in, out, n);
  return launch_status("mx_f32_to_e4m3_device");
}

mx_status launch_expand_scales(const void* in, int32_t kind, int32_t block_n, int32_t G, int32_t N, int32_t K,
                               uint8_t* out, int32_t* reject_count, hipStream_t stream) {
  const uint32_t KB = static_cast<uint32_t>(K / 128);
  const uint32_t total = static_cast<uint32_t>(G) * static_cast<uint32_t>(N) * KB;
  if (total == 0) return MX_OK;
  const uint32_t blocks = (total + kThreads - 1) / kThreads;
  if (kind == MX_SCALE_F32)
    expand_scales_kernel<true><<<blocks, kThreads, 0, stream>>>(in, out, total, static_cast<uint32_t>(N), KB,
                                                                static_cast<uint32_t>(block_n), reject_count);
  else
    expand_scales_kernel<false><<<blocks, kThreads, 0, stream>>>(in, out, total, static_cast<uint32_t>(N), KB,
                                                                 static_cast<uint32_t>(block_n), reject_count);
  return launch_status("mx_woa_expand_scales");
}

}  // namespace mx
