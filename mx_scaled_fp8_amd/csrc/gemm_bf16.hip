// BF16 GEMM for the MXFP8 linear's BF16 branch (gfx950): out[M,N] = x[M,K] * W[N,K]^T.
//
// "[ROCm][DSv4.1][Perf] Dequantize the MXFP8 weight once when dot_scaled
// cannot be used", Purpose: when K % 128 != 0 the weight is held in BF16
// (converted once at load) and the linear is a plain BF16 product with fp32
// accumulation, rounded back to BF16.
//
// Decode-sized M (the pages' case is one row per sequence in the batch): one
// workgroup per 64 rows of x and 16*NT columns n; its four waves take
// interleaved 32-wide K-steps on v_mfma_f32_16x16x32_bf16 and reduce their
// partial sums through LDS.  The weight is the MFMA's first operand, so each
// lane ends with four consecutive n of one row (one 8-byte store).  K only
// has to be a multiple of 32 (288 and 576 are not multiples of 128).
//
// The same kernel runs the decode batch of the BF16 wo_a arm: G independent
// products x[:, g, :] * W[g]^T with x rows G*K apart and out rows G*N apart,
// one grid layer per group.
#include "common.hpp"

namespace mx {

namespace {

typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

__device__ __forceinline__ v8bf as_v8bf(const uint4 v) {
  v8bf r;
  __builtin_memcpy(&r, &v, 16);
  return r;
}

template <int NT>
__global__ __launch_bounds__(256) void gemm_bf16_kernel(const uint16_t* __restrict__ x, const uint16_t* __restrict__ w,
                                                        uint16_t* __restrict__ out, int M, int N, int K,
                                                        int n_groups, int64_t ldx, int64_t ldo) {
  __shared__ float red[4][NT * 4][4][64];
  const int n0 = (blockIdx.x % n_groups) * (16 * NT);
  const int m0 = blockIdx.y * 64;
  const int g = blockIdx.z;                 // group: x + g*K, W + g*N*K, out + g*N
  x += static_cast<size_t>(g) * K;
  w += static_cast<size_t>(g) * N * K;
  out += static_cast<size_t>(g) * N;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int KS = K / 32;
  const int kq = (lane >> 4) * 8;           // element offset inside the 32-wide step

  const uint16_t* pw[NT];
#pragma unroll
  for (int i = 0; i < NT; ++i) pw[i] = w + static_cast<size_t>(min(n0 + i * 16 + (lane & 15), N - 1)) * K + kq;
  const uint16_t* px[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) px[j] = x + static_cast<size_t>(min(m0 + j * 16 + (lane & 15), M - 1)) * ldx + kq;

  v4f acc[NT][4];
#pragma unroll
  for (int i = 0; i < NT; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

  for (int ks = wave; ks < KS; ks += 4) {
    const int ko = ks * 32;
    v8bf fw[NT], fx[4];
#pragma unroll
    for (int i = 0; i < NT; ++i) fw[i] = as_v8bf(*reinterpret_cast<const uint4*>(pw[i] + ko));
#pragma unroll
    for (int j = 0; j < 4; ++j) fx[j] = as_v8bf(*reinterpret_cast<const uint4*>(px[j] + ko));
#pragma unroll
    for (int i = 0; i < NT; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fw[i], fx[j], acc[i][j], 0, 0, 0);
  }

#pragma unroll
  for (int i = 0; i < NT; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) red[wave][i * 4 + j][r][lane] = acc[i][j][r];
  __syncthreads();
  for (int tile = wave; tile < NT * 4; tile += 4) {
    const int i = tile / 4, j = tile % 4;
    float s[4];
#pragma unroll
    for (int r = 0; r < 4; ++r)
      s[r] = red[0][tile][r][lane] + red[1][tile][r][lane] + red[2][tile][r][lane] + red[3][tile][r][lane];
    const int m = m0 + j * 16 + (lane & 15);
    const int n = n0 + i * 16 + (lane >> 4) * 4;
    if (m < M && n < N)
      *reinterpret_cast<uint2*>(out + static_cast<size_t>(m) * ldo + n) =
          make_uint2(pack_bf16x2(s[0], s[1]), pack_bf16x2(s[2], s[3]));
  }
}

}  // namespace

mx_status launch_gemm_bf16(const void* x, const void* w, void* out, int64_t M, int64_t N, int64_t K,
                           hipStream_t stream) {
  if (M == 0 || N == 0) return MX_OK;
  const int n_groups = static_cast<int>((N + 15) / 16);
  const dim3 grid(n_groups, static_cast<unsigned>((M + 63) / 64));
  gemm_bf16_kernel<1><<<grid, 256, 0, stream>>>(static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(w),
                                                 static_cast<uint16_t*>(out), static_cast<int>(M),
                                                 static_cast<int>(N), static_cast<int>(K), n_groups, K, N);
  return launch_status("mx_linear (BF16 GEMM)");
}

// G products out[:, g, :] = x[:, g, :] * W[g]^T with row strides ldx (x) and
// ldo (out) in elements; 32 columns per workgroup (N % 16 == 0, K % 32 == 0).
mx_status launch_gemm_bf16_strided(const void* x, const void* w, void* out, int64_t M, int64_t N, int64_t K,
                                   int32_t G, int64_t ldx, int64_t ldo, hipStream_t stream) {
  if (M == 0 || N == 0) return MX_OK;
  const int n_groups = static_cast<int>((N + 31) / 32);
  const dim3 grid(n_groups, static_cast<unsigned>((M + 63) / 64), static_cast<unsigned>(G));
  gemm_bf16_kernel<2><<<grid, 256, 0, stream>>>(static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(w),
                                                 static_cast<uint16_t*>(out), static_cast<int>(M),
                                                 static_cast<int>(N), static_cast<int>(K), n_groups, ldx, ldo);
  return launch_status("mx_bmm_bf16 (small T)");
}

}  // namespace mx
