// BF16 GEMM for the MXFP8 linear's BF16 branch (gfx950): out[M,N] = x[M,K] * W[N,K]^T.
//
// "[ROCm][DSv4.1][Perf] Dequantize the MXFP8 weight once when dot_scaled
// cannot be used", Purpose: when K % 128 != 0 the weight is held in BF16
// (converted once at load) and the linear is a plain BF16 product with fp32
// accumulation, rounded back to BF16.
//
// Decode-sized M (the pages' case is one row per sequence in the batch; more
// than 64 rows run on the tiled kernel below): one workgroup per 64 rows of x
// and 16*NT columns n; its four waves take
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

// Decode-sized M with a short K (the linear's BF16 branch: K = 288 or 576 at
// the pages' shapes): a wave has at most MAXS K-steps, so it issues the loads
// of all of them before its first MFMA and pays one memory latency, not one
// per step.  MT row tiles of 16, 16 columns n per workgroup.
template <int MT, int MAXS>
__global__ __launch_bounds__(256) void gemm_bf16_upfront_kernel(const uint16_t* __restrict__ x,
                                                                const uint16_t* __restrict__ w,
                                                                uint16_t* __restrict__ out, int M, int N, int K,
                                                                int n_groups) {
  __shared__ float red[4][MT][4][64];
  const int n0 = (blockIdx.x % n_groups) * 16;
  const int m0 = blockIdx.y * 16 * MT;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int KS = K / 32;
  const int kq = (lane >> 4) * 8;           // element offset inside the 32-wide step
  const uint16_t* pw = w + static_cast<size_t>(min(n0 + (lane & 15), N - 1)) * K + kq;
  const uint16_t* px[MT];
#pragma unroll
  for (int j = 0; j < MT; ++j) px[j] = x + static_cast<size_t>(min(m0 + j * 16 + (lane & 15), M - 1)) * K + kq;

  v8bf fw[MAXS], fx[MAXS][MT];
#pragma unroll
  for (int s = 0; s < MAXS; ++s) {          // steps past the end load the last step (never used)
    const int ko = min(wave + 4 * s, KS - 1) * 32;
    fw[s] = as_v8bf(*reinterpret_cast<const uint4*>(pw + ko));
#pragma unroll
    for (int j = 0; j < MT; ++j) fx[s][j] = as_v8bf(*reinterpret_cast<const uint4*>(px[j] + ko));
  }
  v4f acc[MT];
#pragma unroll
  for (int j = 0; j < MT; ++j) acc[j] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < MAXS; ++s) {
    if (wave + 4 * s < KS) {                // uniform per wave
#pragma unroll
      for (int j = 0; j < MT; ++j) acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fw[s], fx[s][j], acc[j], 0, 0, 0);
    }
  }
#pragma unroll
  for (int j = 0; j < MT; ++j)
#pragma unroll
    for (int r = 0; r < 4; ++r) red[wave][j][r][lane] = acc[j][r];
  __syncthreads();
  for (int j = wave; j < MT; j += 4) {
    float v[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) v[r] = red[0][j][r][lane] + red[1][j][r][lane] + red[2][j][r][lane] + red[3][j][r][lane];
    const int m = m0 + j * 16 + (lane & 15);
    const int n = n0 + (lane >> 4) * 4;
    if (m < M && n < N)
      *reinterpret_cast<uint2*>(out + static_cast<size_t>(m) * N + n) = make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
  }
}

// ------------------------------------------------- prefill-sized M (> 64)
//
// 128 (m) x 64*NI (n) tiles, 4 waves of 64 x 32*NI on v_mfma_f32_32x32x16_bf16
// (W the first operand, x the second, as in the kernels above: a lane's
// accumulators are n-runs of one token), K-steps of 32 (K only has to be a
// multiple of 32).  The operands stream into a ring of SLOTS LDS slots by
// LDS-DMA, SLOTS - 1 steps ahead of the MFMAs, so that a step waits for data
// requested SLOTS - 1 steps earlier; one barrier per step.  A 64-byte LDS
// row holds chunk c at slot c ^ ((row / 4) % 4): the 16 rows that a
// ds_read_b128 of 16 lanes touches fall on distinct banks.  A DMA
// instruction writes 16 consecutive rows (lane L: row L / 4, slot L % 4), so
// each lane fetches the chunk that belongs in its slot.
constexpr int kTM = 128;                    // tile rows along m
constexpr int kTK = 32;                     // K elements per step
constexpr int kTRow = kTK * 2;              // 64 bytes per LDS row
constexpr int kTRowsPerDma = 1024 / kTRow;  // 16 rows per DMA instruction

typedef float v16f_t __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void lds_void_t;

__device__ __forceinline__ void tile_barrier() {   // no memory access moves across it
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

// LDS-DMA of step kt into slot `sl` (W rows, then x rows at byte w_bytes).
// A function rather than a lambda in the kernel template: with the lambda,
// hipcc emitted no host launch stub for the kernel.
template <int WD, int XD>
__device__ __forceinline__ void tiled_issue(uint8_t* sl, int w_bytes, const uint8_t* const (&gw)[WD],
                                            const uint8_t* const (&gx)[XD], int kt, int wave) {
#pragma unroll
  for (int u = 0; u < WD; ++u)
    __builtin_amdgcn_global_load_lds(gw[u] + static_cast<size_t>(kt) * kTRow, (lds_void_t*)(sl + (WD * wave + u) * 1024),
                                     16, 0, 0);
#pragma unroll
  for (int u = 0; u < XD; ++u)
    __builtin_amdgcn_global_load_lds(gx[u] + static_cast<size_t>(kt) * kTRow,
                                     (lds_void_t*)(sl + w_bytes + (XD * wave + u) * 1024), 16, 0, 0);
}

template <int NI, int SLOTS>
__global__ __launch_bounds__(256, 2) void gemm_bf16_tiled_kernel(const uint16_t* __restrict__ x,
                                                                 const uint16_t* __restrict__ w,
                                                                 uint16_t* __restrict__ out, int M, int N, int K,
                                                                 int tiles_n) {
  constexpr int kTN = 64 * NI;              // tile rows along n
  constexpr int kWBytes = kTN * kTRow, kXBytes = kTM * kTRow;
  constexpr int kWDma = kTN / kTRowsPerDma / 4, kXDma = kTM / kTRowsPerDma / 4;   // per wave and step
  constexpr int kDma = kWDma + kXDma;
  constexpr int kAhead = SLOTS - 1;
  static_assert(kAhead >= 1 && kAhead <= 3, "waits below cover up to 2 steps in flight");
  __shared__ __attribute__((aligned(1024))) uint8_t ring[SLOTS][kWBytes + kXBytes];   // [slot][W | x]
  const int m0 = (blockIdx.x / tiles_n) * kTM;
  const int n0 = (blockIdx.x % tiles_n) * kTN;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int KT = K / kTK;

  // DMA: wave w, instruction u of an operand writes its rows 16 (k w + u) .. +15
  const uint8_t* gw[kWDma];
  const uint8_t* gx[kXDma];
  const int dr = lane >> 2;
#pragma unroll
  for (int u = 0; u < kWDma; ++u) {
    const int row = kTRowsPerDma * (kWDma * wave + u) + dr;
    const int c = (lane & 3) ^ ((row >> 2) & 3);
    gw[u] = reinterpret_cast<const uint8_t*>(w + static_cast<size_t>(min(n0 + row, N - 1)) * K) + c * 16;
  }
#pragma unroll
  for (int u = 0; u < kXDma; ++u) {
    const int row = kTRowsPerDma * (kXDma * wave + u) + dr;
    const int c = (lane & 3) ^ ((row >> 2) & 3);
    gx[u] = reinterpret_cast<const uint8_t*>(x + static_cast<size_t>(min(m0 + row, M - 1)) * K) + c * 16;
  }
  // fragments: row 32 NI wn + 32 i + lane % 32 of W (64 wm + 32 j + lane % 32
  // of x); for the step's MFMA kk, lane group q = lane / 32 takes chunk 2kk + q
  const int r32 = lane & 31, q = lane >> 5;
  auto frag = [&](const uint8_t* base, int row, int kk) {
    const int c = 2 * kk + q;
    return __builtin_bit_cast(v8bf, *reinterpret_cast<const uint4*>(base + row * kTRow + ((c ^ ((row >> 2) & 3)) << 4)));
  };
  v16f_t acc[NI][2];
#pragma unroll
  for (int i = 0; i < NI; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

#pragma unroll
  for (int st = 0; st < kAhead; ++st)
    if (st < KT) tiled_issue<kWDma, kXDma>(ring[st % SLOTS], kWBytes, gw, gx, st, wave);
  for (int kt = 0; kt < KT; ++kt) {
    // wait for this wave's DMA of step kt (later steps may stay in flight),
    // then for everyone's
    const int ahead = min(KT - 1 - kt, kAhead - 1);
    if (ahead >= 2) __builtin_amdgcn_s_waitcnt(wait_vm(2 * kDma));
    else if (ahead == 1) __builtin_amdgcn_s_waitcnt(wait_vm(kDma));
    else __builtin_amdgcn_s_waitcnt(wait_vm(0));
    tile_barrier();
    // slot of step kt + kAhead = slot of step kt - 1, whose readers all passed the barrier
    if (kt + kAhead < KT) tiled_issue<kWDma, kXDma>(ring[(kt + kAhead) % SLOTS], kWBytes, gw, gx, kt + kAhead, wave);
    const uint8_t* lw = ring[kt % SLOTS];
    const uint8_t* lx = lw + kWBytes;
    v8bf fw[2][NI], fx[2][2];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
#pragma unroll
      for (int i = 0; i < NI; ++i) fw[kk][i] = frag(lw, 32 * NI * wn + 32 * i + r32, kk);
#pragma unroll
      for (int j = 0; j < 2; ++j) fx[kk][j] = frag(lx, 64 * wm + 32 * j + r32, kk);
    }
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
      for (int i = 0; i < NI; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fw[kk][i], fx[kk][j], acc[i][j], 0, 0, 0);
  }

  // epilogue: lane holds token m = 64 wm + 32 j + lane % 32 and n = 32 NI wn
  // + 32 i + 8 (r / 4) + 4 q + r % 4; v_permlane32_swap pairs the lane halves
  // so that each lane stores 8 consecutive n (16 bytes)
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int m = m0 + 64 * wm + 32 * j + r32;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const v16f_t& v = acc[i][j];
#pragma unroll
      for (int pp = 0; pp < 2; ++pp) {
        const uint32_t x0 = pack_bf16x2(v[8 * pp + 0], v[8 * pp + 1]), x1 = pack_bf16x2(v[8 * pp + 2], v[8 * pp + 3]);
        const uint32_t y0 = pack_bf16x2(v[8 * pp + 4], v[8 * pp + 5]), y1 = pack_bf16x2(v[8 * pp + 6], v[8 * pp + 7]);
        const auto s0 = __builtin_amdgcn_permlane32_swap(x0, y0, false, false);
        const auto s1 = __builtin_amdgcn_permlane32_swap(x1, y1, false, false);
        const int n = n0 + 32 * NI * wn + 32 * i + pp * 16 + q * 8;
        if (m < M && n < N)
          *reinterpret_cast<uint4*>(out + static_cast<size_t>(m) * N + n) = make_uint4(s0[0], s1[0], s0[1], s1[1]);
      }
    }
  }
}

template <int NI, int SLOTS>
void launch_tiled(const void* x, const void* w, void* out, int64_t M, int64_t N, int64_t K, hipStream_t stream) {
  const int tiles_n = static_cast<int>((N + 64 * NI - 1) / (64 * NI));
  const int64_t tiles = (M + kTM - 1) / kTM * tiles_n;
  gemm_bf16_tiled_kernel<NI, SLOTS><<<static_cast<unsigned>(tiles), 256, 0, stream>>>(
      static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(w), static_cast<uint16_t*>(out),
      static_cast<int>(M), static_cast<int>(N), static_cast<int>(K), tiles_n);
}

template <int MT, int MAXS>
void launch_upfront(const void* x, const void* w, void* out, int64_t M, int64_t N, int64_t K, hipStream_t stream) {
  const int n_groups = static_cast<int>((N + 15) / 16);
  const dim3 grid(n_groups, static_cast<unsigned>((M + 16 * MT - 1) / (16 * MT)));
  gemm_bf16_upfront_kernel<MT, MAXS><<<grid, 256, 0, stream>>>(
      static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(w), static_cast<uint16_t*>(out),
      static_cast<int>(M), static_cast<int>(N), static_cast<int>(K), n_groups);
}

template <int MT>
bool launch_upfront_k(const void* x, const void* w, void* out, int64_t M, int64_t N, int64_t K, hipStream_t stream) {
  const int64_t steps = (K / 32 + 3) / 4;   // K-steps of wave 0
  if (steps <= 3) launch_upfront<MT, 3>(x, w, out, M, N, K, stream);
  else if (steps <= 5) launch_upfront<MT, 5>(x, w, out, M, N, K, stream);
  else if (steps <= 8) launch_upfront<MT, 8>(x, w, out, M, N, K, stream);
  else return false;
  return true;
}

}  // namespace

mx_status launch_gemm_bf16(const void* x, const void* w, void* out, int64_t M, int64_t N, int64_t K,
                           hipStream_t stream) {
  if (M == 0 || N == 0) return MX_OK;
  // up to 16 rows (a decode batch): all loads up front (measured 4.5 -> 3.7 us at
  // N = 5120, K = 576, M = 1); more rows: the split-K loop below was as fast
  if (M <= 16 && launch_upfront_k<1>(x, w, out, M, N, K, stream)) return launch_status("mx_linear (BF16 GEMM)");
  if (M > 64) {
    // prefill-sized M: 128 x 256 tiles, or 128 x 128 where the wider tiles
    // would give fewer than two per compute unit (M = 8192, N = 5120, K = 576:
    // 75.9 -> 67.3 us with the wider tiles; M = 1000: 18.1 -> 16.8 us with
    // the narrower ones)
    const int64_t wide_tiles = (M + kTM - 1) / kTM * ((N + 255) / 256);
    if (wide_tiles >= 512)
      launch_tiled<4, 3>(x, w, out, M, N, K, stream);
    else
      launch_tiled<2, 3>(x, w, out, M, N, K, stream);
    return launch_status("mx_linear (BF16 GEMM, tiled)");
  }
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
