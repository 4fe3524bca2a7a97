// Block-32 scaled FP8 GEMM of the MXFP8 linear, weight slice resident in LDS
// (gfx950): out[M,N] = xq[M,K] * W[N,K]^T with E8M0 scales [M,K/32], [N,K/32].
//
// "[ROCm][DSv4.1][Perf] Dequantize the MXFP8 weight once when dot_scaled
// cannot be used", Purpose: with K % 128 == 0 the linear stays in FP8 -- x is
// quantised to MXFP8 (block 32) and multiplied with the FP8 weight and its
// E8M0 block scales on the block-scaled MFMA.  This is that GEMM for decode
// batches (M <= 64 rows).
//
// At these sizes the time is the latency of bringing the weight in (a few MB
// spread over every compute unit), so a workgroup of 16 columns n puts its
// whole weight slice, 16 x K bytes, and its scale rows in flight at once by
// LDS-DMA, waits once, and only then runs its MFMAs.  The quantised x rows,
// written just before by the quantiser and so read from L2, go straight to
// registers in the MFMA operand layout; they are issued before the weight so
// that they are not queued behind it.
//
//  * 17..64 rows (TT = 4): wave w multiplies token tile w (x rows
//    16w..16w+15) over all of K; K / 128 <= 18 keeps the x fragments in
//    registers.
//  * 1..16 rows (TT = 1): the four waves take contiguous quarters of K and
//    add their partial sums through LDS in a fixed order.
//
// v_mfma_scale_f32_16x16x128_f8f6f4 operand layout (checked on the hardware
// with one-hot inputs): lane l holds row l % 16; with q = l / 16 its 32 bytes
// are K [16q, 16q+16) and [64+16q, 64+16q+16) of the 128-K step, and its
// scale byte is the one of the step's 32-K block q.  W is the first operand
// and x the second, so a lane ends with four consecutive n of one row.
#include "common.hpp"

namespace mx {

namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void_t;

constexpr int kStep = 128;                   // K bytes per MFMA step
constexpr int kRowsN = 16;                   // weight rows (columns n) per workgroup
constexpr int kStepBytes = kRowsN * kStep;   // 2 KiB of weight per step
constexpr int kMaxStepsTile4 = 18;           // K <= 2304 with four token tiles
constexpr int kMaxStepsTile1 = 64;           // K <= 8192 with one token tile (128 KiB of LDS)

// 16-byte chunk c of weight row r within a step is stored at chunk c ^ swz(r),
// so that the 16 rows' reads of one chunk fall in distinct banks.
__device__ __forceinline__ int swz(int r) { return ((r >> 1) ^ ((r & 1) << 2)) & 7; }

__device__ __forceinline__ v8i make_frag(const uint4 lo, const uint4 hi) {
  v8i r;
  r[0] = lo.x; r[1] = lo.y; r[2] = lo.z; r[3] = lo.w;
  r[4] = hi.x; r[5] = hi.y; r[6] = hi.z; r[7] = hi.w;
  return r;
}

struct WresArgs {
  const uint8_t* xq;   // [M, K] OCP e4m3
  const uint8_t* xs;   // [M, K/32] E8M0
  const uint8_t* w;    // [N, K] OCP e4m3
  const uint8_t* sw;   // [N, K/32] E8M0
  uint16_t* out;       // [M, N] BF16
  int M, N, K;
};

// SPW: K-steps per wave (TT = 4: all K / 128 of them; TT = 1: a quarter,
// rounded up).  Requires N % 16 == 0, K % 128 == 0, K / 128 <= SPW * (TT == 4 ?
// 1 : 4), and 4-byte aligned scale rows.
template <int SPW, int TT>
__global__ __launch_bounds__(256, 1) void gemm_mx32_wres_kernel(WresArgs p) {
  constexpr int kMaxKB = TT == 4 ? SPW : 4 * SPW;
  __shared__ __attribute__((aligned(1024))) uint8_t sW[kMaxKB * kStepBytes];   // [step][row][128 B]
  __shared__ __attribute__((aligned(16))) uint8_t sS[kRowsN * 4 * kMaxKB];     // [row][K/32]

  const int n0 = blockIdx.x * kRowsN;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int KB = p.K / kStep;
  const int SPK = 4 * KB;                      // scale bytes per row
  const int r16 = lane & 15, q = lane >> 4;
  const int kb0 = TT == 4 ? 0 : wave * SPW;    // this wave's first step
  const int tile = TT == 4 ? wave : 0;

  // ---- x fragments and scale bytes to registers.  Rows past M re-read row
  // M - 1 and steps past K re-read the last step: harmless, never stored or
  // multiplied.
  const int m = min(16 * tile + r16, p.M - 1);
  const uint8_t* xrow = p.xq + static_cast<size_t>(m) * p.K + 16 * q;
  const uint8_t* srow = p.xs + static_cast<size_t>(m) * SPK + q;
  v8i xf[SPW];
  int xsb[SPW];
#pragma unroll
  for (int j = 0; j < SPW; ++j) {
    const int kt = min(kb0 + j, KB - 1);
    xf[j] = make_frag(*reinterpret_cast<const uint4*>(xrow + kt * kStep),
                      *reinterpret_cast<const uint4*>(xrow + kt * kStep + 64));
    xsb[j] = srow[4 * kt];
  }

  // ---- the weight slice by LDS-DMA: instruction ii moves rows
  // 8(ii % 2)..8(ii % 2)+7 of step ii / 2 (1 KiB); wave w issues ii = w, w+4, ...
  const int dr = lane >> 3;
  for (int ii = wave; ii < 2 * KB; ii += 4) {
    const int kt = ii >> 1, half = ii & 1, r = 8 * half + dr;
    const uint8_t* src = p.w + static_cast<size_t>(n0 + r) * p.K + kt * kStep + ((lane & 7) ^ swz(r)) * 16;
    __builtin_amdgcn_global_load_lds(src, (lds_void_t*)(sW + kt * kStepBytes + 8 * half * kStep), 16, 0, 0);
  }
  // ... and its scale rows, 4 bytes per lane
  const int sc_bytes = kRowsN * SPK;
  for (int jj = wave; jj * 256 < sc_bytes; jj += 4) {
    const int byte = jj * 256 + 4 * lane;
    if (byte < sc_bytes) {
      const int r = byte / SPK, off = byte - r * SPK;
      __builtin_amdgcn_global_load_lds(p.sw + static_cast<size_t>(n0 + r) * SPK + off, (lds_void_t*)(sS + jj * 256),
                                       4, 0, 0);
    }
  }
  __builtin_amdgcn_s_waitcnt(0x0070);          // vmcnt(0) lgkmcnt(0): this wave's loads have landed
  __builtin_amdgcn_s_barrier();                // and every wave's

  // ---- MFMAs
  const int sz = swz(r16);
  const int c0 = (q ^ sz) * 16, c1 = ((q + 4) ^ sz) * 16;
  const uint8_t* wrow = sW + r16 * kStep;
  const uint8_t* wsc = sS + r16 * SPK + q;
  v4f acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int j = 0; j < SPW; ++j) {
    const int kt = kb0 + j;
    if (TT == 1 && kt >= KB) break;            // uniform across the wave
    const uint8_t* st = wrow + kt * kStepBytes;
    const v8i fw = make_frag(*reinterpret_cast<const uint4*>(st + c0), *reinterpret_cast<const uint4*>(st + c1));
    acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(fw, xf[j], acc, 0, 0, 0, wsc[4 * kt], 0, xsb[j]);
  }

  // the MFMAs take operands from every lane: keep them out of the
  // row-guarded store below
  asm volatile("" ::"v"(acc));

  const int n = n0 + 4 * q;
  if constexpr (TT == 4) {
    const int t = 16 * wave + r16;
    if (t < p.M)
      *reinterpret_cast<uint2*>(p.out + static_cast<size_t>(t) * p.N + n) =
          make_uint2(pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3]));
  } else {
    __shared__ float red[4][4][64];
#pragma unroll
    for (int e = 0; e < 4; ++e) red[wave][e][lane] = acc[e];
    __syncthreads();
    if (wave == 0 && r16 < p.M) {
      float s[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) s[e] = ((red[0][e][lane] + red[1][e][lane]) + red[2][e][lane]) + red[3][e][lane];
      *reinterpret_cast<uint2*>(p.out + static_cast<size_t>(r16) * p.N + n) =
          make_uint2(pack_bf16x2(s[0], s[1]), pack_bf16x2(s[2], s[3]));
    }
  }
}

template <int SPW, int TT>
void launch_wres(const WresArgs& a, int grid, hipStream_t stream) {
  gemm_mx32_wres_kernel<SPW, TT><<<grid, 256, 0, stream>>>(a);
}

#define MX_WRES_CASE(S, TT) \
  case S:                   \
    launch_wres<S, TT>(a, grid, stream); break;

}  // namespace

// The weight-resident GEMM for the shapes it takes (M 1..64; K / 128 <= 64
// for M <= 16, <= 18 otherwise; scale tensors 4-byte aligned).  Returns false,
// launching nothing, for any other shape.
bool launch_gemm_mx32_wres(const uint8_t* xq, const uint8_t* xs, const uint8_t* w, const uint8_t* sw, void* out,
                           int64_t M, int64_t N, int64_t K, hipStream_t stream, mx_status* st) {
  if (M < 1 || M > 64 || N < 16 || N % kRowsN != 0 || K < kStep || K % kStep != 0) return false;
  if (!aligned(xs, 4) || !aligned(sw, 4) || !aligned(xq, 16) || !aligned(w, 16)) return false;
  const int KB = static_cast<int>(K / kStep);
  if (KB > (M <= 16 ? kMaxStepsTile1 : kMaxStepsTile4)) return false;
  const WresArgs a{xq, xs, w, sw, static_cast<uint16_t*>(out), static_cast<int>(M), static_cast<int>(N),
                   static_cast<int>(K)};
  const int grid = static_cast<int>(N / kRowsN);
  if (M <= 16) {
    switch ((KB + 3) / 4) {
      MX_WRES_CASE(1, 1) MX_WRES_CASE(2, 1) MX_WRES_CASE(3, 1) MX_WRES_CASE(4, 1)
      MX_WRES_CASE(5, 1) MX_WRES_CASE(6, 1) MX_WRES_CASE(7, 1) MX_WRES_CASE(8, 1)
      MX_WRES_CASE(9, 1) MX_WRES_CASE(10, 1) MX_WRES_CASE(11, 1) MX_WRES_CASE(12, 1)
      MX_WRES_CASE(13, 1) MX_WRES_CASE(14, 1) MX_WRES_CASE(15, 1) MX_WRES_CASE(16, 1)
      default: return false;
    }
  } else {
    switch (KB) {
      MX_WRES_CASE(1, 4) MX_WRES_CASE(2, 4) MX_WRES_CASE(3, 4) MX_WRES_CASE(4, 4)
      MX_WRES_CASE(5, 4) MX_WRES_CASE(6, 4) MX_WRES_CASE(7, 4) MX_WRES_CASE(8, 4)
      MX_WRES_CASE(9, 4) MX_WRES_CASE(10, 4) MX_WRES_CASE(11, 4) MX_WRES_CASE(12, 4)
      MX_WRES_CASE(13, 4) MX_WRES_CASE(14, 4) MX_WRES_CASE(15, 4) MX_WRES_CASE(16, 4)
      MX_WRES_CASE(17, 4) MX_WRES_CASE(18, 4)
      default: return false;
    }
  }
  *st = launch_status("mx_linear (block-scaled FP8 GEMM)");
  return true;
}

#undef MX_WRES_CASE

}  // namespace mx
