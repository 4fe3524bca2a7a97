// Block-32 scaled FP8 GEMMs of the MXFP8 linear for decode batches (gfx950):
// out[M,N] = x[M,K] * W[N,K]^T with E8M0 scales [M,K/32] and [N,K/32].
//
// "[ROCm][DSv4.1][Perf] Dequantize the MXFP8 weight once when dot_scaled
// cannot be used", Purpose: with K % 128 == 0 the linear stays in FP8 -- x is
// quantised to MXFP8 (block 32) and multiplied with the FP8 weight and its
// E8M0 block scales on the block-scaled MFMA.  These kernels serve that
// branch for M <= 64 rows.
//
// At these sizes the time is the latency of bringing the weight in (a few MB
// spread over every compute unit), so a workgroup of 16 columns n puts its
// whole weight slice, 16 x K bytes, and its scale rows in flight at once by
// LDS-DMA, waits once, and only then runs its MFMAs:
//
//  * gemm_mx32_wres_kernel takes x already quantised (by the quantiser, so
//    read from L2) straight into MFMA operand registers, issued before the
//    weight.  17..64 rows (TT = 4): wave w multiplies token tile w (x rows
//    16w..16w+15) over all of K, K / 128 <= 18 so that the fragments fit the
//    registers.  1..16 rows (TT = 1): the four waves take contiguous quarters
//    of K and add their partial sums through LDS in a fixed order.
//  * linear_mx32_fused_kernel (1..16 rows) takes x in BF16 and quantises it
//    itself, which saves the quantiser's launch.
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
constexpr int kFusedMaxSpw = 8;              // fused kernel: K <= 4096 (a wave's BF16 x quarter in registers)

// 16-byte chunk c of weight row r within a step is stored at chunk c ^ swz(r),
// so that the 16 rows' reads of one chunk fall in distinct banks.
__device__ __forceinline__ int swz(int r) { return ((r >> 1) ^ ((r & 1) << 2)) & 7; }

__device__ __forceinline__ v8i make_frag(const uint4 lo, const uint4 hi) {
  v8i r;
  r[0] = lo.x; r[1] = lo.y; r[2] = lo.z; r[3] = lo.w;
  r[4] = hi.x; r[5] = hi.y; r[6] = hi.z; r[7] = hi.w;
  return r;
}

// The weight slice [16 rows][K] into sW as [step][row][128 B] and its scale
// rows [16][K/32] into sS, by LDS-DMA.  Operand instruction ii moves rows
// 8(ii % 2)..8(ii % 2)+7 of step ii / 2 (1 KiB); wave w issues ii = w, w+4,
// ...  The scale rows move 4 bytes per lane (the slice's scale rows are one
// contiguous range).  The DMA is issued as buffer loads: with a global
// (flat-encoded) LDS-DMA in flight the compiler waits for all vector memory
// before the first use of any loaded register, so a kernel could not work
// on x while the weight is on its way.
__device__ __forceinline__ void dma_weight_slice(const uint8_t* w, const uint8_t* sw, int n0, int K, uint8_t* sW,
                                                 uint8_t* sS, int wave, int lane) {
  const int KB = K / kStep, SPK = K / 32;
  const int dr = lane >> 3;
  const __amdgpu_buffer_rsrc_t wres = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(w + static_cast<size_t>(n0) * K), 0, kRowsN * K, kBufferFlags);
  for (int ii = wave; ii < 2 * KB; ii += 4) {
    const int kt = ii >> 1, half = ii & 1, r = 8 * half + dr;
    const int off = r * K + kt * kStep + ((lane & 7) ^ swz(r)) * 16;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(wres, (lds_void_t*)(sW + kt * kStepBytes + 8 * half * kStep), 16, off, 0,
                                             0, 0);
  }
  const int sc_bytes = kRowsN * SPK;
  const __amdgpu_buffer_rsrc_t sres = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(sw + static_cast<size_t>(n0) * SPK), 0, sc_bytes, kBufferFlags);
  for (int jj = wave; jj * 256 < sc_bytes; jj += 4) {
    const int byte = jj * 256 + 4 * lane;
    if (byte < sc_bytes) __builtin_amdgcn_raw_ptr_buffer_load_lds(sres, (lds_void_t*)(sS + jj * 256), 4, byte, 0, 0, 0);
  }
}

// The wave's MFMAs over steps kb0 .. kb0 + SPW - 1 (with RAGGED, only those
// below K / 128): weight fragments from LDS, x fragments and scale bytes from
// registers.
template <int SPW, bool RAGGED>
__device__ __forceinline__ v4f mfma_steps(const uint8_t* sW, const uint8_t* sS, int K, int kb0, int lane,
                                          const v8i (&xf)[SPW], const int (&xsb)[SPW]) {
  const int KB = K / kStep, SPK = K / 32;
  const int r16 = lane & 15, q = lane >> 4;
  const int sz = swz(r16);
  const int c0 = (q ^ sz) * 16, c1 = ((q + 4) ^ sz) * 16;
  const uint8_t* wrow = sW + r16 * kStep;
  const uint8_t* wsc = sS + r16 * SPK + q;
  v4f acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int j = 0; j < SPW; ++j) {
    const int kt = kb0 + j;
    if (RAGGED && kt >= KB) break;             // uniform across the wave
    const uint8_t* st = wrow + kt * kStepBytes;
    const v8i fw = make_frag(*reinterpret_cast<const uint4*>(st + c0), *reinterpret_cast<const uint4*>(st + c1));
    acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(fw, xf[j], acc, 0, 0, 0, wsc[4 * kt], 0, xsb[j]);
  }
  return acc;
}

// The four waves' partial sums of token tile 0, added in a fixed order and
// stored by wave 0 for the rows below M.
__device__ __forceinline__ void reduce_store(float (&red)[4][4][64], const v4f& acc, uint16_t* out, int M, int N,
                                             int n0, int wave, int lane) {
#pragma unroll
  for (int e = 0; e < 4; ++e) red[wave][e][lane] = acc[e];
  __syncthreads();
  const int r16 = lane & 15, q = lane >> 4;
  if (wave == 0 && r16 < M) {
    float s[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) s[e] = ((red[0][e][lane] + red[1][e][lane]) + red[2][e][lane]) + red[3][e][lane];
    *reinterpret_cast<uint2*>(out + static_cast<size_t>(r16) * N + n0 + 4 * q) =
        make_uint2(pack_bf16x2(s[0], s[1]), pack_bf16x2(s[2], s[3]));
  }
}

// ------------------------------------------------ x quantised beforehand

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

  // ---- x fragments and scale bytes to registers, first.  Rows past M
  // re-read row M - 1 and steps past K re-read the last step: harmless, never
  // stored or multiplied.
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

  dma_weight_slice(p.w, p.sw, n0, p.K, sW, sS, wave, lane);
  __builtin_amdgcn_s_waitcnt(wait_vm(0));      // this wave's loads have landed
  __builtin_amdgcn_s_barrier();                // and every wave's

  const v4f acc = mfma_steps<SPW, TT == 1>(sW, sS, p.K, kb0, lane, xf, xsb);
  if constexpr (TT == 4) {
    // the MFMAs take operands from every lane: keep them out of the
    // row-guarded store below
    asm volatile("" ::"v"(acc));
    const int t = 16 * wave + r16;
    if (t < p.M)
      *reinterpret_cast<uint2*>(p.out + static_cast<size_t>(t) * p.N + n0 + 4 * q) =
          make_uint2(pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3]));
  } else {
    __shared__ float red[4][4][64];
    reduce_store(red, acc, p.out, p.M, p.N, n0, wave, lane);
  }
}

// ------------------------------------------- x quantised inside the GEMM
//
// For 1..16 rows the quantiser's launch costs as much as the GEMM's weight
// stream, so this kernel takes x in BF16 and quantises it itself by the
// quantiser's rule (per-row 32-K blocks, OCP, e = the E8M0 exponent of the
// block amax, codes by v_cvt_scalef32_pk_fp8_bf16 on the scale bits
// (e + 127) << 23; a non-finite block gives codes 0x7F and scale 0xFF).  Each
// workgroup quantises the M rows of its waves' K quarters for itself; the
// quantisation lands straight in the MFMA operand layout:
//  * lane (r, q) holds K [16q, 16q+16) and [64+16q, 64+16q+16) of a step,
//    halves of the 32-K blocks q/2 and 2 + q/2, whose other halves are in
//    lane l ^ 16 (group q ^ 1): the block amax takes one v_permlane16_swap;
//  * the MFMA wants the scale of block q from lane group q: groups 0 and 3
//    computed it themselves, groups 1 and 2 take it from each other (lane
//    l ^ 48) with a v_permlane16_swap and a v_permlane32_swap.
// The lane exchanges are VALU swaps, not LDS-pipe instructions: the compiler
// would make those wait for the weight's DMA.

struct FusedArgs {
  const uint16_t* x;   // [M, K] BF16
  const uint8_t* w;    // [N, K] OCP e4m3
  const uint8_t* sw;   // [N, K/32] E8M0
  uint16_t* out;       // [M, N] BF16
  int M, N, K;
};

// largest BF16 magnitude pattern of the 16 values in a, b (packed u16 max)
__device__ __forceinline__ uint32_t amax16(const uint4 a, const uint4 b) {
  typedef unsigned short v2u16 __attribute__((ext_vector_type(2)));
  const uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
  v2u16 m = __builtin_bit_cast(v2u16, w[0] & 0x7FFF7FFFu);
#pragma unroll
  for (int i = 1; i < 8; ++i) m = __builtin_elementwise_max(m, __builtin_bit_cast(v2u16, w[i] & 0x7FFF7FFFu));
  return max(static_cast<uint32_t>(m[0]), static_cast<uint32_t>(m[1]));
}

// 16 BF16 values (a, b) divided by the E8M0 scale in `sbits` -> 16 OCP codes
__device__ __forceinline__ uint4 encode16(const uint4 a, const uint4 b, float sbits) {
  typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
  typedef short v2s __attribute__((ext_vector_type(2)));
  const uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
  uint32_t c[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v2s v = {0, 0};
    v = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(v, __builtin_bit_cast(v2bf, w[2 * i]), sbits, false);
    v = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(v, __builtin_bit_cast(v2bf, w[2 * i + 1]), sbits, true);
    c[i] = __builtin_bit_cast(uint32_t, v);
  }
  return make_uint4(c[0], c[1], c[2], c[3]);
}

// SPW: K-steps per wave (a quarter of K / 128, rounded up).  Requires M <= 16,
// N % 16 == 0, K % 128 == 0, K / 128 <= 4 SPW, and a 4-byte aligned scale
// tensor.
template <int SPW>
__global__ __launch_bounds__(256, 1) void linear_mx32_fused_kernel(FusedArgs p) {
  __shared__ __attribute__((aligned(1024))) uint8_t sW[4 * SPW * kStepBytes];   // [step][row][128 B]
  __shared__ __attribute__((aligned(16))) uint8_t sS[kRowsN * 4 * 4 * SPW];     // [row][K/32]
  __shared__ float red[4][4][64];

  const int n0 = blockIdx.x * kRowsN;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int KB = p.K / kStep;
  const int r16 = lane & 15, q = lane >> 4;
  const int kb0 = wave * SPW;

  // ---- BF16 x of this wave's steps to registers, first: lane (r, q) loads
  // K [16q, 16q+16) and [64+16q, 64+16q+16) of each step of row r.  Rows past
  // M re-read row M - 1 and steps past K the last step: never stored or
  // multiplied.
  const uint16_t* xrow = p.x + static_cast<size_t>(min(r16, p.M - 1)) * p.K + 16 * q;
  uint4 xb[SPW][4];
#pragma unroll
  for (int j = 0; j < SPW; ++j) {
    const uint16_t* src = xrow + min(kb0 + j, KB - 1) * kStep;
    xb[j][0] = *reinterpret_cast<const uint4*>(src);
    xb[j][1] = *reinterpret_cast<const uint4*>(src + 8);
    xb[j][2] = *reinterpret_cast<const uint4*>(src + 64);
    xb[j][3] = *reinterpret_cast<const uint4*>(src + 72);
  }

  dma_weight_slice(p.w, p.sw, n0, p.K, sW, sS, wave, lane);

  // ---- quantise x into MFMA fragments while the weight's DMA is in flight
  // (its buffer-load form lets the compiler wait for the x loads alone)
  v8i xf[SPW];
  int xsb[SPW];
#pragma unroll
  for (int j = 0; j < SPW; ++j) {
    // v_permlane16_swap(v, v) leaves rows (R0, R0, R2, R2) in the first
    // result and (R1, R1, R3, R3) in the second: their max is the max with
    // lane l ^ 16, per 16-bit half
    const uint32_t a12 = amax16(xb[j][0], xb[j][1]) | (amax16(xb[j][2], xb[j][3]) << 16);
    const auto sw16 = __builtin_amdgcn_permlane16_swap(a12, a12, false, false);
    const uint32_t a1 = max(sw16[0] & 0xFFFFu, sw16[1] & 0xFFFFu), a2 = max(sw16[0] >> 16, sw16[1] >> 16);
    const bool f1 = a1 < 0x7F80u, f2 = a2 < 0x7F80u;
    const int e1 = e8m0_exponent<8>(f1 ? a1 : 0), e2 = e8m0_exponent<8>(f2 ? a2 : 0);
    const uint4 nan4 = make_uint4(0x7F7F7F7Fu, 0x7F7F7F7Fu, 0x7F7F7F7Fu, 0x7F7F7F7Fu);
    const uint4 lo = f1 ? encode16(xb[j][0], xb[j][1], __uint_as_float(static_cast<uint32_t>(e1 + 127) << 23)) : nan4;
    const uint4 hi = f2 ? encode16(xb[j][2], xb[j][3], __uint_as_float(static_cast<uint32_t>(e2 + 127) << 23)) : nan4;
    xf[j] = make_frag(lo, hi);
    const uint32_t s1 = f1 ? e1 + 127 : 0xFF, s2 = f2 ? e2 + 127 : 0xFF;
    // rows (R0, R0, R2, R2) | (R1, R1, R3, R3), then the 32-lane swap of the
    // two: (R0, R0, R1, R1) | (R2, R2, R3, R3) -- row 1 finds row 2 in the
    // second result and row 2 finds row 1 in the first
    const uint32_t s12 = s1 | (s2 << 8);
    const auto t16 = __builtin_amdgcn_permlane16_swap(s12, s12, false, false);
    const auto t32 = __builtin_amdgcn_permlane32_swap(t16[0], t16[1], false, false);
    xsb[j] = static_cast<int>(q == 0 ? s1 : q == 3 ? s2 : q == 1 ? (t32[1] & 0xFFu) : ((t32[0] >> 8) & 0xFFu));
  }
  __builtin_amdgcn_s_waitcnt(wait_vm(0));      // this wave's loads have landed
  __builtin_amdgcn_s_barrier();                // and every wave's

  const v4f acc = mfma_steps<SPW, true>(sW, sS, p.K, kb0, lane, xf, xsb);
  reduce_store(red, acc, p.out, p.M, p.N, n0, wave, lane);
}

template <int SPW, int TT>
void launch_wres(const WresArgs& a, int grid, hipStream_t stream) {
  gemm_mx32_wres_kernel<SPW, TT><<<grid, 256, 0, stream>>>(a);
}

template <int SPW>
void launch_fused(const FusedArgs& a, int grid, hipStream_t stream) {
  linear_mx32_fused_kernel<SPW><<<grid, 256, 0, stream>>>(a);
}

}  // namespace

#define MX_CASE(S, CALL) \
  case S:                \
    CALL;                \
    break;

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
      MX_CASE(1, (launch_wres<1, 1>(a, grid, stream))) MX_CASE(2, (launch_wres<2, 1>(a, grid, stream)))
      MX_CASE(3, (launch_wres<3, 1>(a, grid, stream))) MX_CASE(4, (launch_wres<4, 1>(a, grid, stream)))
      MX_CASE(5, (launch_wres<5, 1>(a, grid, stream))) MX_CASE(6, (launch_wres<6, 1>(a, grid, stream)))
      MX_CASE(7, (launch_wres<7, 1>(a, grid, stream))) MX_CASE(8, (launch_wres<8, 1>(a, grid, stream)))
      MX_CASE(9, (launch_wres<9, 1>(a, grid, stream))) MX_CASE(10, (launch_wres<10, 1>(a, grid, stream)))
      MX_CASE(11, (launch_wres<11, 1>(a, grid, stream))) MX_CASE(12, (launch_wres<12, 1>(a, grid, stream)))
      MX_CASE(13, (launch_wres<13, 1>(a, grid, stream))) MX_CASE(14, (launch_wres<14, 1>(a, grid, stream)))
      MX_CASE(15, (launch_wres<15, 1>(a, grid, stream))) MX_CASE(16, (launch_wres<16, 1>(a, grid, stream)))
      default: return false;
    }
  } else {
    switch (KB) {
      MX_CASE(1, (launch_wres<1, 4>(a, grid, stream))) MX_CASE(2, (launch_wres<2, 4>(a, grid, stream)))
      MX_CASE(3, (launch_wres<3, 4>(a, grid, stream))) MX_CASE(4, (launch_wres<4, 4>(a, grid, stream)))
      MX_CASE(5, (launch_wres<5, 4>(a, grid, stream))) MX_CASE(6, (launch_wres<6, 4>(a, grid, stream)))
      MX_CASE(7, (launch_wres<7, 4>(a, grid, stream))) MX_CASE(8, (launch_wres<8, 4>(a, grid, stream)))
      MX_CASE(9, (launch_wres<9, 4>(a, grid, stream))) MX_CASE(10, (launch_wres<10, 4>(a, grid, stream)))
      MX_CASE(11, (launch_wres<11, 4>(a, grid, stream))) MX_CASE(12, (launch_wres<12, 4>(a, grid, stream)))
      MX_CASE(13, (launch_wres<13, 4>(a, grid, stream))) MX_CASE(14, (launch_wres<14, 4>(a, grid, stream)))
      MX_CASE(15, (launch_wres<15, 4>(a, grid, stream))) MX_CASE(16, (launch_wres<16, 4>(a, grid, stream)))
      MX_CASE(17, (launch_wres<17, 4>(a, grid, stream))) MX_CASE(18, (launch_wres<18, 4>(a, grid, stream)))
      default: return false;
    }
  }
  *st = launch_status("mx_linear (block-scaled FP8 GEMM)");
  return true;
}

// x quantised inside the GEMM, for M 1..16 and K / 128 <= 32 (scale tensor
// 4-byte aligned).  Returns false, launching nothing, for any other shape.
bool launch_linear_mx32_fused(const void* x, const uint8_t* w, const uint8_t* sw, void* out, int64_t M, int64_t N,
                              int64_t K, hipStream_t stream, mx_status* st) {
  if (M < 1 || M > 16 || N < 16 || N % kRowsN != 0 || K < kStep || K % kStep != 0) return false;
  if (!aligned(x, 16) || !aligned(w, 16) || !aligned(sw, 4)) return false;
  const int KB = static_cast<int>(K / kStep);
  if (KB > 4 * kFusedMaxSpw) return false;
  const FusedArgs a{static_cast<const uint16_t*>(x), w, sw, static_cast<uint16_t*>(out), static_cast<int>(M),
                    static_cast<int>(N), static_cast<int>(K)};
  const int grid = static_cast<int>(N / kRowsN);
  switch ((KB + 3) / 4) {
    MX_CASE(1, (launch_fused<1>(a, grid, stream))) MX_CASE(2, (launch_fused<2>(a, grid, stream)))
    MX_CASE(3, (launch_fused<3>(a, grid, stream))) MX_CASE(4, (launch_fused<4>(a, grid, stream)))
    MX_CASE(5, (launch_fused<5>(a, grid, stream))) MX_CASE(6, (launch_fused<6>(a, grid, stream)))
    MX_CASE(7, (launch_fused<7>(a, grid, stream))) MX_CASE(8, (launch_fused<8>(a, grid, stream)))
    default: return false;
  }
  *st = launch_status("mx_linear (block-scaled FP8 GEMM, x quantised in the kernel)");
  return true;
}

#undef MX_CASE

}  // namespace mx
