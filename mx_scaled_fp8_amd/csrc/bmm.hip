// Batched a8w8 GEMM with E8M0 block scales on CDNA4 block-scaled FP8 MFMA (gfx950).
//
// "[ROCm][DSV4][Perf] Use FP8 WO_A output projection", Summary item 2: the
// quantised activation A [T, G, K] (E8M0 scale per 128 consecutive K) is
// multiplied with the checkpoint's FP8 weight W [G, N, K] (E8M0 scale per
// (g, n, 128-K block)), out[t, g, n] = sum_k A*sa * W*sw, in place of the BF16
// grouped einsum.
//
// The contraction runs on v_mfma_scale_f32_16x16x128_f8f6f4: one instruction
// multiplies a 16x128 FP8 tile by a 128x16 FP8 tile, applies one E8M0 scale
// per lane to each operand, and accumulates in fp32.  Operand layout (checked
// on the hardware with one-hot inputs): lane l holds row l%16; with q = l/16,
// its first 16 bytes are K [16q, 16q+16) and its last 16 bytes K
// [64+16q, 64+16q+16), and its scale byte covers the 32-K block q.  A
// 128-wide scale group covers an instruction's whole K, so for the wo_a GEMM
// all four lanes of a row pass the same byte and any K order common to both
// operands is correct; the block-32 GEMM of the MXFP8 linear needs the exact
// order above.  The weight is the MFMA's
// first operand and the activation its second, so each lane's four fp32
// results are four consecutive n of one token: one 8-byte BF16 store.
//
// FNUZ activations: an FNUZ code c times 2^s equals the OCP code c times
// 2^(s-1) (the FNUZ grid is the OCP grid halved), so FNUZ bytes are fed to
// the OCP MFMA with their scale byte lowered by one (0xFF stays NaN; 0 cannot
// go lower and is kept -- the block is then 2x too large, below 2^-119).
//
// Two kernels:
//  * large: 256 (t) x 256 (n) tiles, 4 waves of 128x128, K-steps of 128.  A
//    and W tiles go global -> LDS by LDS-DMA (global_load_lds_dwordx4, no
//    VGPR staging) into a 2-stage ring; 16-byte chunks are XOR-swizzled so
//    that the MFMA operand reads (two ds_read_b128 per operand) are bank
//    conflict free.  Tiles are mapped to workgroups XCD-aware: the 8 XCDs
//    each own a contiguous range of tiles, n fastest, so the n-tiles sharing
//    one activation panel run together on one XCD's L2.
//  * small-T (T <= 64, decode and the MXFP8 linear): one workgroup per
//    (g, 16*NT n) with all T rows; the 4 waves split K and reduce through LDS.
//    Operands stream straight from global memory (weight-bandwidth bound).
#include "common.hpp"

namespace mx {

namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void_t;

constexpr int kFmtFp8 = 0;   // MFMA operand format code: FP8 (OCP e4m3)

__device__ __forceinline__ v4f mfma_scaled(const v8i& a, const v8i& b, const v4f& c, int sa, int sb) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, kFmtFp8, kFmtFp8, 0, sa, 0, sb);
}

__device__ __forceinline__ v8i make_v8i(const uint4 lo, const uint4 hi) {
  v8i r;
  r[0] = lo.x; r[1] = lo.y; r[2] = lo.z; r[3] = lo.w;
  r[4] = hi.x; r[5] = hi.y; r[6] = hi.z; r[7] = hi.w;
  return r;
}

// FNUZ scale byte -> the OCP scale byte of the same values.
__device__ __forceinline__ int fnuz_scale_to_ocp(int s) { return (s == 0 || s == 0xFF) ? s : s - 1; }

__device__ __forceinline__ uint2 pack4_bf16(const v4f& v) {
  return make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
}

// ------------------------------------------------------------- large tiles

constexpr int kLT = 256;            // tile rows along t
constexpr int kLN = 256;            // tile rows along n
constexpr int kBK = 128;            // K bytes per step
constexpr int kRowChunks = kBK / 16;
constexpr int kTileBytes = kLT * kBK;   // 32 KiB per operand per stage

// physical 16-byte chunk of logical chunk c in row r: conflict free for 8
// consecutive rows (32 banks) and for 16 consecutive rows (64 banks)
__device__ __forceinline__ int swz(int r) { return ((r >> 1) ^ ((r & 1) << 2)) & 7; }

struct LargeArgs {
  const uint8_t* a;      // [T, G, K]
  const uint8_t* sa;     // [T, G, K/128]
  const uint8_t* w;      // [G, N, K]
  const uint8_t* sw;     // [G, N, K/128]
  uint16_t* out;         // [T, G, N]
  int T, G, N, K;
  int tiles_t, tiles_n, total_tiles, per_xcd;
};

constexpr int kScaleWin = 32;    // K-steps whose scales are staged in LDS at once

template <bool A_FNUZ>
__global__ __launch_bounds__(256, 1) void bmm_large_kernel(LargeArgs p) {
  __shared__ __attribute__((aligned(1024))) uint8_t lds[2][2][kTileBytes];   // [stage][W|A]
  // scales of a window of K-steps, [step][W|A][wave half][row % 16][row / 16 % 8]:
  // one 8-byte read gives a lane the scales of its 8 tiles
  __shared__ __attribute__((aligned(16))) uint8_t lds_sc[kScaleWin][2][2][16][8];

  // XCD-aware work id: workgroup i runs on XCD i % 8
  const int xcd = blockIdx.x & 7;
  const int work = xcd * p.per_xcd + (blockIdx.x >> 3);
  if (work >= p.total_tiles) return;
  const int nt = work % p.tiles_n;
  const int tt = (work / p.tiles_n) % p.tiles_t;
  const int g = work / (p.tiles_n * p.tiles_t);
  const int t0 = tt * kLT, n0 = nt * kLN;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wn = wave & 1, wt = wave >> 1;     // wave's 128x128 sub-tile
  const int KB = p.K / kBK;
  const uint32_t rowA = static_cast<uint32_t>(p.G) * p.K;   // activation row stride

  // LDS-DMA sources, relative to the tile's first row: wave `wave` fills
  // rows it*32 + wave*8 + lane/8 of each operand tile (it = 0..7), lane i ->
  // physical chunk i%8.  Rows past T or N re-read the last valid row.
  const uint8_t* baseW = p.w + (static_cast<size_t>(g) * p.N + n0) * p.K;
  const uint8_t* baseA = p.a + static_cast<size_t>(t0) * rowA + static_cast<size_t>(g) * p.K;
  const int dma_row = wave * 8 + (lane >> 3);
  const uint32_t dma_chunk = static_cast<uint32_t>((lane & 7) ^ swz(dma_row)) * 16;   // swz(r) = swz(r % 16)
  const int limW = p.N - 1 - n0, limA = p.T - 1 - t0;

  // operand reads inside a stage: row wn*128 + i*16 + lane%16; the swizzle
  // only depends on row % 16, so tile i sits at +i*16 rows
  // (lane group q reads the 16-byte chunks q and q + 4: K [16q, 16q+16) and
  // [64+16q, 64+16q+16), the hardware's operand order)
  const int r16 = lane & 15;
  const int q4 = lane >> 4;
  const int rdW = (wn * 128 + r16) * kBK;
  const int rdA = (wt * 128 + r16) * kBK;
  const int ch0 = (q4 ^ swz(r16)) << 4;
  const int ch1 = ((q4 + 4) ^ swz(r16)) << 4;

  // thread `tid` stages the scales of W row tid and A row tid
  const uint8_t* scW = p.sw + (static_cast<size_t>(g) * p.N + n0 + min(tid, limW)) * KB;
  const uint8_t* scA = p.sa + (static_cast<size_t>(t0 + min(tid, limA)) * p.G + g) * KB;
  uint8_t* sc_dst = &lds_sc[0][0][tid >> 7][tid & 15][(tid >> 4) & 7];
  constexpr int kScStep = 2 * 2 * 16 * 8;     // bytes per step in lds_sc
  constexpr int kScOp = 2 * 16 * 8;           // W -> A offset

  v4f acc[8][8];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

  auto issue = [&](int kt, int stage) {
    const uint32_t koff = static_cast<uint32_t>(kt) * kBK + dma_chunk;
#pragma unroll
    for (int it = 0; it < 8; ++it) {
      const int r = it * 32 + dma_row;
      const uint8_t* gw = baseW + static_cast<uint32_t>(min(r, limW)) * static_cast<uint32_t>(p.K) + koff;
      const uint8_t* ga = baseA + static_cast<uint32_t>(min(r, limA)) * rowA + koff;
      __builtin_amdgcn_global_load_lds(gw, (lds_void_t*)(&lds[stage][0][(it * 32 + wave * 8) * kBK]), 16, 0, 0);
      __builtin_amdgcn_global_load_lds(ga, (lds_void_t*)(&lds[stage][1][(it * 32 + wave * 8) * kBK]), 16, 0, 0);
    }
  };

  issue(0, 0);
  for (int kt = 0; kt < KB; ++kt) {
    const int stage = kt & 1;
    if (kt % kScaleWin == 0) {
      __syncthreads();                 // everyone is done with the previous window
      const int n = min(kScaleWin, KB - kt);
      if ((KB & 3) == 0) {
        for (int s4 = 0; s4 < n; s4 += 4) {
          const uint32_t vw = *reinterpret_cast<const uint32_t*>(scW + kt + s4);
          const uint32_t va = *reinterpret_cast<const uint32_t*>(scA + kt + s4);
#pragma unroll
          for (int b = 0; b < 4; ++b) {
            const int sa = (va >> (8 * b)) & 0xFF;
            sc_dst[(s4 + b) * kScStep] = static_cast<uint8_t>(vw >> (8 * b));
            sc_dst[(s4 + b) * kScStep + kScOp] = static_cast<uint8_t>(A_FNUZ ? fnuz_scale_to_ocp(sa) : sa);
          }
        }
      } else {
        for (int s = 0; s < n; ++s) {
          const int sa = scA[kt + s];
          sc_dst[s * kScStep] = scW[kt + s];
          sc_dst[s * kScStep + kScOp] = static_cast<uint8_t>(A_FNUZ ? fnuz_scale_to_ocp(sa) : sa);
        }
      }
    }
    // this wave's DMA into `stage` has landed; after the barrier everyone's
    // has, and everyone is done reading the other stage (step kt-1)
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();

    // all operands of this step into registers first ...
    const int ks = kt % kScaleWin;
    const uint2 swv = *reinterpret_cast<const uint2*>(&lds_sc[ks][0][wn][r16][0]);
    const uint2 sav = *reinterpret_cast<const uint2*>(&lds_sc[ks][1][wt][r16][0]);
    v8i fa[8], fw[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const uint8_t* q = &lds[stage][1][rdA + j * 16 * kBK];
      fa[j] = make_v8i(*reinterpret_cast<const uint4*>(q + ch0), *reinterpret_cast<const uint4*>(q + ch1));
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint8_t* q = &lds[stage][0][rdW + i * 16 * kBK];
      fw[i] = make_v8i(*reinterpret_cast<const uint4*>(q + ch0), *reinterpret_cast<const uint4*>(q + ch1));
    }
    // ... then the next step's DMA (after the reads in program order, so the
    // compiler has no LDS write-after-read hazard to wait for) ...
    if (kt + 1 < KB) issue(kt + 1, stage ^ 1);
    // ... then the 64 MFMAs while it flies
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int sw_i = static_cast<int>(((i < 4 ? swv.x : swv.y) >> (8 * (i & 3))) & 0xFF);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int sa_j = static_cast<int>(((j < 4 ? sav.x : sav.y) >> (8 * (j & 3))) & 0xFF);
        acc[i][j] = mfma_scaled(fw[i], fa[j], acc[i][j], sw_i, sa_j);
      }
    }
  }

  // epilogue: lane holds out[t][n..n+3] for t = col, n = 4*(lane/16) + r
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int t = t0 + wt * 128 + j * 16 + r16;
    if (t >= p.T) continue;
    uint16_t* orow = p.out + (static_cast<size_t>(t) * p.G + g) * p.N;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int n = n0 + wn * 128 + i * 16 + (lane >> 4) * 4;
      if (n < p.N) *reinterpret_cast<uint2*>(orow + n) = pack4_bf16(acc[i][j]);
    }
  }
}

// ----------------------------------------------------------- small T (<= 64)

struct SmallArgs {
  const uint8_t* a;      // [T, G, K]  (G = 1 for the linear)
  const uint8_t* sa;     // [T, G, K/SB]
  const uint8_t* w;      // [G, N, K]
  const uint8_t* sw;     // [G, N, K/SB]
  uint16_t* out;         // [T, G, N]
  int T, G, N, K;
  int n_groups;          // ceil(N / (16*NT))
};

// One workgroup: all T (<= 64) rows x 16*NT columns n of one group g.  Wave w
// takes K-steps w, w+4, ...; partial sums meet in LDS.
template <int NT, int SB, bool A_FNUZ>
__global__ __launch_bounds__(256) void bmm_small_kernel(SmallArgs p) {
  __shared__ float red[4][NT * 4][4][64];   // [wave][tile][reg][lane]
  const int g = blockIdx.x / p.n_groups;
  const int n0 = (blockIdx.x % p.n_groups) * (16 * NT);
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int KB = p.K / kBK;
  const int SPK = p.K / SB;                   // scale bytes per row
  const int kq = lane >> 4;                   // lane group: K bytes 16kq.. and 64+16kq.., scale block kq
  const size_t rowA = static_cast<size_t>(p.G) * p.K;

  const uint8_t* pw[NT];
  const uint8_t* psw[NT];
#pragma unroll
  for (int i = 0; i < NT; ++i) {
    const int n = min(n0 + i * 16 + (lane & 15), p.N - 1);
    pw[i] = p.w + (static_cast<size_t>(g) * p.N + n) * p.K + kq * 16;
    psw[i] = p.sw + (static_cast<size_t>(g) * p.N + n) * SPK + (SB == 32 ? kq : 0);
  }
  const uint8_t* pa[4];
  const uint8_t* psa[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int t = min(j * 16 + (lane & 15), p.T - 1);
    pa[j] = p.a + static_cast<size_t>(t) * rowA + static_cast<size_t>(g) * p.K + kq * 16;
    psa[j] = p.sa + (static_cast<size_t>(t) * p.G + g) * SPK + (SB == 32 ? kq : 0);
  }
  constexpr int kScalesPerStep = kBK / SB;

  v4f acc[NT][4];
#pragma unroll
  for (int i = 0; i < NT; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

  for (int kt = wave; kt < KB; kt += 4) {
    const size_t ko = static_cast<size_t>(kt) * kBK;
    v8i fw[NT], fa[4];
    int s_w[NT], s_a[4];
#pragma unroll
    for (int i = 0; i < NT; ++i) {
      fw[i] = make_v8i(*reinterpret_cast<const uint4*>(pw[i] + ko), *reinterpret_cast<const uint4*>(pw[i] + ko + 64));
      s_w[i] = psw[i][kt * kScalesPerStep];
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      fa[j] = make_v8i(*reinterpret_cast<const uint4*>(pa[j] + ko), *reinterpret_cast<const uint4*>(pa[j] + ko + 64));
      const int s = psa[j][kt * kScalesPerStep];
      s_a[j] = A_FNUZ ? fnuz_scale_to_ocp(s) : s;
    }
#pragma unroll
    for (int i = 0; i < NT; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = mfma_scaled(fw[i], fa[j], acc[i][j], s_w[i], s_a[j]);
  }

#pragma unroll
  for (int i = 0; i < NT; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) red[wave][i * 4 + j][r][lane] = acc[i][j][r];
  __syncthreads();
  // wave w finalises tiles w, w+4, ...
  for (int tile = wave; tile < NT * 4; tile += 4) {
    const int i = tile / 4, j = tile % 4;
    v4f s;
#pragma unroll
    for (int r = 0; r < 4; ++r)
      s[r] = red[0][tile][r][lane] + red[1][tile][r][lane] + red[2][tile][r][lane] + red[3][tile][r][lane];
    const int t = j * 16 + (lane & 15);
    const int n = n0 + i * 16 + (lane >> 4) * 4;
    if (t < p.T && n < p.N)
      *reinterpret_cast<uint2*>(p.out + (static_cast<size_t>(t) * p.G + g) * p.N + n) = pack4_bf16(s);
  }
}

template <int NT, int SB>
void launch_small(const SmallArgs& a, bool fnuz, hipStream_t s) {
  const int grid = a.G * a.n_groups;
  if (fnuz)
    bmm_small_kernel<NT, SB, true><<<grid, 256, 0, s>>>(a);
  else
    bmm_small_kernel<NT, SB, false><<<grid, 256, 0, s>>>(a);
}

}  // namespace

// Batched GEMM dispatch (arguments validated by the caller).
mx_status launch_bmm(const uint8_t* a, const uint8_t* sa, int32_t a_fmt, const uint8_t* w, const uint8_t* sw,
                     void* out, int64_t T, int32_t G, int32_t N, int32_t K, hipStream_t stream) {
  if (T == 0) return MX_OK;
  const bool fnuz = a_fmt == MX_FP8_E4M3_FNUZ;
  if (T <= 64) {
    SmallArgs s{a, sa, w, sw, static_cast<uint16_t*>(out), static_cast<int>(T), G, N, K, (N + 63) / 64};
    launch_small<4, 128>(s, fnuz, stream);
    count(C_BMM_SMALL);
    return launch_status("mx_bmm_a8w8_mxscale (small T)");
  }
  LargeArgs p;
  p.a = a; p.sa = sa; p.w = w; p.sw = sw;
  p.out = static_cast<uint16_t*>(out);
  p.T = static_cast<int>(T); p.G = G; p.N = N; p.K = K;
  p.tiles_t = static_cast<int>((T + kLT - 1) / kLT);
  p.tiles_n = (N + kLN - 1) / kLN;
  p.total_tiles = p.tiles_t * p.tiles_n * G;
  p.per_xcd = (p.total_tiles + 7) / 8;
  const int grid = p.per_xcd * 8;
  if (fnuz)
    bmm_large_kernel<true><<<grid, 256, 0, stream>>>(p);
  else
    bmm_large_kernel<false><<<grid, 256, 0, stream>>>(p);
  count(C_BMM_LARGE);
  return launch_status("mx_bmm_a8w8_mxscale");
}

// Block-32 scaled FP8 GEMM for the MXFP8 linear: out[M,N] = xq[M,K] * W[N,K]^T
// with scales [M,K/32] and [N,K/32], M <= 64.
mx_status launch_gemm_mx32(const uint8_t* xq, const uint8_t* xs, const uint8_t* w, const uint8_t* sw, void* out,
                           int64_t M, int64_t N, int64_t K, hipStream_t stream) {
  if (M == 0 || N == 0) return MX_OK;
  SmallArgs s{xq, xs, w, sw, static_cast<uint16_t*>(out), static_cast<int>(M), 1, static_cast<int>(N),
              static_cast<int>(K), static_cast<int>((N + 15) / 16)};
  launch_small<1, 32>(s, false, stream);
  return launch_status("mx_linear (block-scaled FP8 GEMM)");
}

}  // namespace mx
