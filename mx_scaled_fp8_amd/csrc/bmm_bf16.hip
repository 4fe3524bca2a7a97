// Batched BF16 GEMM: the BF16 arm of wo_a (gfx950).
//
// "[ROCm][DSV4][Perf] Use FP8 WO_A output projection", Summary and Related
// work: before the FP8 path, wo_a ran as an inverse RoPE followed by a BF16
// grouped einsum over a BF16 copy of the weight made once at load, and that
// path stays as the fallback the FP8 one is measured against.  Here
// out[t, g, n] = sum_k x[t, g, k] * W[g, n, k] with BF16 x [T, G, K] and
// W [G, N, K], fp32 accumulation, BF16 output (nearest even).
//
// T > 64: the machinery of the FP8 GEMM's persistent kernel without the
// scales.  256 (t) x 256 (n) tiles, 4 waves of 128 x 128 on
// v_mfma_f32_32x32x16_bf16 with the accumulators in AGPRs; K moves 128 bytes
// (64 BF16) per stage, global -> LDS by LDS-DMA into two stage buffers with
// XOR-swizzled 16-byte chunks; one barrier per stage, the second half's
// fragments read during the first half's MFMAs; one resident workgroup per
// compute unit walks its XCD's tiles and fetches the next tile's first two
// stages during the current tile's last two.  The 32-byte fragment a lane
// reads per operand is here two 16-byte BF16 fragments, one per MFMA: both
// operands split a stage's K the same way, which is all the sum needs.  A
// stage holds half the K of an FP8 stage at the same MFMA time (64 MFMAs of 8
// passes against 32 of 16), so the pipeline keeps its timing and moves twice
// the bytes per flop.
//
// T <= 64 (decode): the FP8 decode-batch kernel's LDS-DMA ring with BF16
// MFMAs for K of 512 to 4096, else the split-K BF16 kernel of the MXFP8
// linear, one launch over all groups.
#include <algorithm>
#include <type_traits>

#include "common.hpp"

namespace mx {

mx_status launch_gemm_bf16_strided(const void* x, const void* w, void* out, int64_t M, int64_t N, int64_t K,
                                   int32_t G, int64_t ldx, int64_t ldo, hipStream_t stream);
bool launch_bmm_bf16_decode(const void* x, const void* w, void* out, int64_t T, int32_t G, int32_t N, int32_t K,
                            hipStream_t stream);

namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void lds_void_t;

constexpr int kTile = 256;               // tile rows along t and along n
constexpr int kRowBytes = 128;           // bytes of a row per stage (64 BF16)
constexpr int kStageK = kRowBytes / 2;   // K elements per stage
constexpr int kOpBytes = kTile * kRowBytes;

struct Bf16Args {
  const uint8_t* x;      // [T, G, K] BF16
  const uint8_t* w;      // [G, N, K] BF16
  uint16_t* out;         // [T, G, N] BF16
  int T, G, N, K;        // K in elements
  int tiles_t, tiles_n, total_tiles, per_xcd, wg_per_xcd;
};

__device__ __forceinline__ v8i make_v8i(const uint4 lo, const uint4 hi) {
  v8i r;
  r[0] = lo.x; r[1] = lo.y; r[2] = lo.z; r[3] = lo.w;
  r[4] = hi.x; r[5] = hi.y; r[6] = hi.z; r[7] = hi.w;
  return r;
}

// 16-byte half H of a 32-byte fragment, as 8 BF16
template <int H>
__device__ __forceinline__ v8bf half_of(const v8i& v) {
  const v4i h = __builtin_shufflevector(v, v, 4 * H, 4 * H + 1, 4 * H + 2, 4 * H + 3);
  return __builtin_bit_cast(v8bf, h);
}

// physical 16-byte chunk of logical chunk c in a 128-byte row r is c ^ swz8(r)
__device__ __forceinline__ int swz8(int r) { return ((r >> 1) ^ ((r & 1) << 2)) & 7; }

// W tile I times x tile J over K-piece H of the fragments; with FIRST the
// accumulator input is zero (the tile's first MFMA on this block).
template <int I, int J, int H, bool FIRST>
__device__ __forceinline__ void mfma_bf(v16f (&acc)[4][4], const v8i (&w)[4], const v8i (&a)[4]) {
  const v16f zero = {};
  acc[I][J] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(half_of<H>(w[I]), half_of<H>(a[J]), FIRST ? zero : acc[I][J],
                                                      0, 0, 0);
}

// the 16 blocks on K-piece H (only piece 0 may start the sums)
template <int H, bool FIRST>
__device__ __forceinline__ void mma_piece(v16f (&acc)[4][4], const v8i (&w)[4], const v8i (&a)[4]) {
  mfma_bf<0, 0, H, FIRST>(acc, w, a);
  mfma_bf<0, 1, H, FIRST>(acc, w, a);
  mfma_bf<1, 0, H, FIRST>(acc, w, a);
  mfma_bf<1, 1, H, FIRST>(acc, w, a);
  mfma_bf<0, 2, H, FIRST>(acc, w, a);
  mfma_bf<1, 2, H, FIRST>(acc, w, a);
  mfma_bf<2, 0, H, FIRST>(acc, w, a);
  mfma_bf<2, 1, H, FIRST>(acc, w, a);
  mfma_bf<2, 2, H, FIRST>(acc, w, a);
  mfma_bf<0, 3, H, FIRST>(acc, w, a);
  mfma_bf<1, 3, H, FIRST>(acc, w, a);
  mfma_bf<2, 3, H, FIRST>(acc, w, a);
  mfma_bf<3, 0, H, FIRST>(acc, w, a);
  mfma_bf<3, 1, H, FIRST>(acc, w, a);
  mfma_bf<3, 2, H, FIRST>(acc, w, a);
  mfma_bf<3, 3, H, FIRST>(acc, w, a);
}

__global__ __launch_bounds__(256, 1) void bmm_bf16_persistent_kernel(Bf16Args p) {
  __shared__ __attribute__((aligned(1024))) uint8_t st0[2 * kOpBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t st1[2 * kOpBytes];

  const int xcd = blockIdx.x & 7;
  const int slot = blockIdx.x >> 3;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wn = wave & 1, wt = wave >> 1;
  const int KB = p.K / kStageK;                // even, >= 2
  const uint32_t rowW = static_cast<uint32_t>(p.K) * 2;
  const uint32_t rowA = static_cast<uint32_t>(p.G) * rowW;

  // tile r of this workgroup; false past the end of its XCD's range
  auto tile_at = [&](int r, int& g, int& t0, int& n0, int& kb0) {
    const int li = slot + r * p.wg_per_xcd;
    const int work = xcd * p.per_xcd + li;
    if (li >= p.per_xcd || work >= p.total_tiles) return false;
    const int nt = work % p.tiles_n;
    const int tt = (work / p.tiles_n) % p.tiles_t;
    g = work / (p.tiles_n * p.tiles_t);
    t0 = tt * kTile;
    n0 = nt * kTile;
    kb0 = (tt + nt) % KB;                      // K rotation: tiles sharing an operand stay near in K
    return true;
  };

  // ---- DMA of the stages of one tile
  const int dma_row = wave * 8 + (lane >> 3);
  const uint32_t dma_chunk = static_cast<uint32_t>((lane & 7) ^ swz8(dma_row)) * 16;
  uint32_t offW[8], offA[8];
  const uint8_t* dW;
  const uint8_t* dA;
  int dkb0;
  auto set_dma_tile = [&](int g, int t0, int n0, int kb0) {
    dW = p.w + (static_cast<size_t>(g) * p.N + n0) * rowW;
    dA = p.x + static_cast<size_t>(t0) * rowA + static_cast<size_t>(g) * rowW;
    dkb0 = kb0;
    const int limW = p.N - 1 - n0, limA = p.T - 1 - t0;   // rows past N or T re-read the last row
#pragma unroll
    for (int it = 0; it < 8; ++it) {
      const int r = it * 32 + dma_row;
      offW[it] = static_cast<uint32_t>(min(r, limW)) * rowW + dma_chunk;
      offA[it] = static_cast<uint32_t>(min(r, limA)) * rowA + dma_chunk;
    }
  };
  auto issue = [&](uint8_t* buf, int kb) {   // kb < KB
    int kr = kb + dkb0;
    kr -= kr >= KB ? KB : 0;
    const uint8_t* bW = dW + static_cast<uint32_t>(kr) * kRowBytes;
    const uint8_t* bA = dA + static_cast<uint32_t>(kr) * kRowBytes;
#pragma unroll
    for (int it = 0; it < 8; ++it) {
      const int rb = it * 32 + wave * 8;
      __builtin_amdgcn_global_load_lds(bW + offW[it], (lds_void_t*)(buf + rb * kRowBytes), 16, 0, 0);
      __builtin_amdgcn_global_load_lds(bA + offA[it], (lds_void_t*)(buf + kOpBytes + rb * kRowBytes), 16, 0, 0);
    }
  };

  // ---- fragments: lane (row r32, half q2) reads chunks {q2, q2 + 2} of a row
  // for the first 64 bytes of a stage and {4 + q2, 6 + q2} for the second
  const int r32 = lane & 31;
  const int q2 = lane >> 5;
  const int rdW = (wn * 128 + r32) * kRowBytes;
  const int rdA = kOpBytes + (wt * 128 + r32) * kRowBytes;
  const int sz = swz8(r32);
  const int ch00 = (q2 ^ sz) << 4, ch01 = ((q2 + 2) ^ sz) << 4;
  const int ch10 = ((4 + q2) ^ sz) << 4, ch11 = ((6 + q2) ^ sz) << 4;
  v8i fw[2][4], fa[2][4];
  auto read_frag = [&](const uint8_t* q, int c0, int c1) {
    return make_v8i(*reinterpret_cast<const uint4*>(q + c0), *reinterpret_cast<const uint4*>(q + c1));
  };
  auto read_half = [&](const uint8_t* buf, int c0, int c1, v8i (&w)[4], v8i (&a)[4]) {
    const uint8_t* qw = buf + rdW;
    const uint8_t* qa = buf + rdA;
    w[0] = read_frag(qw, c0, c1);
    a[0] = read_frag(qa, c0, c1);
    a[1] = read_frag(qa + 32 * kRowBytes, c0, c1);
    w[1] = read_frag(qw + 32 * kRowBytes, c0, c1);
    a[2] = read_frag(qa + 64 * kRowBytes, c0, c1);
    w[2] = read_frag(qw + 64 * kRowBytes, c0, c1);
    a[3] = read_frag(qa + 96 * kRowBytes, c0, c1);
    w[3] = read_frag(qw + 96 * kRowBytes, c0, c1);
  };
  v16f acc[4][4];
  auto pin_acc = [&]() {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) asm volatile("" ::"a"(acc[i][j]));
  };
  constexpr int kWaitAll = wait_vm(0);
  // the prologue leaves stage 1's DMA in flight: issue() is 8 row groups x 2
  // operands per wave
  constexpr int kWaitNewest16 = wait_vm(2 * (kTile / 32));
  static_assert(2 * (kTile / 32) == 16, "DMA instructions per stage");

  // front: MFMAs of a stage's first 64 bytes (32 of them) while its second
  // half is read from `cur`; then wait for everything and barrier.
  auto front = [&](const uint8_t* cur, auto first) {
    constexpr bool F = decltype(first)::value;
    __builtin_amdgcn_sched_barrier(0);
    mma_piece<0, F>(acc, fw[0], fa[0]);
    mma_piece<1, false>(acc, fw[0], fa[0]);
    read_half(cur, ch10, ch11, fw[1], fa[1]);
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one MFMA
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // one LDS read
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 16, 0);
    pin_acc();
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(kWaitAll);
    __builtin_amdgcn_s_barrier();
  };
  // back: DMA of stage `dma_kb` of the DMA tile into `cur`; MFMAs of the
  // second half; the next stage's first half read from `nxt`.
  auto back = [&](uint8_t* cur, const uint8_t* nxt, int dma_kb) {
    issue(cur, dma_kb);
    mma_piece<0, false>(acc, fw[1], fa[1]);
    mma_piece<1, false>(acc, fw[1], fa[1]);
    read_half(nxt, ch00, ch01, fw[0], fa[0]);
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);   // one DMA per two MFMAs
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    }
    pin_acc();
    __builtin_amdgcn_sched_barrier(0);
  };

  // ---- first tile: prologue
  int cg, ct0, cn0, ckb0;
  if (!tile_at(0, cg, ct0, cn0, ckb0)) return;
  set_dma_tile(cg, ct0, cn0, ckb0);
  issue(st0, 0);
  issue(st1, 1);
  __builtin_amdgcn_s_waitcnt(kWaitNewest16);
  __builtin_amdgcn_s_barrier();
  read_half(st0, ch00, ch01, fw[0], fa[0]);

  const std::true_type yes{};
  const std::false_type no{};
  for (int r = 0;; ++r) {
    front(st0, yes);                             // stage 0 (first half): starts the sums
    for (int kb = 0; kb + 2 < KB; kb += 2) {     // stages kb, kb+1 finish; kb+2 begins
      back(st0, st1, kb + 2);
      front(st1, no);
      back(st1, st0, kb + 3);
      front(st0, no);
    }
    // stages KB-2 (begun) and KB-1 remain; fetch the next tile meanwhile
    int ng, nt0, nn0, nkb0;
    const bool more = tile_at(r + 1, ng, nt0, nn0, nkb0);
    if (!more) {                                 // refetch this tile: harmless, never read
      ng = cg;
      nt0 = ct0;
      nn0 = cn0;
      nkb0 = ckb0;
    }
    set_dma_tile(ng, nt0, nn0, nkb0);
    back(st0, st1, 0);                           // next tile's stage 0 -> st0
    front(st1, no);
    back(st1, st0, 1);                           // next tile's stage 1 -> st1; its stage 0 half 0

    // epilogue: 32x32 C layout (lane column r32 = t, rows n); permlane32_swap
    // pairs the lane halves so that each lane stores 8 consecutive n
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int t = ct0 + wt * 128 + j * 32 + r32;
      uint16_t* orow = p.out + (static_cast<size_t>(t) * p.G + cg) * p.N;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const v16f& v = acc[i][j];
#pragma unroll
        for (int pp = 0; pp < 2; ++pp) {
          const uint32_t x0 = pack_bf16x2(v[8 * pp + 0], v[8 * pp + 1]), x1 = pack_bf16x2(v[8 * pp + 2], v[8 * pp + 3]);
          const uint32_t y0 = pack_bf16x2(v[8 * pp + 4], v[8 * pp + 5]), y1 = pack_bf16x2(v[8 * pp + 6], v[8 * pp + 7]);
          const auto s0 = __builtin_amdgcn_permlane32_swap(x0, y0, false, false);
          const auto s1 = __builtin_amdgcn_permlane32_swap(x1, y1, false, false);
          const int n = cn0 + wn * 128 + i * 32 + pp * 16 + q2 * 8;
          if (t < p.T && n < p.N)
            *reinterpret_cast<uint4*>(orow + n) = make_uint4(s0[0], s1[0], s0[1], s1[1]);
        }
      }
    }
    if (!more) break;
    cg = ng;
    ct0 = nt0;
    cn0 = nn0;
    ckb0 = nkb0;
  }
  __builtin_amdgcn_s_waitcnt(kWaitAll);          // no DMA outlives the workgroup
}

}  // namespace

// Batched BF16 GEMM dispatch (arguments validated by the caller: K % 128 == 0,
// N % 16 == 0, x, w, out 16-byte aligned).
mx_status launch_bmm_bf16(const void* x, const void* w, void* out, int64_t T, int32_t G, int32_t N, int32_t K,
                          hipStream_t stream) {
  if (T == 0) return MX_OK;
  const int cus = device_cu_count();
  if (T <= 64 && launch_bmm_bf16_decode(x, w, out, T, G, N, K, stream)) {
    count(C_BMM_BF16_SMALL);
    return launch_status("mx_bmm_bf16 (decode batch)");
  }
  if (T <= 64 || cus < 8) {
    count(C_BMM_BF16_SMALL);
    return launch_gemm_bf16_strided(x, w, out, T, N, K, G, static_cast<int64_t>(G) * K,
                                    static_cast<int64_t>(G) * N, stream);
  }
  Bf16Args p;
  p.x = static_cast<const uint8_t*>(x);
  p.w = static_cast<const uint8_t*>(w);
  p.out = static_cast<uint16_t*>(out);
  p.T = static_cast<int>(T); p.G = G; p.N = N; p.K = K;
  p.tiles_t = static_cast<int>((T + kTile - 1) / kTile);
  p.tiles_n = (N + kTile - 1) / kTile;
  p.total_tiles = p.tiles_t * p.tiles_n * G;
  p.per_xcd = (p.total_tiles + 7) / 8;
  // one resident workgroup per compute unit, XCD-major (workgroup i runs on XCD i % 8)
  p.wg_per_xcd = std::min(p.per_xcd, cus / 8);
  bmm_bf16_persistent_kernel<<<p.wg_per_xcd * 8, 256, 0, stream>>>(p);
  count(C_BMM_BF16_LARGE);
  return launch_status("mx_bmm_bf16");
}

}  // namespace mx
