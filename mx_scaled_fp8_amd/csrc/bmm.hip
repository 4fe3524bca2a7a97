// Batched a8w8 GEMM with E8M0 block scales on CDNA4 block-scaled FP8 MFMA (gfx950).
//
// "[ROCm][DSV4][Perf] Use FP8 WO_A output projection", Summary item 2: the
// quantised activation A [T, G, K] (E8M0 scale per 128 consecutive K) is
// multiplied with the checkpoint's FP8 weight W [G, N, K] (E8M0 scale per
// (g, n, 128-K block)), out[t, g, n] = sum_k A*sa * W*sw, in place of the BF16
// grouped einsum.
//
// Small-T kernels run on v_mfma_scale_f32_16x16x128_f8f6f4: one instruction
// multiplies a 16x128 FP8 tile by a 128x16 FP8 tile, applies one E8M0 scale
// per lane to each operand, and accumulates in fp32.  Operand layout (checked
// on the hardware with one-hot inputs): lane l holds row l%16; with q = l/16,
// its first 16 bytes are K [16q, 16q+16) and its last 16 bytes K
// [64+16q, 64+16q+16), and its scale byte covers the 32-K block q.  A
// 128-wide scale group covers an instruction's whole K, so for the wo_a GEMM
// all four lanes of a row pass the same byte and any K order common to both
// operands is correct; the block-32 GEMM of the MXFP8 linear needs the exact
// order above.  The weight is the MFMA's first operand and the activation its
// second, so each lane's four fp32 results are four consecutive n of one
// token: one 8-byte BF16 store.  The large-tile kernels run on the 32x32x64
// form of the same instruction (4 x 4 tiles per wave).
//
// FNUZ activations: an FNUZ code c times 2^s equals the OCP code c times
// 2^(s-1) (the FNUZ grid is the OCP grid halved), so FNUZ bytes are fed to
// the OCP MFMA with their scale byte lowered by one (0xFF stays NaN; 0 cannot
// go lower and is kept -- the block is then 2x too large, below 2^-119).
//
// Kernels:
//  * bmm_large_kernel / bmm_persistent_kernel (T > 64): 256 (t) x 256 (n)
//    tiles, 4 waves of 128x128, K-steps of 128.  A and W tiles go global ->
//    LDS by LDS-DMA (global_load_lds_dwordx4, no VGPR staging) into a 2-stage
//    ring; 16-byte chunks are XOR-swizzled so that the MFMA operand reads
//    (two ds_read_b128 per operand) are bank conflict free.  Tiles are mapped
//    to workgroups XCD-aware: the 8 XCDs each own a contiguous range of
//    tiles, n fastest, so the n-tiles sharing one activation panel run
//    together on one XCD's L2.  The persistent kernel (K = 2048 or 4096)
//    keeps one workgroup per compute unit, runs the stage pipeline across
//    tile boundaries and stores each tile through LDS as 128-byte row pieces
//    while the next tile's first MFMAs run.
//  * bmm_decode_kernel (T <= 64, K of 1024 to 8192): one workgroup per
//    (g, 64 n) with all T rows; both operands through an LDS-DMA ring of 4
//    K-steps; the waves split n.  A BF16 mode serves the BF16 arm.
//  * bmm_small_kernel (T <= 64, other K): the 4 waves split K, operands
//    double-buffered in registers, partial sums reduced through LDS.
//  * gemm_mx32_dma_kernel: the MXFP8 linear's block-32 GEMM (M <= 64) on the
//    decode kernel's ring, for the shapes the weight-resident kernels of
//    linear_mx32.hip do not take; more rows run on bmm_large_kernel with
//    block-32 scales.
#include <algorithm>
#include <type_traits>

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
//
// 256 (t) x 256 (n) workgroup tile, 4 waves of 128 x 128, on
// v_mfma_scale_f32_32x32x64_f8f6f4 (4 x 4 MFMA tiles per wave, accumulators
// in AGPRs).  K advances 128 bytes per stage, so every row of a tile is read
// from L2 as whole 128-byte lines (64-byte pieces cost a quarter of the L2 to
// CU bandwidth).  Two stages live in LDS as separate __shared__ arrays and the
// stage loop is unrolled by two, so every access names its buffer statically
// and the compiler can see that the DMA filling the other stage does not alias
// the fragments being read.  Inside a stage the two 64-K halves are double
// buffered in registers: the reads of the second half overlap the MFMAs of
// the first.

constexpr int kLT = 256;                 // tile rows along t
constexpr int kLN = 256;                 // tile rows along n
constexpr int kBK = 128;                 // K bytes per stage = one scale group
constexpr int kOpBytes = kLT * kBK;      // 32 KiB per operand per stage
constexpr int kScaleWin = 32;            // stages whose scales are staged in LDS at once
// LDS-DMA instructions a wave issues per stage: rows are moved 8 per
// instruction per wave (32 per row group over the 4 waves), for both operands
constexpr int kLargeDmaPerStage = 2 * (kLT / 32);
static_assert(kLT == kLN && kLargeDmaPerStage == 16, "DMA instructions per stage");
// stores a wave issues in the persistent kernel's folded epilogue: 8 chunks
// of 32 rows, each leaving as 4 instructions of 8 rows x 128 bytes
constexpr int kFoldStores = 8 * 4;

typedef float v16f __attribute__((ext_vector_type(16)));

// physical 16-byte chunk of logical chunk c in a 128-byte row r is c ^ swz8(r):
// conflict free for 8 consecutive rows (32 banks) and for 16 (64 banks)
__device__ __forceinline__ int swz8(int r) { return ((r >> 1) ^ ((r & 1) << 2)) & 7; }

struct LargeArgs {
  const uint8_t* a;      // [T, G, K]
  const uint8_t* sa;     // [T, G, K/128]
  const uint8_t* w;      // [G, N, K]
  const uint8_t* sw;     // [G, N, K/128]
  uint16_t* out;         // [T, G, N]
  int T, G, N, K;
  int tiles_t, tiles_n, total_tiles, per_xcd;
  int wg_per_xcd;        // persistent kernel: resident workgroups per XCD
};

// One 32x32x64 block-scaled MFMA of the large kernel: W tile I times A tile
// J.  The scale operands are 4-byte words holding the scales of tiles 0..3;
// the byte-select operands pick byte I of the W word and byte J of the A word.
// With FIRST the accumulator input is zero: the first MFMA of a tile starts
// its sum, so the accumulators need no clearing between tiles.
template <int I, int J, bool FIRST = false>
__device__ __forceinline__ void mfma_ij(v16f (&acc)[4][4], const v8i (&w)[4], const v8i (&a)[4], uint32_t swv,
                                        uint32_t sav) {
  const v16f zero = {};
  acc[I][J] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(w[I], a[J], FIRST ? zero : acc[I][J], kFmtFp8,
                                                             kFmtFp8, I, static_cast<int>(swv), J,
                                                             static_cast<int>(sav));
}

// SB is the K extent of one scale byte: 128 (the wo_a layout, one scale per
// stage and row) or 32 (the MXFP8 linear's blocks, four per stage and row).
// With 32, the scale a 32x32x64 MFMA applies to the K-block of lane group q
// is the block's own: in 64-K half h of a stage, lane group q passes block
// 2h + q (the lane data layout is the same for both: byte j of a half is the
// instruction's k = j).
template <bool A_FNUZ, int SB>
__global__ __launch_bounds__(256, 1) void bmm_large_kernel(LargeArgs p) {
  static_assert(SB == 128 || SB == 32, "scale block");
  constexpr int kSPS = kBK / SB;                 // scale blocks per stage and row: 1 or 4
  constexpr int kWin = kScaleWin / kSPS;         // stages per scale window: 32 or 8
  // stage buffers: [W tile 256 x 128 B | A tile 256 x 128 B]
  __shared__ __attribute__((aligned(1024))) uint8_t st0[2 * kOpBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t st1[2 * kOpBytes];
  // scales of a window of stages, [stage][block][W|A][wave half][row % 32][tile]:
  // one 4-byte read gives a lane the scales of its 4 tiles of one operand
  __shared__ __attribute__((aligned(16))) uint8_t lds_sc[kWin][kSPS][2][2][32][4];

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
  const int KB = p.K / kBK;                    // stages
  // Tiles start their K loop at stage (tt + nt) mod KB: the workgroups that
  // share an XCD spread over a few neighbouring K offsets (so their rows do
  // not all hit one memory channel at once), while the tiles that share an
  // activation panel (same tt) or a weight tile (same nt) stay within a few
  // stages of each other and still find the shared rows in L2.  Rotation
  // needs every scale in one window, so it is used when K fits one.
  const int kb0 = KB <= kWin ? (tt + nt) % KB : 0;
  const uint32_t rowA = static_cast<uint32_t>(p.G) * p.K;   // activation row stride

  // LDS-DMA sources: wave `wave` fills rows it*32 + wave*8 + lane/8 (it =
  // 0..7) of each operand tile, lane i -> physical chunk i%8; rows past T or
  // N re-read the last valid row
  const uint8_t* baseW = p.w + (static_cast<size_t>(g) * p.N + n0) * p.K;
  const uint8_t* baseA = p.a + static_cast<size_t>(t0) * rowA + static_cast<size_t>(g) * p.K;
  const int dma_row = wave * 8 + (lane >> 3);
  const uint32_t dma_chunk = static_cast<uint32_t>((lane & 7) ^ swz8(dma_row)) * 16;   // swz8(r) = swz8(r % 16)
  const int limW = p.N - 1 - n0, limA = p.T - 1 - t0;
  uint32_t offW[8], offA[8];
#pragma unroll
  for (int it = 0; it < 8; ++it) {
    const int r = it * 32 + dma_row;
    offW[it] = static_cast<uint32_t>(min(r, limW)) * static_cast<uint32_t>(p.K) + dma_chunk;
    offA[it] = static_cast<uint32_t>(min(r, limA)) * rowA + dma_chunk;
  }
  auto issue = [&](uint8_t* buf, int kb) {   // kb >= KB re-reads the last stage
    int kr = min(kb, KB - 1) + kb0;
    kr -= kr >= KB ? KB : 0;
    // uniform base + 32-bit lane offset: the scalar-base addressing form
    const uint8_t* bW = baseW + static_cast<uint32_t>(kr) * kBK;
    const uint8_t* bA = baseA + static_cast<uint32_t>(kr) * kBK;
    // all weight rows, then all activation rows (as in bmm_persistent_kernel)
#pragma unroll
    for (int it = 0; it < 8; ++it)
      __builtin_amdgcn_global_load_lds(bW + offW[it], (lds_void_t*)(buf + (it * 32 + wave * 8) * kBK), 16, 0, 0);
#pragma unroll
    for (int it = 0; it < 8; ++it)
      __builtin_amdgcn_global_load_lds(bA + offA[it], (lds_void_t*)(buf + kOpBytes + (it * 32 + wave * 8) * kBK), 16,
                                       0, 0);
  };

  // fragment reads: row wn*128 + 32*i + lane%32 (W) / wt*128 + 32*j + lane%32
  // (A); for the 64-K half h, lane group q = lane/32 takes logical chunks
  // 4h + q and 4h + q + 2
  const int r32 = lane & 31;
  const int q2 = lane >> 5;
  const int rdW = (wn * 128 + r32) * kBK;
  const int rdA = kOpBytes + (wt * 128 + r32) * kBK;
  const int sz = swz8(r32);
  const int ch00 = (q2 ^ sz) << 4, ch01 = ((q2 + 2) ^ sz) << 4;        // half 0
  const int ch10 = ((4 + q2) ^ sz) << 4, ch11 = ((6 + q2) ^ sz) << 4;  // half 1

  v8i fw[2][4], fa[2][4];
  auto read_frag = [&](const uint8_t* q, int c0, int c1) {
    return make_v8i(*reinterpret_cast<const uint4*>(q + c0), *reinterpret_cast<const uint4*>(q + c1));
  };
  auto read_half = [&](const uint8_t* buf, int c0, int c1, v8i (&w)[4], v8i (&a)[4]) {
    const uint8_t* qw = buf + rdW;
    const uint8_t* qa = buf + rdA;
    w[0] = read_frag(qw, c0, c1);
    a[0] = read_frag(qa, c0, c1);
    a[1] = read_frag(qa + 32 * kBK, c0, c1);
    w[1] = read_frag(qw + 32 * kBK, c0, c1);
    a[2] = read_frag(qa + 64 * kBK, c0, c1);
    w[2] = read_frag(qw + 64 * kBK, c0, c1);
    a[3] = read_frag(qa + 96 * kBK, c0, c1);
    w[3] = read_frag(qw + 96 * kBK, c0, c1);
  };

  // scale staging: thread tid owns W row tid and A row tid.  LDS slot s of
  // the window holds stage s of the window (the actual stage, not the loop
  // index: with the rotation, loop stage kb reads slot (kb + kb0) mod KB).
  const int SPR = KB * kSPS;                   // scale bytes per row
  const uint8_t* scW = p.sw + (static_cast<size_t>(g) * p.N + n0 + min(tid, limW)) * SPR;
  const uint8_t* scA = p.sa + (static_cast<size_t>(t0 + min(tid, limA)) * p.G + g) * SPR;
  uint8_t* sc_dst = &lds_sc[0][0][0][tid >> 7][tid & 31][(tid >> 5) & 3];
  constexpr int kScBlk = 2 * 2 * 32 * 4;
  constexpr int kScStep = kSPS * kScBlk;
  constexpr int kScOp = 2 * 32 * 4;
  auto put_scales = [&](int s, int blk, uint32_t bw, uint32_t ba) {
    sc_dst[s * kScStep + blk * kScBlk] = static_cast<uint8_t>(bw);
    sc_dst[s * kScStep + blk * kScBlk + kScOp] =
        static_cast<uint8_t>(A_FNUZ ? fnuz_scale_to_ocp(static_cast<int>(ba)) : ba);
  };
  auto stage_scales_serial = [&](int first) {   // few registers: for the loop (K > one window)
    const int n = min(kWin, KB - first);
    for (int s = 0; s < n; ++s)
#pragma unroll
      for (int b = 0; b < kSPS; ++b) put_scales(s, b, scW[(first + s) * kSPS + b], scA[(first + s) * kSPS + b]);
  };
  auto stage_scales_first = [&]() {             // the first window, before the loop
    if (SB == 128 && (KB & 15) == 0 &&
        ((reinterpret_cast<uintptr_t>(scW) | reinterpret_cast<uintptr_t>(scA)) & 15) == 0) {
      // two 16-byte loads per row instead of 32 byte loads
      const uint4 w0 = *reinterpret_cast<const uint4*>(scW), a0 = *reinterpret_cast<const uint4*>(scA);
      uint4 w1 = make_uint4(0, 0, 0, 0), a1 = w1;
      if (KB >= 32) {
        w1 = *reinterpret_cast<const uint4*>(scW + 16);
        a1 = *reinterpret_cast<const uint4*>(scA + 16);
      }
      const uint32_t ww[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
      const uint32_t aw[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
#pragma unroll
      for (int s = 0; s < kScaleWin; ++s)        // slots past the last stage are never read
        put_scales(s, 0, (ww[s >> 2] >> (8 * (s & 3))) & 0xFF, (aw[s >> 2] >> (8 * (s & 3))) & 0xFF);
    } else {
      uint8_t bw[kWin * kSPS], ba[kWin * kSPS];  // all loads first, then the LDS writes
#pragma unroll
      for (int s = 0; s < kWin; ++s) {
        const int ks = min(s, KB - 1);           // slots past the last stage read a valid byte
#pragma unroll
        for (int b = 0; b < kSPS; ++b) {
          bw[s * kSPS + b] = scW[ks * kSPS + b];
          ba[s * kSPS + b] = scA[ks * kSPS + b];
        }
      }
#pragma unroll
      for (int s = 0; s < kWin; ++s)
#pragma unroll
        for (int b = 0; b < kSPS; ++b) put_scales(s, b, bw[s * kSPS + b], ba[s * kSPS + b]);
    }
  };
  // the scale words of loop stage kb: [h] for 64-K half h (one word for both
  // halves when SB = 128; block 2h + q2 of the stage when SB = 32)
  constexpr int H1 = kSPS == 1 ? 0 : 1;         // index of half 1's words
  auto read_scales = [&](int kb, uint32_t (&swv)[2], uint32_t (&sav)[2]) {
    int ks = kb + kb0;                           // the stage loop index kb covers
    ks -= ks >= KB ? KB : 0;
    const int s = ks & (kWin - 1);
    if constexpr (kSPS == 1) {
      swv[0] = *reinterpret_cast<const uint32_t*>(&lds_sc[s][0][0][wn][r32][0]);
      sav[0] = *reinterpret_cast<const uint32_t*>(&lds_sc[s][0][1][wt][r32][0]);
    } else {
      const int q = lane >> 5;
      swv[0] = *reinterpret_cast<const uint32_t*>(&lds_sc[s][q][0][wn][r32][0]);
      sav[0] = *reinterpret_cast<const uint32_t*>(&lds_sc[s][q][1][wt][r32][0]);
      swv[1] = *reinterpret_cast<const uint32_t*>(&lds_sc[s][2 + q][0][wn][r32][0]);
      sav[1] = *reinterpret_cast<const uint32_t*>(&lds_sc[s][2 + q][1][wt][r32][0]);
    }
  };

  v16f acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  // The 16 MFMAs of a 64-K half, in the order the fragments arrive (read_half
  // reads w0 a0 a1 w1 a2 w2 a3 w3), so that each MFMA waits only for the
  // fragments it uses.  The scale operand is the whole 4-byte word; the
  // instruction's byte select picks tile i's (j's) byte.
  auto mma_half = [&](const v8i (&w)[4], const v8i (&a)[4], uint32_t swv, uint32_t sav) {
    mfma_ij<0, 0>(acc, w, a, swv, sav);
    mfma_ij<0, 1>(acc, w, a, swv, sav);
    mfma_ij<1, 0>(acc, w, a, swv, sav);
    mfma_ij<1, 1>(acc, w, a, swv, sav);
    mfma_ij<0, 2>(acc, w, a, swv, sav);
    mfma_ij<1, 2>(acc, w, a, swv, sav);
    mfma_ij<2, 0>(acc, w, a, swv, sav);
    mfma_ij<2, 1>(acc, w, a, swv, sav);
    mfma_ij<2, 2>(acc, w, a, swv, sav);
    mfma_ij<0, 3>(acc, w, a, swv, sav);
    mfma_ij<1, 3>(acc, w, a, swv, sav);
    mfma_ij<2, 3>(acc, w, a, swv, sav);
    mfma_ij<3, 0>(acc, w, a, swv, sav);
    mfma_ij<3, 1>(acc, w, a, swv, sav);
    mfma_ij<3, 2>(acc, w, a, swv, sav);
    mfma_ij<3, 3>(acc, w, a, swv, sav);
  };
  // the MFMAs are pure, so without a use the compiler would sink them below
  // the following waits and barrier
  auto pin_acc = [&]() {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) asm volatile("" ::"a"(acc[i][j]));
  };

  // s_waitcnt immediates, from the instruction counts they stand for.  The
  // builtin, unlike inline asm, is seen by the compiler's own wait
  // insertion, so it does not add a second, later drain.
  constexpr int kWaitAll = wait_vm(0);
  // the prologue leaves stage 1's DMA in flight: issue() is kLT / 32 row
  // groups x 2 operands = kLargeDmaPerStage instructions per wave
  constexpr int kWaitNewest16 = wait_vm(kLargeDmaPerStage);
  constexpr int kWaitLgkm = kWaitLgkmOnly;

  // One stage, one barrier, in two parts.  On entry to front(kb) the first
  // 64-K half of stage kb is in registers (fw[0], fa[0]) with its scales,
  // `cur` holds stage kb and this wave's DMA of stage kb+1 into `nxt` may be
  // in flight.
  //   front: MFMAs of half 0 while reading half 1 of `cur`; wait for this
  //          wave's reads and DMA, barrier -- now stage kb+1 is in `nxt` and
  //          no wave reads `cur` any more;
  //   back:  refill `cur` with stage kb+2 by DMA, then the MFMAs of half 1
  //          while reading half 0 of stage kb+1 (and its scales) from `nxt`.
  // Fragment reads always overlap MFMAs and each DMA has one stage to land.
  // The loop runs back..front, so at its head (just after a barrier that
  // followed a full wait) no DMA is pending: the compiler then sees, in
  // straight-line code, that the reads of one buffer never alias the DMA into
  // the other and adds no wait of its own.
  uint32_t swv[2], sav[2];
  auto front = [&](const uint8_t* cur, int kb, bool new_window) {
    __builtin_amdgcn_sched_barrier(0);
    mma_half(fw[0], fa[0], swv[0], sav[0]);
    read_half(cur, ch10, ch11, fw[1], fa[1]);
    // reads early in the half (two per MFMA), so they land before the half ends
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one MFMA
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);   // two LDS reads
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);
    pin_acc();
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(kWaitAll);
    __builtin_amdgcn_s_barrier();
    if (new_window) {                        // K spans several windows: restage the scales
      stage_scales_serial(kb + 1);
      __builtin_amdgcn_s_waitcnt(kWaitLgkm);
      __builtin_amdgcn_s_barrier();
    }
  };
  auto back = [&](uint8_t* cur, const uint8_t* nxt, int kb, bool dma) {
    if (dma) issue(cur, kb + 2);
    uint32_t swv1[2], sav1[2];
    read_scales(kb + 1, swv1, sav1);
    mma_half(fw[1], fa[1], swv[H1], sav[H1]);
    read_half(nxt, ch00, ch01, fw[0], fa[0]);
    // one DMA instruction per MFMA: a burst of 16 would stall this wave on the
    // texture-address unit, which takes the four waves' DMA at about the rate
    // the MFMAs run; the LDS reads go early (two per MFMA)
#pragma unroll
    for (int k = 0; k < 9; ++k) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);   // one DMA
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);   // (the first two are the scales)
    }
#pragma unroll
    for (int k = 0; k < 7; ++k) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
    }
    pin_acc();
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int h = 0; h <= H1; ++h) {
      swv[h] = swv1[h];
      sav[h] = sav1[h];
    }
  };
  auto window_at = [&](int kb) {             // front(kb) restages scales for stage kb+1
    return KB > kWin && (kb + 1) % kWin == 0 && kb + 1 < KB;
  };

  // prologue: scales of the first window, stages 0 and 1 in flight, half 0 of
  // stage 0 in registers
  issue(st0, 0);
  stage_scales_first();                         // its loads complete after stage 0's DMA
  issue(st1, min(1, KB - 1));                   // (KB == 1: a harmless second copy of stage 0)
  __builtin_amdgcn_s_waitcnt(kWaitNewest16);
  __builtin_amdgcn_s_barrier();
  read_scales(0, swv, sav);
  read_half(st0, ch00, ch01, fw[0], fa[0]);

  front(st0, 0, window_at(0));
  int kb = 0;
  // Both DMAs of the body are unconditional: a conditional one would be
  // issued as a block ahead of the MFMAs.  With an odd number of stages the
  // last iteration's second DMA asks for stage KB; issue() clamps it to a
  // valid stage, and the buffer it fills (st1) is not read again.
  for (; kb + 2 < KB; kb += 2) {               // stages kb, kb+1 finish; kb+2 begins
    back(st0, st1, kb, true);
    front(st1, kb + 1, window_at(kb + 1));
    back(st1, st0, kb + 1, true);
    front(st0, kb + 2, window_at(kb + 2));
  }
  if (kb + 1 < KB) {                            // two stages left, the first begun
    back(st0, st1, kb, false);
    front(st1, kb + 1, false);
  }
  mma_half(fw[1], fa[1], swv[H1], sav[H1]);     // second half of the last stage
  __builtin_amdgcn_s_waitcnt(kWaitAll);         // no DMA or LDS read outlives the loop

  // Epilogue straight from the accumulators.  Lane holds tile element (t, n)
  // for t = wt*128 + 32j + lane%32 and n = wn*128 + 32i + 8*(r/4) +
  // 4*(lane/32) + r%4 (32x32 accumulator layout): four consecutive n per four
  // registers.  v_permlane32_swap exchanges the register groups r/4 = 2p+1 of
  // lanes 0..31 with the groups 2p of lanes 32..63, after which lane l < 32
  // holds n = 16p .. 16p+7 of its token and lane l + 32 n = 16p+8 .. 16p+15:
  // one 16-byte store each, 32 bytes per token row per instruction.
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int t = t0 + wt * 128 + j * 32 + r32;
    uint16_t* orow = p.out + (static_cast<size_t>(t) * p.G + g) * p.N;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const v16f& v = acc[i][j];
#pragma unroll
      for (int pp = 0; pp < 2; ++pp) {
        const uint32_t x0 = pack_bf16x2(v[8 * pp + 0], v[8 * pp + 1]), x1 = pack_bf16x2(v[8 * pp + 2], v[8 * pp + 3]);
        const uint32_t y0 = pack_bf16x2(v[8 * pp + 4], v[8 * pp + 5]), y1 = pack_bf16x2(v[8 * pp + 6], v[8 * pp + 7]);
        const auto s0 = __builtin_amdgcn_permlane32_swap(x0, y0, false, false);
        const auto s1 = __builtin_amdgcn_permlane32_swap(x1, y1, false, false);
        const int n = n0 + wn * 128 + i * 32 + pp * 16 + q2 * 8;
        if (t < p.T && n < p.N)
          *reinterpret_cast<uint4*>(orow + n) = make_uint4(s0[0], s1[0], s0[1], s1[1]);
      }
    }
  }
}

// ------------------------------------------------- persistent large tiles
//
// The tiles, stages and fragment pipeline of bmm_large_kernel, with each
// workgroup resident for the whole GEMM: workgroup (xcd, slot) takes one tile
// of each round of wg_per_xcd tiles of its XCD's range (which one rotates
// from round to round, see tile_at).  The next tile's stages 0 and 1 and its
// scales are fetched during the current tile's last two stages (scales go to
// the other of two LDS scale buffers), so the stage pipeline runs through
// tile boundaries; a tile's epilogue is folded into the first half-stage of
// the next (front_fold).  Requires K / 128 in {16, 32} (an even number of
// stages, all scales of a tile in one window) and 16-byte aligned scale
// tensors; other shapes use bmm_large_kernel.

// calls f(integral_constant<int, k>) for k = B .. E-1, in order
template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
}
// the order of the 16 MFMAs of a half-stage (W tile I, A tile J): each
// fragment is first used as late as the read order below allows
constexpr int kOrdI[16] = {0, 0, 1, 1, 0, 1, 2, 2, 2, 0, 1, 2, 3, 3, 3, 3};
constexpr int kOrdJ[16] = {0, 1, 0, 1, 2, 2, 0, 1, 2, 3, 3, 3, 0, 1, 2, 3};

template <bool A_FNUZ>
__global__ __launch_bounds__(256, 1) void bmm_persistent_kernel(LargeArgs p) {
  __shared__ __attribute__((aligned(1024))) uint8_t st0[2 * kOpBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t st1[2 * kOpBytes];
  // two scale buffers (current tile, next tile), each [stage][W|A][wave half][row % 32][tile]
  __shared__ __attribute__((aligned(16))) uint8_t lds_sc[2][kScaleWin][2][2][32][4];

  const int xcd = blockIdx.x & 7;
  const int slot = blockIdx.x >> 3;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wn = wave & 1, wt = wave >> 1;
  const int KB = p.K / kBK;                    // 16 or 32
  const uint32_t rowA = static_cast<uint32_t>(p.G) * p.K;

  // Tile r of this workgroup; false past the end of its XCD's range.  Round
  // r of an XCD covers tiles [r * wg_per_xcd, (r + 1) * wg_per_xcd) of its
  // range, and the slots take them rotated by 11 r.  Without the rotation
  // the same compute units would lead every round: the tile at the smallest
  // K offset of those sharing an activation panel (n-tile 0) or a weight
  // tile (first t-tile of the round) misses in L2 on every stage, while the
  // tiles behind it find the rows there; with it the leading role moves
  // between compute units from round to round, so no unit falls behind on
  // all of its tiles (about 2% less time for the launch at T = 8192).  The
  // K loop of tile (tt, nt) starts at stage (tt + nt) mod KB, as in
  // bmm_large_kernel.  (Spacing the tiles that share a panel two stages
  // apart took the same time but fetched 1.5 GB per launch from beyond L2
  // instead of 1.0 GB: the 8 tiles sharing a weight tile then spread over 16
  // stages, longer than its rows stay in the XCD's L2.)  Token tiles are
  // taken from the last to the first: the activation rows the quantiser wrote
  // last are the ones still in the 256 MB last-level cache when the GEMM
  // starts (about 1.7% less GEMM time right after the quantiser).  When
  // every XCD's range is whole groups, it is walked token tile by token tile
  // across its groups (n fastest, then group): the rows the quantiser wrote
  // last are read for all of the XCD's groups first (about 1.4% less).
  const int tpg = p.tiles_n * p.tiles_t;         // tiles per group
  const bool by_token = p.per_xcd % tpg == 0 && p.total_tiles == 8 * p.per_xcd;
  const int gpx = p.per_xcd / tpg;               // groups per XCD when by_token
  auto tile_at = [&](int r, int& g, int& t0, int& n0, int& kb0) {
    const int li = (slot + r * 11) % p.wg_per_xcd + r * p.wg_per_xcd;
    const int work = xcd * p.per_xcd + li;
    if (li >= p.per_xcd || work >= p.total_tiles) return false;
    int nt, tt;
    if (by_token) {
      nt = li % p.tiles_n;
      g = xcd * gpx + (li / p.tiles_n) % gpx;
      tt = p.tiles_t - 1 - li / (p.tiles_n * gpx);
    } else {
      nt = work % p.tiles_n;
      tt = p.tiles_t - 1 - (work / p.tiles_n) % p.tiles_t;
      g = work / tpg;
    }
    t0 = tt * kLT;
    n0 = nt * kLN;
    kb0 = (tt + nt) % KB;
    return true;
  };

  // ---- DMA of one tile's stages (the tile whose stages are being fetched)
  const int dma_row = wave * 8 + (lane >> 3);
  const uint32_t dma_chunk = static_cast<uint32_t>((lane & 7) ^ swz8(dma_row)) * 16;
  // lane's byte offset in its first row group; row groups it = 1..7 add
  // it * 32 rows, and rows past N or T are clamped to the last row (re-read)
  const uint32_t baseW = static_cast<uint32_t>(dma_row) * static_cast<uint32_t>(p.K) + dma_chunk;
  const uint32_t baseA = static_cast<uint32_t>(dma_row) * rowA + dma_chunk;
  uint32_t capW, capA;
  const uint8_t* dW;
  const uint8_t* dA;
  int dkb0;
  auto set_dma_tile = [&](int g, int t0, int n0, int kb0) {
    dW = p.w + (static_cast<size_t>(g) * p.N + n0) * p.K;
    dA = p.a + static_cast<size_t>(t0) * rowA + static_cast<size_t>(g) * p.K;
    dkb0 = kb0;
    // the caps count at most a tile's rows: (T - 1 - t0) * rowA itself can
    // pass 2^32 (T * G * K >= 4 GiB) and would wrap to a cap inside the tile
    capW = static_cast<uint32_t>(min(p.N - 1 - n0, kLN - 1)) * static_cast<uint32_t>(p.K) + dma_chunk;
    capA = static_cast<uint32_t>(min(p.T - 1 - t0, kLT - 1)) * rowA + dma_chunk;
  };
  auto issue = [&](uint8_t* buf, int kb) {   // kb < KB
    int kr = kb + dkb0;
    kr -= kr >= KB ? KB : 0;
    const uint8_t* bW = dW + static_cast<uint32_t>(kr) * kBK;
    const uint8_t* bA = dA + static_cast<uint32_t>(kr) * kBK;
#pragma unroll
    for (int it = 0; it < 8; ++it) {             // weight rows, then activation rows (see dma_k)
      const uint32_t oW = min(baseW + static_cast<uint32_t>(it * 32) * static_cast<uint32_t>(p.K), capW);
      __builtin_amdgcn_global_load_lds(bW + oW, (lds_void_t*)(buf + (it * 32 + wave * 8) * kBK), 16, 0, 0);
    }
#pragma unroll
    for (int it = 0; it < 8; ++it) {
      const uint32_t oA = min(baseA + static_cast<uint32_t>(it * 32) * rowA, capA);
      __builtin_amdgcn_global_load_lds(bA + oA, (lds_void_t*)(buf + kOpBytes + (it * 32 + wave * 8) * kBK), 16, 0, 0);
    }
  };

  // ---- scales: a slot holds one stage's 4-byte words [operand][wave half]
  // [row % 32] (tile bytes 0..3); slot s of a buffer holds stage s (loop
  // stage kb reads slot (kb + kb0) mod KB).  Thread tid builds the words of
  // operand tid/128, wave half (tid/64)%2, row tid%32 for half of the stages,
  // (tid/32)%2: it loads that stage range of the 4 rows (one per tile) and
  // transposes their bytes into words, so that each word is one LDS store.
  constexpr int kScStep = 2 * 2 * 32 * 4;
  constexpr int kScBuf = kScaleWin * kScStep;
  const int sc_op = tid >> 7, sc_half = (tid >> 6) & 1, sc_sh = (tid >> 5) & 1, sc_r = tid & 31;
  uint8_t* const sc_dst = &lds_sc[0][0][sc_op][sc_half][sc_r][0] + sc_sh * (KB / 2) * kScStep;
  uint4 lr[4];                                   // rows of tiles 0..3: stages [sc_sh*KB/2, +KB/2)
  auto load_scales = [&](int g, int t0, int n0) {   // into registers
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = sc_half * 128 + i * 32 + sc_r;
      const uint8_t* src = sc_op == 0
          ? p.sw + (static_cast<size_t>(g) * p.N + n0 + min(row, p.N - 1 - n0)) * KB + sc_sh * (KB / 2)
          : p.sa + (static_cast<size_t>(t0 + min(row, p.T - 1 - t0)) * p.G + g) * KB + sc_sh * (KB / 2);
      if (KB > 16) {
        lr[i] = *reinterpret_cast<const uint4*>(src);
      } else {
        const uint2 v = *reinterpret_cast<const uint2*>(src);
        lr[i] = make_uint4(v.x, v.y, 0, 0);
      }
    }
  };
  auto store_scales = [&](int sb) {              // registers -> LDS buffer sb
    uint8_t* dst = sc_dst + sb * kScBuf;
#pragma unroll
    for (int k = 0; k < 4; ++k) {                // dword k of each row: stages 4k..4k+3 of the range
      if (k >= KB / 8) break;
      uint32_t r[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        r[i] = k == 0 ? lr[i].x : k == 1 ? lr[i].y : k == 2 ? lr[i].z : lr[i].w;
        if (A_FNUZ && sc_op == 1) {              // FNUZ activation scales -> OCP scales, per byte
          uint32_t o = 0;
#pragma unroll
          for (int b = 0; b < 4; ++b) o |= static_cast<uint32_t>(fnuz_scale_to_ocp((r[i] >> (8 * b)) & 0xFF)) << (8 * b);
          r[i] = o;
        }
      }
      // 4 x 4 byte transpose: word j = byte j of rows 0, 1, 2, 3
      const uint32_t t0 = __builtin_amdgcn_perm(r[1], r[0], 0x05010400u);   // r0b0 r1b0 r0b1 r1b1
      const uint32_t t1 = __builtin_amdgcn_perm(r[3], r[2], 0x05010400u);   // r2b0 r3b0 r2b1 r3b1
      const uint32_t t2 = __builtin_amdgcn_perm(r[1], r[0], 0x07030602u);   // r0b2 r1b2 r0b3 r1b3
      const uint32_t t3 = __builtin_amdgcn_perm(r[3], r[2], 0x07030602u);   // r2b2 r3b2 r2b3 r3b3
      const uint32_t w[4] = {__builtin_amdgcn_perm(t1, t0, 0x05040100u), __builtin_amdgcn_perm(t1, t0, 0x07060302u),
                             __builtin_amdgcn_perm(t3, t2, 0x05040100u), __builtin_amdgcn_perm(t3, t2, 0x07060302u)};
#pragma unroll
      for (int j = 0; j < 4; ++j) *reinterpret_cast<uint32_t*>(dst + (4 * k + j) * kScStep) = w[j];
    }
  };
  auto read_scales = [&](int kb, int kb0, int sb, uint32_t& swv, uint32_t& sav) {
    int ks = kb + kb0;
    ks -= ks >= KB ? KB : 0;
    swv = *reinterpret_cast<const uint32_t*>(&lds_sc[sb][ks][0][wn][(lane & 31)][0]);
    sav = *reinterpret_cast<const uint32_t*>(&lds_sc[sb][ks][1][wt][(lane & 31)][0]);
  };

  // ---- fragments and MFMAs (as bmm_large_kernel)
  const int r32 = lane & 31;
  const int q2 = lane >> 5;
  const int rdW = (wn * 128 + r32) * kBK;
  const int rdA = kOpBytes + (wt * 128 + r32) * kBK;
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
    a[1] = read_frag(qa + 32 * kBK, c0, c1);
    w[1] = read_frag(qw + 32 * kBK, c0, c1);
    a[2] = read_frag(qa + 64 * kBK, c0, c1);
    w[2] = read_frag(qw + 64 * kBK, c0, c1);
    a[3] = read_frag(qa + 96 * kBK, c0, c1);
    w[3] = read_frag(qw + 96 * kBK, c0, c1);
  };
  v16f acc[4][4];
  auto pin_acc = [&]() {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) asm volatile("" ::"a"(acc[i][j]));
  };
  constexpr int kWaitAll = wait_vm(0);
  // the prologue leaves stage 1's DMA (kLargeDmaPerStage instructions) in flight
  constexpr int kWaitNewest16 = wait_vm(kLargeDmaPerStage);
  constexpr int kWaitLgkm = kWaitLgkmOnly;
  // front_fold of an interior tile issues kFoldStores stores after the DMA
  // of the next tile's stage 1; they may stay in flight
  constexpr int kWaitOlder32 = wait_vm(kFoldStores);

  // front / back: the two halves of a stage, as in bmm_large_kernel.  back()
  // fetches stage `dma_kb` of the DMA tile into `cur` and reads the scales of
  // stage rs_kb (rotation rs_kb0, buffer rs_sb) with the first half of the
  // next stage from `nxt`.
  uint32_t swv, sav;
  // Step k of a half-stage: MFMA k (in kOrdI/kOrdJ order), fragment read k
  // of the other half (k < 8, in read order), and in back() DMA instruction
  // k.  Each step is fenced with a scheduling barrier, so the compiler keeps
  // this one-to-one interleave; left to itself it bunched the DMA at the end
  // of the half once the DMA addresses no longer went through VGPRs.
  auto mfma_k = [&](auto K, const v8i (&w)[4], const v8i (&a)[4], auto first) {
    constexpr int k = decltype(K)::value;
    mfma_ij<kOrdI[k], kOrdJ[k], decltype(first)::value>(acc, w, a, swv, sav);
  };
  auto read_k = [&](auto K, const uint8_t* buf, int c0, int c1, v8i (&w)[4], v8i (&a)[4]) {
    constexpr int k = decltype(K)::value;   // read order: w0 a0 a1 w1 a2 w2 a3 w3
    constexpr bool isW = k == 0 || k == 3 || k == 5 || k == 7;
    constexpr int idx = k == 0 ? 0 : k == 1 ? 0 : k == 2 ? 1 : k == 3 ? 1 : k == 4 ? 2 : k == 5 ? 2 : 3;
    if constexpr (isW)
      w[idx] = read_frag(buf + rdW + idx * 32 * kBK, c0, c1);
    else
      a[idx] = read_frag(buf + rdA + idx * 32 * kBK, c0, c1);
  };
  // The weight rows go first (steps 0..7), then the activation rows (8..15):
  // alternating the operands instruction by instruction made the GEMM about
  // 6% slower (T = 8192, G = 16, N = 1024, K = 4096: 451 against 423 us in
  // the step, bit-identical).
  auto dma_k = [&](auto K, uint8_t* buf, const uint8_t* bW, const uint8_t* bA) {
    constexpr int k = decltype(K)::value, it = k & 7;
    const int rb = it * 32 + wave * 8;
    if constexpr (k < 8) {
      uint32_t b = baseW;
      // opaque copy: the offsets are formed here rather than hoisted out of
      // the loop as 16 precomputed 64-bit addresses (32 VGPRs)
      asm volatile("" : "+v"(b));
      const uint32_t oW = min(b + static_cast<uint32_t>(it * 32) * static_cast<uint32_t>(p.K), capW);
      __builtin_amdgcn_global_load_lds(bW + oW, (lds_void_t*)(buf + rb * kBK), 16, 0, 0);
    } else {
      uint32_t b = baseA;
      asm volatile("" : "+v"(b));
      const uint32_t oA = min(b + static_cast<uint32_t>(it * 32) * rowA, capA);
      __builtin_amdgcn_global_load_lds(bA + oA, (lds_void_t*)(buf + kOpBytes + rb * kBK), 16, 0, 0);
    }
  };
  // front(cur, first, with_scales): `first` starts the tile's sums;
  // `with_scales` also writes the next tile's staged scales (load_scales) to
  // LDS buffer `scale_sb` before the barrier, so they are visible after it.
  auto front = [&](const uint8_t* cur, auto first, auto with_scales, int scale_sb) {
    __builtin_amdgcn_sched_barrier(0);
    static_for<0, 16>([&](auto K) {
      mfma_k(K, fw[0], fa[0], first);
      if constexpr (decltype(K)::value < 8) read_k(K, cur, ch10, ch11, fw[1], fa[1]);
      __builtin_amdgcn_sched_barrier(0);
    });
    pin_acc();
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(kWaitAll);
    if constexpr (decltype(with_scales)::value) {
      store_scales(scale_sb);
      __builtin_amdgcn_s_waitcnt(kWaitLgkm);
    }
    __builtin_amdgcn_s_barrier();
  };
  auto back = [&](uint8_t* cur, const uint8_t* nxt, int dma_kb, int rs_kb, int rs_kb0, int rs_sb) {
    // the scale reads go before the DMA: with a run-time buffer index the
    // compiler cannot tell them from the DMA's target and would make them
    // wait for it
    uint32_t swv1, sav1;
    read_scales(rs_kb, rs_kb0, rs_sb, swv1, sav1);
    int kr = dma_kb + dkb0;
    kr -= kr >= KB ? KB : 0;
    const uint8_t* bW = dW + static_cast<uint32_t>(kr) * kBK;
    const uint8_t* bA = dA + static_cast<uint32_t>(kr) * kBK;
    __builtin_amdgcn_sched_barrier(0);
    static_for<0, 16>([&](auto K) {
      mfma_k(K, fw[1], fa[1], std::false_type{});
      dma_k(K, cur, bW, bA);
      if constexpr (decltype(K)::value < 8) read_k(K, nxt, ch00, ch01, fw[0], fa[0]);
      __builtin_amdgcn_sched_barrier(0);
    });
    pin_acc();
    __builtin_amdgcn_sched_barrier(0);
    swv = swv1;
    sav = sav1;
  };

  // ---- first tile: prologue
  int cg, ct0, cn0, ckb0;
  if (!tile_at(0, cg, ct0, cn0, ckb0)) return;
  int csb = 0;
  set_dma_tile(cg, ct0, cn0, ckb0);
  issue(st0, 0);
  load_scales(cg, ct0, cn0);
  issue(st1, 1);
  store_scales(0);                               // waits for the scale loads (after stage 0's DMA)
  __builtin_amdgcn_s_waitcnt(kWaitNewest16);
  __builtin_amdgcn_s_barrier();
  read_scales(0, ckb0, 0, swv, sav);
  read_half(st0, ch00, ch01, fw[0], fa[0]);

  const std::true_type yes{};
  const std::false_type no{};
  // ---- epilogue, folded into the next tile's first half-stage
  //
  // In the accumulator layout a lane holds one token and two lanes share a
  // row, so a direct store writes 32 bytes per row.  Instead the wave's
  // 128 x 128 sub-tile leaves in 8 chunks of 32 rows (accumulator row tile
  // j) x 64 columns (tiles 2 ip, 2 ip + 1): a chunk is converted to BF16,
  // written to LDS (the finishing tile's scale buffer, free since the
  // transition barrier; 4 KiB per wave, 16-byte chunks XOR-swizzled by row),
  // read back as 8 rows x 128 bytes per instruction and stored.  As soon as
  // a chunk is in LDS, the two MFMAs that start the next tile's sums in its
  // blocks are issued, so they run while the chunk makes its LDS round trip
  // and the next chunk is converted.  The staging goes through inline asm
  // with its own lgkmcnt waits: written as plain LDS accesses, the compiler
  // could not tell the run-time scale buffer from the LDS-DMA targets and
  // waited for all outstanding DMA and stores before each access.  The
  // restarting MFMAs are inline asm too, tied to the block's registers: as
  // builtins with a zero accumulator the register allocator gave the new
  // sums fresh registers and spilled.
  uint8_t* const stg_base = &lds_sc[0][0][0][0][0][0] + wave * 4096;
  const int er = lane >> 3, ec = lane & 7;   // staging read side: row in group of 8, 16-byte chunk
  typedef unsigned int v4u_t __attribute__((ext_vector_type(4)));
  // front_fold(cur, ft0, fn0, fg, fsb): the first half of the next tile's
  // stage 0 (fragments fw[0] / fa[0], buffer `cur`) with the epilogue of the
  // finishing tile (ft0, fn0, fg; scale buffer fsb) folded in
  auto front_fold = [&](const uint8_t* cur, int ft0, int fn0, int fg, int fsb) {
    uint8_t* const stg = stg_base + fsb * (kScaleWin * kScStep);
    // LDS byte address for ds_read / ds_write: the low 32 bits of the generic
    // address (the shared aperture is 4 GiB aligned)
    const uint32_t wa = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(stg));
    // this lane's store address for rows ft0 + wt*128 + er (+ j*32 + sg*8) and
    // columns fn0 + wn*128 + ec*8 (+ ip*64): one 64-bit product per tile, the
    // per-store offsets are compile-time multiples of a uniform row stride
    const int trow = ft0 + wt * 128 + er, ncol = fn0 + wn * 128 + ec * 8;
    uint16_t* const obase = p.out + (static_cast<size_t>(trow) * p.G + fg) * p.N + ncol;
    const size_t rs8 = static_cast<size_t>(8) * p.G * p.N;   // 8 rows
    __builtin_amdgcn_sched_barrier(0);
    // the fragments of this half have landed (stated here, the compiler
    // puts no wait of its own between a chunk's LDS writes and its MFMAs)
    __builtin_amdgcn_s_waitcnt(kWaitLgkm);
    static_for<0, 8>([&](auto C) {
      constexpr int c8 = decltype(C)::value, j = c8 >> 1, ip = c8 & 1;
#pragma unroll
      for (int ii = 0; ii < 2; ++ii) {
        const v16f& v = acc[2 * ip + ii][j];
#pragma unroll
        for (int pp = 0; pp < 2; ++pp) {
          const uint32_t x0 = pack_bf16x2(v[8 * pp + 0], v[8 * pp + 1]), x1 = pack_bf16x2(v[8 * pp + 2], v[8 * pp + 3]);
          const uint32_t y0 = pack_bf16x2(v[8 * pp + 4], v[8 * pp + 5]), y1 = pack_bf16x2(v[8 * pp + 6], v[8 * pp + 7]);
          const auto s0 = __builtin_amdgcn_permlane32_swap(x0, y0, false, false);
          const auto s1 = __builtin_amdgcn_permlane32_swap(x1, y1, false, false);
          const int c = ii * 4 + pp * 2 + q2;
          const uint32_t a = wa + r32 * 128 + ((c ^ (r32 & 7)) << 4);
          const v4u_t dv = {s0[0], s1[0], s0[1], s1[1]};
          asm volatile("ds_write_b128 %0, %1" ::"v"(a), "v"(dv) : "memory");
        }
      }
      // the next tile's first MFMAs on this chunk's two blocks (accumulator
      // input 0, result in the block's own registers; the blocks were read
      // out above)
      asm volatile("v_mfma_scale_f32_32x32x64_f8f6f4 %0, %1, %2, 0, %3, %4 op_sel:[%5,%6,0] op_sel_hi:[%7,%8,0]"
                   : "+a"(acc[2 * ip][j])
                   : "v"(fw[0][2 * ip]), "v"(fa[0][j]), "v"(swv), "v"(sav), "n"((2 * ip) & 1), "n"(j & 1),
                     "n"((2 * ip) >> 1), "n"(j >> 1));
      asm volatile("v_mfma_scale_f32_32x32x64_f8f6f4 %0, %1, %2, 0, %3, %4 op_sel:[%5,%6,0] op_sel_hi:[%7,%8,0]"
                   : "+a"(acc[2 * ip + 1][j])
                   : "v"(fw[0][2 * ip + 1]), "v"(fa[0][j]), "v"(swv), "v"(sav), "n"((2 * ip + 1) & 1), "n"(j & 1),
                     "n"((2 * ip + 1) >> 1), "n"(j >> 1));
      v4u_t d0, d1, d2, d3;
      asm volatile(
          "s_waitcnt lgkmcnt(0)\n"
          "ds_read_b128 %0, %4\n"
          "ds_read_b128 %1, %4 offset:1024\n"
          "ds_read_b128 %2, %4 offset:2048\n"
          "ds_read_b128 %3, %4 offset:3072\n"
          "s_waitcnt lgkmcnt(0)"
          : "=&v"(d0), "=&v"(d1), "=&v"(d2), "=&v"(d3)
          : "v"(wa + er * 128 + ((ec ^ er) << 4))
          : "memory");
      const v4u_t d[4] = {d0, d1, d2, d3};
#pragma unroll
      for (int sg = 0; sg < 4; ++sg) {
        if (trow + j * 32 + sg * 8 < p.T && ncol + ip * 64 < p.N)
          *reinterpret_cast<uint4*>(obase + (j * 4 + sg) * rs8 + ip * 64) =
              make_uint4(d[sg][0], d[sg][1], d[sg][2], d[sg][3]);
      }
      __builtin_amdgcn_sched_barrier(0);
    });
    static_for<0, 8>([&](auto K) { read_k(K, cur, ch10, ch11, fw[1], fa[1]); });
    pin_acc();
    __builtin_amdgcn_sched_barrier(0);
    // an interior tile issued exactly 32 stores per wave after the DMA of
    // the next tile's stage 1; vector memory completes in issue order, so the
    // wait for that DMA can leave the stores in flight
    if (ft0 + kLT <= p.T && fn0 + kLN <= p.N)
      __builtin_amdgcn_s_waitcnt(kWaitOlder32);
    else
      __builtin_amdgcn_s_waitcnt(kWaitAll);
    __builtin_amdgcn_s_barrier();
  };

  front(st0, yes, no, 0);                        // first tile, stage 0 (first half): starts the sums
  for (int r = 0;; ++r) {
    int kb = 0;
    for (; kb + 2 < KB; kb += 2) {               // stages kb, kb+1 finish; kb+2 begins
      back(st0, st1, kb + 2, kb + 1, ckb0, csb);
      front(st1, no, no, 0);
      back(st1, st0, kb + 3, kb + 2, ckb0, csb);
      front(st0, no, no, 0);
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
    load_scales(ng, nt0, nn0);
    back(st0, st1, 0, KB - 1, ckb0, csb);        // next tile's stage 0 -> st0
    front(st1, no, yes, csb ^ 1);                // waits for it and for the scale loads; stages the scales
    back(st1, st0, 1, 0, nkb0, csb ^ 1);         // next tile's stage 1 -> st1; its stage 0 half 0

    front_fold(st0, ct0, cn0, cg, csb);          // next tile's stage 0 (first half) + this tile's epilogue
    if (!more) break;
    cg = ng;
    ct0 = nt0;
    cn0 = nn0;
    ckb0 = nkb0;
    csb ^= 1;
  }
  __builtin_amdgcn_s_waitcnt(kWaitAll);          // no DMA outlives the workgroup
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

constexpr int kSmallWaves = 4;
constexpr int kSmallThreads = 64 * kSmallWaves;

// One workgroup: all T (<= 64) rows x 16*NT columns n of one group g, kSmallWaves
// waves.  Wave w takes K-steps w, w+kSmallWaves, ...; partial sums meet in
// LDS.  The workgroup's scale rows are staged in LDS once (W rows n0.. are one
// contiguous block; A rows one per token), so the loop reads only operand
// bytes from memory; the operands of a wave's next K-step are loaded while the
// current one's MFMAs run.
template <int NT, int SB, bool A_FNUZ>
__global__ __launch_bounds__(kSmallThreads) void bmm_small_kernel(SmallArgs p) {
  __shared__ float red[4][NT * 4][4][64];   // [wave % 4][tile][reg][lane]
  extern __shared__ uint8_t scl[];          // [16*NT W rows | 64 A rows][SPK]
  const int g = blockIdx.x / p.n_groups;
  const int n0 = (blockIdx.x % p.n_groups) * (16 * NT);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  // wave-uniform (a scalar): the K loop below is then a uniform loop
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int KB = p.K / kBK;
  const int SPK = p.K / SB;                   // scale bytes per row
  const int kq = lane >> 4;                   // lane group: K bytes 16kq.. and 64+16kq.., scale block kq
  const size_t rowA = static_cast<size_t>(p.G) * p.K;
  constexpr int kRowsW = 16 * NT;


  const uint8_t* pw[NT];
  const uint8_t* lsw[NT];
#pragma unroll
  for (int i = 0; i < NT; ++i) {
    const int n = min(n0 + i * 16 + (lane & 15), p.N - 1);
    pw[i] = p.w + (static_cast<size_t>(g) * p.N + n) * p.K + kq * 16;
    lsw[i] = scl + (i * 16 + (lane & 15)) * SPK + (SB == 32 ? kq : 0);
  }
  const uint8_t* pa[4];
  const uint8_t* lsa[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int t = min(j * 16 + (lane & 15), p.T - 1);
    pa[j] = p.a + static_cast<size_t>(t) * rowA + static_cast<size_t>(g) * p.K + kq * 16;
    lsa[j] = scl + (kRowsW + j * 16 + (lane & 15)) * SPK + (SB == 32 ? kq : 0);
  }
  constexpr int kScalesPerStep = kBK / SB;

  v4f acc[NT][4];
#pragma unroll
  for (int i = 0; i < NT; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

  // Two K-steps of operands in registers: the loads of this wave's next step
  // are in flight while the MFMAs of the current one run.  Steps past the end
  // load a clamped, valid step whose data is never used.
  v8i fw[2][NT], fa[2][4];
  auto load = [&](int kt, int b) {
    kt = min(kt, KB - 1);
    const size_t ko = static_cast<size_t>(kt) * kBK;
#pragma unroll
    for (int i = 0; i < NT; ++i)
      fw[b][i] = make_v8i(*reinterpret_cast<const uint4*>(pw[i] + ko), *reinterpret_cast<const uint4*>(pw[i] + ko + 64));
#pragma unroll
    for (int j = 0; j < 4; ++j)
      fa[b][j] = make_v8i(*reinterpret_cast<const uint4*>(pa[j] + ko), *reinterpret_cast<const uint4*>(pa[j] + ko + 64));
  };
  auto compute = [&](int kt, int b) {
    int s_w[NT], s_a[4];
#pragma unroll
    for (int i = 0; i < NT; ++i) s_w[i] = lsw[i][kt * kScalesPerStep];
#pragma unroll
    for (int j = 0; j < 4; ++j) s_a[j] = lsa[j][kt * kScalesPerStep];
#pragma unroll
    for (int i = 0; i < NT; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = mfma_scaled(fw[b][i], fa[b][j], acc[i][j], s_w[i], s_a[j]);
  };
  constexpr int W = kSmallWaves;
  load(wave, 0);                              // the first operands fly while the scales are staged
  load(wave + W, 1);

  // ---- stage the scales: rows past N or T repeat the last valid row
  {
    const int nW = min(kRowsW, p.N - n0);
    const uint8_t* srcW = p.sw + (static_cast<size_t>(g) * p.N + n0) * SPK;
    if ((SPK & 3) == 0 && ((reinterpret_cast<uintptr_t>(p.sw) | reinterpret_cast<uintptr_t>(p.sa)) & 3) == 0) {
      const int dw = SPK >> 2;                // dwords per row
      const int nw = kRowsW * dw, na = 64 * dw;
      // all loads first (one round trip), then the LDS writes; up to kPer
      // dwords per thread per operand that way, a loop for anything beyond
      constexpr int kPer = 8;
      uint32_t vw[kPer], va[kPer];
#pragma unroll
      for (int u = 0; u < kPer; ++u) {
        const int e = tid + u * kSmallThreads;
        if (e < nw) {
          const int r = e / dw, c = e - r * dw;
          vw[u] = *reinterpret_cast<const uint32_t*>(srcW + static_cast<size_t>(min(r, nW - 1)) * SPK + 4 * c);
        }
        if (e < na) {
          const int r = e / dw, c = e - r * dw;
          va[u] = *reinterpret_cast<const uint32_t*>(p.sa + (static_cast<size_t>(min(r, p.T - 1)) * p.G + g) * SPK + 4 * c);
        }
      }
#pragma unroll
      for (int u = 0; u < kPer; ++u) {
        const int e = tid + u * kSmallThreads;
        if (e < nw) {
          const int r = e / dw, c = e - r * dw;
          *reinterpret_cast<uint32_t*>(scl + r * SPK + 4 * c) = vw[u];
        }
        if (e < na) {
          const int r = e / dw, c = e - r * dw;
          uint32_t v = va[u];
          if (A_FNUZ) {
            uint32_t o = 0;
#pragma unroll
            for (int b = 0; b < 4; ++b) o |= static_cast<uint32_t>(fnuz_scale_to_ocp((v >> (8 * b)) & 0xFF)) << (8 * b);
            v = o;
          }
          *reinterpret_cast<uint32_t*>(scl + (kRowsW + r) * SPK + 4 * c) = v;
        }
      }
      for (int e = tid + kPer * kSmallThreads; e < nw; e += kSmallThreads) {
        const int r = e / dw, c = e - r * dw;
        *reinterpret_cast<uint32_t*>(scl + r * SPK + 4 * c) =
            *reinterpret_cast<const uint32_t*>(srcW + static_cast<size_t>(min(r, nW - 1)) * SPK + 4 * c);
      }
      for (int e = tid + kPer * kSmallThreads; e < na; e += kSmallThreads) {
        const int r = e / dw, c = e - r * dw;
        uint32_t v = *reinterpret_cast<const uint32_t*>(p.sa + (static_cast<size_t>(min(r, p.T - 1)) * p.G + g) * SPK + 4 * c);
        if (A_FNUZ) {
          uint32_t o = 0;
#pragma unroll
          for (int b = 0; b < 4; ++b) o |= static_cast<uint32_t>(fnuz_scale_to_ocp((v >> (8 * b)) & 0xFF)) << (8 * b);
          v = o;
        }
        *reinterpret_cast<uint32_t*>(scl + (kRowsW + r) * SPK + 4 * c) = v;
      }
    } else {
      for (int e = tid; e < kRowsW * SPK; e += kSmallThreads) {
        const int r = e / SPK, c = e - r * SPK;
        scl[r * SPK + c] = srcW[static_cast<size_t>(min(r, nW - 1)) * SPK + c];
      }
      for (int e = tid; e < 64 * SPK; e += kSmallThreads) {
        const int r = e / SPK, c = e - r * SPK;
        const int t = min(r, p.T - 1);
        const int v = p.sa[(static_cast<size_t>(t) * p.G + g) * SPK + c];
        scl[(kRowsW + r) * SPK + c] = static_cast<uint8_t>(A_FNUZ ? fnuz_scale_to_ocp(v) : v);
      }
    }
  }
  __syncthreads();
  int kt = wave;
  for (; kt + W < KB; kt += 2 * W) {          // branch-free body: both steps exist
    compute(kt, 0);
    load(kt + 2 * W, 0);
    compute(kt + W, 1);
    load(kt + 3 * W, 1);
  }
  if (kt < KB) compute(kt, 0);                // a last single step (buffer 0 holds it)
  __builtin_amdgcn_s_waitcnt(wait_vm(0));     // the clamped prefetches end here too

  // reduce over the waves in two rounds through 4 slots: waves 4..7 hand
  // their sums to waves 0..3, which then meet in the slots
  static_assert(kSmallWaves == 4 || kSmallWaves == 8, "one or two reduction rounds of four");
  if (kSmallWaves == 8 && wave >= 4) {
#pragma unroll
    for (int i = 0; i < NT; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) red[wave - 4][i * 4 + j][r][lane] = acc[i][j][r];
  }
  if (kSmallWaves == 8) {
    __syncthreads();
    if (wave < 4) {
#pragma unroll
      for (int i = 0; i < NT; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[i][j][r] += red[wave][i * 4 + j][r][lane];
    }
    __syncthreads();
  }
  if (wave < 4) {
#pragma unroll
    for (int i = 0; i < NT; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) red[wave][i * 4 + j][r][lane] = acc[i][j][r];
  }
  __syncthreads();
  // wave w < 4 finalises tiles w, w+4, ...
  for (int tile = wave; tile < NT * 4 && wave < 4; tile += 4) {
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

// ------------------------------------------ decode batch: T <= 64, K % 1024 == 0
//
// One workgroup per (g, 64 n) with all T rows, as bmm_small_kernel, but the
// operands go global -> LDS by LDS-DMA through a ring of kDecR stages (one
// 128-byte K-step of the 64 W rows and the 64 A rows each, 16 KiB), so that
// kDecR - 1 K-steps (48 KiB) per compute unit are in flight and every DMA
// instruction reads 8 whole 128-byte lines.  (8 stages, 112 KiB in flight,
// were no faster: 17.4 against 17.2 us per call; the weight's access pattern,
// all 64 rows advancing 128 bytes at a time, sets the pace.)  The four waves split n (wave w
// owns rows 16w..16w+15 of the workgroup's W), so every wave consumes every
// stage and no partial sums are reduced; one barrier per stage recycles the
// ring.  Each slot is its own __shared__ array and the stage loop is unrolled
// over the ring, so every access names its slot statically (the compiler can
// then see that the DMA into one slot does not alias the reads of another).
constexpr int kDecR = 4;
constexpr int kDecRows = 64;
// operand modes of the decode kernel: FP8 A in OCP or FNUZ bytes (E8M0
// scales), or BF16 A and W (no scales; a stage is then 64 elements and the
// K and row strides in SmallArgs are in bytes)
constexpr int kDecOcp = 0, kDecFnuz = 1, kDecBf16 = 2;

typedef __bf16 v8bf_t __attribute__((ext_vector_type(8)));
typedef int v4i_t __attribute__((ext_vector_type(4)));
template <int H>
__device__ __forceinline__ v8bf_t bf16_half(const v8i& v) {
  const v4i_t h = __builtin_shufflevector(v, v, 4 * H, 4 * H + 1, 4 * H + 2, 4 * H + 3);
  return __builtin_bit_cast(v8bf_t, h);
}
constexpr int kDecStage = 2 * kDecRows * kBK;      // 16 KiB: W rows, then A rows
constexpr int kDecScaleMax = 16 * 1024;            // staged scale rows: 128 rows x K/128 bytes

template <int KB, int MODE>
__global__ __launch_bounds__(256, 1) void bmm_decode_kernel(SmallArgs p) {
  __shared__ __attribute__((aligned(1024))) uint8_t s0[kDecStage];
  __shared__ __attribute__((aligned(1024))) uint8_t s1[kDecStage];
  __shared__ __attribute__((aligned(1024))) uint8_t s2[kDecStage];
  __shared__ __attribute__((aligned(1024))) uint8_t s3[kDecStage];
  __shared__ __attribute__((aligned(16))) uint8_t scl[kDecScaleMax];   // [64 W rows | 64 A rows][KB]
  uint8_t* const ring[kDecR] = {s0, s1, s2, s3};
  static_assert(kDecR == 4, "one __shared__ array per ring slot");

  // XCD-aware: workgroup b runs on XCD b % 8; when the work divides evenly,
  // each XCD takes a contiguous range of (g, n-block) work items, so the
  // workgroups sharing one group's activation rows share one XCD's L2
  // (decode batch: 18.1 -> 17.4 us per call in a 40-call graph)
  const int total = p.G * p.n_groups;
  const int work = total % 8 == 0 ? static_cast<int>(blockIdx.x % 8) * (total / 8) + static_cast<int>(blockIdx.x / 8)
                                  : static_cast<int>(blockIdx.x);
  const int g = work / p.n_groups;
  const int n0 = (work % p.n_groups) * kDecRows;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const size_t rowA = static_cast<size_t>(p.G) * p.K;
  static_assert(KB % kDecR == 0 && 2 * kDecRows * KB <= kDecScaleMax, "K-steps");

  // ---- scale rows -> LDS by LDS-DMA as well (an LDS store after the operand
  // DMA would have to wait for all of it): 128 rows (64 W, 64 A) x KB bytes,
  // 4 bytes per lane, 256 bytes per instruction, KB/8 instructions per wave;
  // issued before the operand stages, so the first stage's wait covers them
  constexpr int kScInstr = MODE == kDecBf16 ? 0 : KB / 8;
#pragma unroll
  for (int it = 0; it < kScInstr; ++it) {
    const int ii = wave * kScInstr + it;
    const int byte = ii * 256 + 4 * lane;
    const int r = byte / KB, off = byte - r * KB;
    const uint8_t* src = r < kDecRows
        ? p.sw + (static_cast<size_t>(g) * p.N + min(n0 + r, p.N - 1)) * KB + off
        : p.sa + (static_cast<size_t>(min(r - kDecRows, p.T - 1)) * p.G + g) * KB + off;
    __builtin_amdgcn_global_load_lds(src, (lds_void_t*)(scl + ii * 256), 4, 0, 0);
  }

  // ---- DMA: wave w fills W rows 16w..16w+15 and A rows 16w..16w+15 of a stage,
  // 8 rows per instruction (lane i writes LDS byte 16i of the instruction's
  // 1 KiB); the global side reads the chunk that the swizzle puts at lane i
  const uint8_t* pW[2];
  const uint8_t* pA[2];
#pragma unroll
  for (int it = 0; it < 2; ++it) {
    const int r = 16 * wave + 8 * it + (lane >> 3);
    const uint32_t chunk = static_cast<uint32_t>((lane & 7) ^ swz8(r)) * 16;
    pW[it] = p.w + (static_cast<size_t>(g) * p.N + min(n0 + r, p.N - 1)) * p.K + chunk;
    pA[it] = p.a + static_cast<size_t>(min(r, p.T - 1)) * rowA + static_cast<size_t>(g) * p.K + chunk;
  }
  auto issue = [&](uint8_t* slot, int kt) {
    const size_t ko = static_cast<size_t>(min(kt, KB - 1)) * kBK;   // past the end: a harmless refetch
#pragma unroll
    for (int it = 0; it < 2; ++it) {
      const int rb = 16 * wave + 8 * it;
      __builtin_amdgcn_global_load_lds(pW[it] + ko, (lds_void_t*)(slot + rb * kBK), 16, 0, 0);
      __builtin_amdgcn_global_load_lds(pA[it] + ko, (lds_void_t*)(slot + (kDecRows + rb) * kBK), 16, 0, 0);
    }
  };
#pragma unroll
  for (int u = 0; u < kDecR - 1; ++u) issue(ring[u], u);

  // ---- fragments: lane l holds row l%16 of a 16-row tile; K bytes 16q.. and
  // 64+16q.. (q = l/16) sit at physical chunks q ^ s and (q + 4) ^ s
  const int sw16 = swz8(lane & 15);
  const int q = lane >> 4;
  const int c0 = (q ^ sw16) * 16, c1 = ((q + 4) ^ sw16) * 16;
  const int rdW = (16 * wave + (lane & 15)) * kBK;
  const uint8_t* sclW = scl + (16 * wave + (lane & 15)) * KB;
  const uint8_t* sclA = scl + (kDecRows + (lane & 15)) * KB;
  v4f acc[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) acc[j] = v4f{0.f, 0.f, 0.f, 0.f};
  // a stage is kDecDmaPerStage instructions per wave (issue(): 2 row groups x
  // 2 operands); at the wait for stage kt, stages kt+1 .. kt+kDecR-2 may be
  // in flight (the scale DMA is older than all of them)
  constexpr int kDecDmaPerStage = 2 * 2;
  constexpr int kWaitStage = wait_vm(kDecDmaPerStage * (kDecR - 2));
  static_assert(kWaitStage == 0x0078, "vmcnt(8)");

#pragma unroll 1
  for (int kt0 = 0; kt0 < KB; kt0 += kDecR) {
#pragma unroll
    for (int u = 0; u < kDecR; ++u) {
      const int kt = kt0 + u;
      __builtin_amdgcn_s_waitcnt(kWaitStage);       // this wave's part of stage kt is in LDS
      __builtin_amdgcn_s_barrier();                 // everyone's part; everyone is done with stage kt-1
      issue(ring[(u + kDecR - 1) % kDecR], kt + kDecR - 1);
      const uint8_t* st = ring[u];
      // all of the stage's reads, then its MFMAs
      const v8i fw = make_v8i(*reinterpret_cast<const uint4*>(st + rdW + c0),
                              *reinterpret_cast<const uint4*>(st + rdW + c1));
      v8i fa[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint8_t* ra = st + (kDecRows + 16 * j + (lane & 15)) * kBK;
        fa[j] = make_v8i(*reinterpret_cast<const uint4*>(ra + c0), *reinterpret_cast<const uint4*>(ra + c1));
      }
      if constexpr (MODE == kDecBf16) {
        // a lane's two 16-byte chunks are its K-pieces of two 16x16x32 BF16 MFMAs
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bf16_half<0>(fw), bf16_half<0>(fa[j]), acc[j], 0, 0, 0);
          acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bf16_half<1>(fw), bf16_half<1>(fa[j]), acc[j], 0, 0, 0);
        }
      } else {
        int sa_[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          sa_[j] = sclA[16 * j * KB + kt];
          if (MODE == kDecFnuz) sa_[j] = fnuz_scale_to_ocp(sa_[j]);   // FNUZ activation scale -> OCP scale
        }
        const int sw_ = sclW[kt];
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[j] = mfma_scaled(fw, fa[j], acc[j], sw_, sa_[j]);
      }
    }
  }
  __builtin_amdgcn_s_waitcnt(wait_vm(0));           // no DMA outlives the workgroup

  // ---- C layout: lane l holds column l%16 (a token) and rows 4(l/16)..+3 (n)
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int t = 16 * j + (lane & 15);
    const int n = n0 + 16 * wave + 4 * q;
    if (t < p.T && n < p.N)
      *reinterpret_cast<uint2*>(p.out + (static_cast<size_t>(t) * p.G + g) * p.N + n) = pack4_bf16(acc[j]);
  }
}

// --------------------------- MXFP8 linear, block-32 scales, M <= 64 (LDS-DMA)
//
// The decode kernel's ring for the linear's shapes (N of a few thousand, K a
// multiple of 128 but not of 1024): one workgroup per 16 columns n, so that
// N = 4096 still gives 256 workgroups; a stage is one 128-byte K-step of the
// 16 W rows and the 64 x rows (10 KiB), kLinR of them in the ring; wave w
// owns token tile w (x rows 16w..16w+15), one MFMA per stage.  A stage is
// moved by 12 DMA instructions, 3 per wave: the ten that carry its rows and
// two that re-read x rows 0..15 into 2 KiB of the slot nobody reads.  A DMA
// issued on some waves only would leave the compiler unsure which LDS it
// writes, and it would then drain all DMA before the scale reads.
constexpr int kLinR = 8;                    // (the compiler tracks 9 LDS-DMA targets: 8 slots + scales)
constexpr int kLinRowsW = 16;
constexpr int kLinRows = kLinRowsW + 64;
constexpr int kLinStage = (kLinRows + 16) * kBK;   // 10 KiB of rows + 2 KiB written by the padding DMA
constexpr int kLinScaleMax = kLinRows * 256;       // scale rows of K <= 8192

__global__ __launch_bounds__(256, 1) void gemm_mx32_dma_kernel(SmallArgs p) {
  __shared__ __attribute__((aligned(1024))) uint8_t s0[kLinStage];
  __shared__ __attribute__((aligned(1024))) uint8_t s1[kLinStage];
  __shared__ __attribute__((aligned(1024))) uint8_t s2[kLinStage];
  __shared__ __attribute__((aligned(1024))) uint8_t s3[kLinStage];
  __shared__ __attribute__((aligned(1024))) uint8_t s4[kLinStage];
  __shared__ __attribute__((aligned(1024))) uint8_t s5[kLinStage];
  __shared__ __attribute__((aligned(1024))) uint8_t s6[kLinStage];
  __shared__ __attribute__((aligned(1024))) uint8_t s7[kLinStage];
  __shared__ __attribute__((aligned(16))) uint8_t scl[kLinScaleMax];   // [16 W rows | 64 x rows][K/32]
  uint8_t* const ring[kLinR] = {s0, s1, s2, s3, s4, s5, s6, s7};

  const int n0 = blockIdx.x * kLinRowsW;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int KB = p.K / kBK;
  const int SPK = 4 * KB;                             // scale bytes per row (block 32)

  // ---- scale rows by LDS-DMA, 4 bytes per lane, before the operand stages
  const int sc_bytes = kLinRows * SPK;
  for (int ii = wave; ii * 256 < sc_bytes; ii += 4) {
    const int byte = ii * 256 + 4 * lane;
    if (byte < sc_bytes) {
      const int r = byte / SPK, off = byte - r * SPK;
      const uint8_t* src = r < kLinRowsW ? p.sw + static_cast<size_t>(min(n0 + r, p.N - 1)) * SPK + off
                                         : p.sa + static_cast<size_t>(min(r - kLinRowsW, p.T - 1)) * SPK + off;
      __builtin_amdgcn_global_load_lds(src, (lds_void_t*)(scl + ii * 256), 4, 0, 0);
    }
  }

  // ---- operand DMA: instruction ii (0..11) of a stage moves its rows
  // 8ii..8ii+7 (W rows 0..15, x rows 0..63, then the padding rows 80..95,
  // read from x rows 0..15); wave w issues ii = w, w + 4, w + 8
  const uint8_t* src_row[3];
#pragma unroll
  for (int it = 0; it < 3; ++it) {
    const int ii = wave + 4 * it;
    const int r = 8 * ii + (lane >> 3);               // stage row
    const int xr = r < kLinRows ? r - kLinRowsW : r - kLinRows;   // x row (padding: rows 0..15 again)
    const uint32_t chunk = static_cast<uint32_t>((lane & 7) ^ swz8(r)) * 16;
    src_row[it] = r < kLinRowsW ? p.w + static_cast<size_t>(min(n0 + r, p.N - 1)) * p.K + chunk
                                : p.a + static_cast<size_t>(min(xr, p.T - 1)) * p.K + chunk;
  }
  auto issue = [&](uint8_t* slot, int kt) {
    const size_t ko = static_cast<size_t>(min(kt, KB - 1)) * kBK;   // past the end: a harmless refetch
#pragma unroll
    for (int it = 0; it < 3; ++it)
      __builtin_amdgcn_global_load_lds(src_row[it] + ko, (lds_void_t*)(slot + 8 * (wave + 4 * it) * kBK), 16, 0, 0);
  };
#pragma unroll
  for (int u = 0; u < kLinR - 1; ++u) issue(ring[u], u);

  // ---- fragments (as the decode kernel) and block-32 scales: lane group q's
  // byte is block 4kt + q of its row
  const int sw16 = swz8(lane & 15);
  const int q = lane >> 4;
  const int c0 = (q ^ sw16) * 16, c1 = ((q + 4) ^ sw16) * 16;
  const int rdW = (lane & 15) * kBK;
  const int rdA = (kLinRowsW + 16 * wave + (lane & 15)) * kBK;
  const uint8_t* sclW = scl + (lane & 15) * SPK + q;
  const uint8_t* sclA = scl + (kLinRowsW + 16 * wave + (lane & 15)) * SPK + q;
  v4f acc = v4f{0.f, 0.f, 0.f, 0.f};
  // a stage is kLinDmaPerWave instructions per wave (issue(): ii = wave,
  // wave + 4, wave + 8 of the (kLinRows + 16) / 8 = 12 row groups); at the
  // wait for stage kt, stages kt+1 .. kt+kLinR-2 may be in flight (the scale
  // DMA is older than all of them)
  constexpr int kLinDmaPerWave = 3;
  static_assert(4 * kLinDmaPerWave * 8 == kLinRows + 16, "row groups per stage");
  constexpr int kWaitStage = wait_vm(kLinDmaPerWave * (kLinR - 2));
  static_assert(kWaitStage == 0x4072, "vmcnt(18)");

  // (the compiler drains the DMA once per pass of this loop, at its head:
  // it cannot tell which slot the DMA pending there writes)
#pragma unroll 1
  for (int kt0 = 0; kt0 < KB; kt0 += kLinR) {
#pragma unroll
    for (int u = 0; u < kLinR; ++u) {
      const int kt = kt0 + u;
      if (kt >= KB) break;                          // uniform: every wave leaves at the same stage
      __builtin_amdgcn_s_waitcnt(kWaitStage);
      __builtin_amdgcn_s_barrier();
      issue(ring[(u + kLinR - 1) % kLinR], kt + kLinR - 1);
      const uint8_t* st = ring[u];
      const v8i fw = make_v8i(*reinterpret_cast<const uint4*>(st + rdW + c0),
                              *reinterpret_cast<const uint4*>(st + rdW + c1));
      const v8i fa = make_v8i(*reinterpret_cast<const uint4*>(st + rdA + c0),
                              *reinterpret_cast<const uint4*>(st + rdA + c1));
      acc = mfma_scaled(fw, fa, acc, sclW[4 * kt], sclA[4 * kt]);
    }
  }
  __builtin_amdgcn_s_waitcnt(wait_vm(0));           // no DMA outlives the workgroup

  const int t = 16 * wave + (lane & 15);
  const int n = n0 + 4 * q;
  if (t < p.T && n < p.N) *reinterpret_cast<uint2*>(p.out + static_cast<size_t>(t) * p.N + n) = pack4_bf16(acc);
}

// LDS the small-T kernel stages its scale rows in (dynamic shared memory).
constexpr size_t kSmallScaleLdsMax = 48 * 1024;
template <int NT, int SB>
constexpr size_t small_scale_lds(int K) { return static_cast<size_t>(16 * NT + 64) * (K / SB); }

template <int MODE>
void launch_decode(const SmallArgs& a, hipStream_t s) {   // a.K (bytes) = 1024, 2048, 4096 or 8192
  const int grid = a.G * a.n_groups;
  switch (a.K / kBK) {
    case 8: bmm_decode_kernel<8, MODE><<<grid, 256, 0, s>>>(a); break;
    case 16: bmm_decode_kernel<16, MODE><<<grid, 256, 0, s>>>(a); break;
    case 32: bmm_decode_kernel<32, MODE><<<grid, 256, 0, s>>>(a); break;
    default: bmm_decode_kernel<64, MODE><<<grid, 256, 0, s>>>(a); break;
  }
}

template <int NT, int SB>
void launch_small(const SmallArgs& a, bool fnuz, hipStream_t s) {
  const int grid = a.G * a.n_groups;
  const size_t lds = small_scale_lds<NT, SB>(a.K);   // staged scale rows
  if (fnuz)
    bmm_small_kernel<NT, SB, true><<<grid, kSmallThreads, lds, s>>>(a);
  else
    bmm_small_kernel<NT, SB, false><<<grid, kSmallThreads, lds, s>>>(a);
}

}  // namespace

// Batched GEMM dispatch (arguments validated by the caller).
mx_status launch_bmm(const uint8_t* a, const uint8_t* sa, int32_t a_fmt, const uint8_t* w, const uint8_t* sw,
                     void* out, int64_t T, int32_t G, int32_t N, int32_t K, hipStream_t stream) {
  if (T == 0) return MX_OK;
  const bool fnuz = a_fmt == MX_FP8_E4M3_FNUZ;
  if (T <= 64 && (K == 1024 || K == 2048 || K == 4096 || K == 8192) && aligned(sa, 4) && aligned(sw, 4)) {
    SmallArgs s{a, sa, w, sw, static_cast<uint16_t*>(out), static_cast<int>(T), G, N, K, (N + kDecRows - 1) / kDecRows};
    if (fnuz)
      launch_decode<kDecFnuz>(s, stream);
    else
      launch_decode<kDecOcp>(s, stream);
    count(C_BMM_SMALL);
    return launch_status("mx_bmm_a8w8_mxscale (decode batch)");
  }
  if (T <= 64 && small_scale_lds<4, 128>(K) <= kSmallScaleLdsMax) {   // (else the tiled kernels)
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
  const int KB = K / kBK;
  const int cus = device_cu_count();
  const bool persistent = (KB == 16 || KB == 32) && cus >= 8 && aligned(sa, 16) && aligned(sw, 16);
  if (persistent) {
    // one resident workgroup per compute unit, XCD-major (workgroup i runs on XCD i % 8)
    p.wg_per_xcd = std::min(p.per_xcd, cus / 8);
    const int grid = p.wg_per_xcd * 8;
    if (fnuz)
      bmm_persistent_kernel<true><<<grid, 256, 0, stream>>>(p);
    else
      bmm_persistent_kernel<false><<<grid, 256, 0, stream>>>(p);
  } else {
    p.wg_per_xcd = 0;
    const int grid = p.per_xcd * 8;
    if (fnuz)
      bmm_large_kernel<true, 128><<<grid, 256, 0, stream>>>(p);
    else
      bmm_large_kernel<false, 128><<<grid, 256, 0, stream>>>(p);
  }
  count(C_BMM_LARGE);
  return launch_status("mx_bmm_a8w8_mxscale");
}

// Block-32 scaled FP8 GEMM for the MXFP8 linear: out[M,N] = xq[M,K] * W[N,K]^T
// with scales [M,K/32] and [N,K/32], any M >= 1.
mx_status launch_gemm_mx32(const uint8_t* xq, const uint8_t* xs, const uint8_t* w, const uint8_t* sw, void* out,
                           int64_t M, int64_t N, int64_t K, hipStream_t stream) {
  if (M == 0 || N == 0) return MX_OK;
  if (M <= 64 && K <= 8192 && aligned(xs, 4) && aligned(sw, 4)) {
    // the LDS-DMA ring (M = 64, N = 4096: 10.9 -> 7.8 us at K = 1152 against
    // bmm_small_kernel<1, 32>)
    SmallArgs s{xq, xs, w, sw, static_cast<uint16_t*>(out), static_cast<int>(M), 1, static_cast<int>(N),
                static_cast<int>(K), static_cast<int>((N + kLinRowsW - 1) / kLinRowsW)};
    gemm_mx32_dma_kernel<<<s.n_groups, 256, 0, stream>>>(s);
    return launch_status("mx_linear (block-scaled FP8 GEMM)");
  }
  if (M <= 64 && small_scale_lds<1, 32>(static_cast<int>(K)) <= kSmallScaleLdsMax) {
    SmallArgs s{xq, xs, w, sw, static_cast<uint16_t*>(out), static_cast<int>(M), 1, static_cast<int>(N),
                static_cast<int>(K), static_cast<int>((N + 15) / 16)};
    launch_small<1, 32>(s, false, stream);
    return launch_status("mx_linear (block-scaled FP8 GEMM)");
  }
  // more rows (or K past the small kernels' scale staging): 256 x 256 tiles
  // of bmm_large_kernel with block-32 scales, one group
  LargeArgs p;
  p.a = xq; p.sa = xs; p.w = w; p.sw = sw;
  p.out = static_cast<uint16_t*>(out);
  p.T = static_cast<int>(M); p.G = 1; p.N = static_cast<int>(N); p.K = static_cast<int>(K);
  p.tiles_t = static_cast<int>((M + kLT - 1) / kLT);
  p.tiles_n = static_cast<int>((N + kLN - 1) / kLN);
  p.total_tiles = p.tiles_t * p.tiles_n;
  p.per_xcd = (p.total_tiles + 7) / 8;
  p.wg_per_xcd = 0;
  bmm_large_kernel<false, 32><<<p.per_xcd * 8, 256, 0, stream>>>(p);
  return launch_status("mx_linear (block-scaled FP8 GEMM, 256 x 256 tiles)");
}

// BF16 decode batch of the BF16 wo_a arm on the decode kernel: x [T, G, K],
// W [G, N, K] BF16, T <= 64, K in {512, 1024, 2048, 4096} (a row of 1, 2, 4 or
// 8 KiB); false if the shape is not one of these.
bool launch_bmm_bf16_decode(const void* x, const void* w, void* out, int64_t T, int32_t G, int32_t N, int32_t K,
                            hipStream_t stream) {
  const int bytes = 2 * K;
  if (T > 64 || !(bytes == 1024 || bytes == 2048 || bytes == 4096 || bytes == 8192)) return false;
  SmallArgs a{static_cast<const uint8_t*>(x), nullptr, static_cast<const uint8_t*>(w), nullptr,
              static_cast<uint16_t*>(out), static_cast<int>(T), G, N, bytes, (N + kDecRows - 1) / kDecRows};
  launch_decode<kDecBf16>(a, stream);
  return true;
}

}  // namespace mx
