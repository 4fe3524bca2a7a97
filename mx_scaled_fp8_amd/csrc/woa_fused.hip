// Single-kernel wo_a (gfx950): inverse RoPE, group-128 E8M0 quantisation and
// the batched a8w8 MX-scale GEMM in one pass, the activation going from BF16
// to FP8 inside the GEMM's A-tile load.
//
// "[ROCm][DSV4][Perf] Use FP8 WO_A output projection", Summary: the path is
// an inverse RoPE fused with per-token E8M0 group quantisation, then the MX
// batched GEMM with the checkpoint's FP8 weight.  The pages run the two as
// separate operators; here the quantiser's output never leaves the compute
// unit: out[t, g, n] = sum_k dec(q[t,g,k]) 2^(sa-127) dec(W[g,n,k]) 2^(sw-127)
// with q, sa exactly the quantiser's (OCP codes; the result of an FNUZ run
// is the same), fp32 accumulation, BF16 out.
//
// Design: one 256 (t) x 256 (n) tile per workgroup, 8 waves (two per SIMD)
// of 64 t x 128 n on v_mfma_scale_f32_32x32x64_f8f6f4, K-steps of 128.  A
// 128-wide K-step of a token row is exactly one quantisation group, so each
// stage quantises whole groups:
//  * A arrives as BF16 in registers by buffer loads, two stages ahead: each
//    wave quantises 32 of the tile's rows, 8 lanes per row, each lane two
//    16-byte chunks (a, a + d) of the row's 256-byte stage slice;
//  * a stage that holds the last 128 dims of a head rotates its last R dims
//    (R <= 64; fp32, products and sums rounded one by one, BF16 nearest
//    even): with d = 8 the interleaved pairs lie inside a chunk, with
//    d = R/16 the split-half pairs (i, i + R/2) are the lane's two chunks;
//    the tokens' cos/sin rows come by LDS-DMA into the stage's A slot,
//    each where its token's codes will go;
//  * the group amax is a packed-u16 max over the lane's 16 values and three
//    DPP steps over the row's 8 lanes; the E8M0 byte is integer arithmetic on
//    its bits; the codes come from v_cvt_scalef32_pk_fp8_bf16 (the
//    quantiser's instructions, so the codes are the quantiser's);
//  * codes go to the stage's A slot in LDS (the swizzled layout the MFMA
//    fragment reads use), scale bytes to a per-buffer A-scale array;
//  * W goes global -> LDS by LDS-DMA (buffer loads) as in bmm_large_kernel.
// Per stage: the MFMAs of stage kb from LDS, with the quantisation of stage
// kb+1 (into the other A slot) and the loads of stage kb+2's BF16 placed
// between them; one barrier; then the W DMA of stage kb+2 into the slot
// stage kb used.  A token whose position is outside the table gets NaN
// scales (its outputs are NaN), as from the quantiser.
#include <algorithm>
#include <type_traits>

#include "common.hpp"

namespace mx {

namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
typedef short v2s __attribute__((ext_vector_type(2)));
typedef unsigned short v2u16 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) void lds_void_t;

constexpr int kTile = 256;                  // tile rows along t and n
constexpr int kBK = 128;                    // K bytes of FP8 per stage = one quantisation group
constexpr int kOpBytes = kTile * kBK;       // 32 KiB per operand per stage
constexpr int kMaxKB = 32;                  // K <= 4096: the W scales of a tile stay in LDS
constexpr int kFmtFp8 = 0;
constexpr int kWaitVmMax = kWaitLgkmOnly;  // LDS traffic only
template <int N>
using ic = std::integral_constant<int, N>;
typedef unsigned int v4u __attribute__((ext_vector_type(4)));
// calls f(ic<k>) for k = B .. E-1, in order
template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(ic<B>{});
    static_for<B + 1, E>(f);
  }
}
// MFMA q of a row group is issued at point hook_of(per_group, q) (0..3) of
// the group's work: 0 and 2 for two MFMAs per group, else 0, 1, 2, ...
constexpr int hook_of(int per_group, int q) { return per_group == 2 ? 2 * q : q; }

struct FusedArgs {
  const uint16_t* x;          // [T, H*D] BF16
  const int64_t* pos;         // [T]
  const uint16_t* cos;        // [max_pos, R/2]
  const uint16_t* sin;
  int64_t max_pos;
  const uint8_t* w;           // [G, N, K] OCP e4m3
  const uint8_t* sw;          // [G, N, K/128]
  uint16_t* out;              // [T, G, N]
  int T, G, N, K, D, R;
  int cd;                     // chunk distance of a lane's two chunks: 8, or R/16 (split halves)
  int tiles_t, tiles_n, total_tiles, per_xcd;
};

__device__ __forceinline__ int swz8(int r) { return ((r >> 1) ^ ((r & 1) << 2)) & 7; }

// Workgroup barrier that the compiler may not move memory accesses across
// (the waits that make the data visible are issued explicitly before it).
__device__ __forceinline__ void stage_barrier() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

__device__ __forceinline__ v8i make_v8i(const uint4 lo, const uint4 hi) {
  v8i r;
  r[0] = lo.x; r[1] = lo.y; r[2] = lo.z; r[3] = lo.w;
  r[4] = hi.x; r[5] = hi.y; r[6] = hi.z; r[7] = hi.w;
  return r;
}

template <int CTRL>
__device__ __forceinline__ uint32_t dpp(uint32_t v) {
  return static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), CTRL, 0xF, 0xF, false));
}

// max over the 8 lanes of a row: xor 1, xor 2 (quad permutes), then lane i
// against lane 7 - i (row_half_mirror) joins the two quads
__device__ __forceinline__ uint32_t max8(uint32_t m) {
  m = max(m, dpp<0xB1>(m));
  m = max(m, dpp<0x4E>(m));
  m = max(m, dpp<0x141>(m));
  return m;
}

__device__ __forceinline__ uint32_t amax_bits8(const uint4 v) {
  const v2u16 a = __builtin_bit_cast(v2u16, v.x & 0x7FFF7FFFu);
  const v2u16 b = __builtin_bit_cast(v2u16, v.y & 0x7FFF7FFFu);
  const v2u16 c = __builtin_bit_cast(v2u16, v.z & 0x7FFF7FFFu);
  const v2u16 d = __builtin_bit_cast(v2u16, v.w & 0x7FFF7FFFu);
  const v2u16 m = __builtin_elementwise_max(__builtin_elementwise_max(a, b), __builtin_elementwise_max(c, d));
  return max(static_cast<uint32_t>(m[0]), static_cast<uint32_t>(m[1]));
}

__device__ __forceinline__ uint32_t pk_bf16(float lo, float hi) {
  const v2bf r = {static_cast<__bf16>(lo), static_cast<__bf16>(hi)};
  return __builtin_bit_cast(uint32_t, r);
}

// (x, y) -> (x*c + y*s, y*c - x*s), every operation rounded to fp32
__device__ __forceinline__ void inv_rotate(float x, float y, float c, float s, float& xr, float& yr) {
  const float xc = x * c, ys = y * s, yc = y * c, xs = x * s;
  xr = xc + ys;
  yr = yc - xs;
}

// OCP codes of the 8 BF16 values of v divided by 2^e (sbits: E8M0 byte << 23)
__device__ __forceinline__ uint2 encode8(const uint4 v, float sbits) {
  // both halves of lo and hi are written: their initial values are any bits
  // at hand (v.x and v.y, so that the pair lands in adjacent registers)
  v2s lo = __builtin_bit_cast(v2s, v.x), hi = __builtin_bit_cast(v2s, v.y);
  lo = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(lo, __builtin_bit_cast(v2bf, v.x), sbits, false);
  lo = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(lo, __builtin_bit_cast(v2bf, v.y), sbits, true);
  hi = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(hi, __builtin_bit_cast(v2bf, v.z), sbits, false);
  hi = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(hi, __builtin_bit_cast(v2bf, v.w), sbits, true);
  return make_uint2(__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi));
}

// W tile I times A tile J (of the wave's NJ); the scale operands are 4-byte
// words holding the scales of the wave's tiles and the byte selects pick
// tile I's and J's
template <int I, int J, int NJ>
__device__ __forceinline__ void mfma_ij(v16f (&acc)[4][NJ], const v8i (&w)[4], const v8i (&a)[NJ], uint32_t swv,
                                        uint32_t sav) {
  acc[I][J] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(w[I], a[J], acc[I][J], kFmtFp8, kFmtFp8, I,
                                                             static_cast<int>(swv), J, static_cast<int>(sav));
}

template <int IJ, int END, int NJ>
__device__ __forceinline__ void mfma_range(v16f (&acc)[4][NJ], const v8i (&w)[4], const v8i (&a)[NJ], uint32_t swv,
                                           uint32_t sav) {
  if constexpr (IJ < END) {
    mfma_ij<IJ / NJ, IJ % NJ, NJ>(acc, w, a, swv, sav);
    mfma_range<IJ + 1, END, NJ>(acc, w, a, swv, sav);
  }
}

template <int NW, bool ROPE, bool NEOX>
__global__ __launch_bounds__(64 * NW, 1) void woa_fused_kernel(FusedArgs p) {
  static_assert(NW == 4 || NW == 8, "4 or 8 waves");
  constexpr int NJ = NW == 4 ? 4 : 2;              // A tiles of 32 rows per wave (W tiles: 4)
  constexpr int kRowsPerWave = kTile / NW;         // rows a wave quantises: 64 or 32
  constexpr int NG = kRowsPerWave / 8;             // its row groups of 8 rows
  constexpr int kWDma = kTile / (8 * NW);          // W DMA instructions per wave and stage
  constexpr int kALoads = 2 * NG;                  // A loads per wave and stage
  constexpr int kMfmas = 8 * NJ;                   // MFMAs per wave and stage (two K-halves)
  constexpr int kPure = kMfmas / 4;                // MFMAs of a stage before its quantisation work
  constexpr int kPerGroup = (kMfmas - kPure) / NG; // MFMAs with each row group
  static_assert(kPerGroup * NG + kPure == kMfmas && kPerGroup >= 1 && kPerGroup <= 4, "MFMAs per row group");
  // stage buffers 0 and 1: W tile 256 x 128 B (sw) and A tile 256 x 128 B
  // (sa), four separate arrays so that the compiler can tell the weight DMA
  // from the activation codes and tables (with one array per stage it made
  // the code stores and table reads wait for the weight DMA of the stage)
  __shared__ __attribute__((aligned(1024))) uint8_t sw0[kOpBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t sa0[kOpBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t sw1[kOpBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t sa1[kOpBytes];
  // W scales of every stage of the tile, [stage][wave half][row % 32][tile]
  __shared__ __attribute__((aligned(16))) uint8_t wsc[kMaxKB][2][32][4];
  // A scales of the stage in each buffer, [buffer][wave row wt][row % 32][tile j < NJ]
  __shared__ __attribute__((aligned(16))) uint8_t asc[2][4][32][4];
  // positions of the tile's rows (-1: outside the table)
  __shared__ int32_t spos[kTile];

  const int xcd = blockIdx.x & 7;
  const int work = xcd * p.per_xcd + (blockIdx.x >> 3);
  if (work >= p.total_tiles) return;
  const int nt = work % p.tiles_n;
  const int tt = (work / p.tiles_n) % p.tiles_t;
  const int g = work / (p.tiles_n * p.tiles_t);
  const int t0 = tt * kTile, n0 = nt * kTile;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wn = wave & 1, wt = wave >> 1;
  const int KB = p.K / kBK;                        // <= kMaxKB
  // K rotation by token tile only: the tile's 4 n-tiles (neighbouring
  // workgroups of one XCD) read each stage's BF16 activation rows at about
  // the same time, so the rows come from HBM once and from L2 for the rest
  // (with the n-tiles a stage apart, as in bmm_large_kernel, 2.0-2.4 GB were
  // fetched per prefill chunk against 1.47 GB)
  const int kb0 = tt % KB;
  const int L = p.G * p.K;                         // elements per token row (H * D)
  auto real_stage = [&](int kb) __attribute__((always_inline)) {
    int kr = kb + kb0;
    return kr >= KB ? kr - KB : kr;
  };

  // ---- W: LDS-DMA of the stage's 256 rows (rows past N re-read the last one).
  // Every LDS-DMA here is a buffer load: with a global (flat-encoded) LDS-DMA
  // in flight the compiler waits for all vector memory before the first use of
  // any loaded register, which would hold each stage's quantisation until the
  // weight DMA issued just before it had landed.
  const int dma_row = wave * 8 + (lane >> 3);
  const uint32_t dma_chunk = static_cast<uint32_t>((lane & 7) ^ swz8(dma_row)) * 16;
  const uint8_t* baseW = p.w + (static_cast<size_t>(g) * p.N + n0) * p.K;
  const int limW = p.N - 1 - n0;
  // lane offset of row group 0 and the cap past which rows re-read the last one
  const uint32_t offW0 = static_cast<uint32_t>(dma_row) * static_cast<uint32_t>(p.K) + dma_chunk;
  const uint32_t capW = static_cast<uint32_t>(limW) * static_cast<uint32_t>(p.K) + dma_chunk;
  const __amdgpu_buffer_rsrc_t wres = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(baseW), 0, static_cast<int>(static_cast<uint32_t>(limW + 1) * static_cast<uint32_t>(p.K)),
      kBufferFlags);
  auto issue_w = [&](uint8_t* bw, int kb) __attribute__((always_inline)) {
    const int so = real_stage(kb) * kBK;
#pragma unroll
    for (int it = 0; it < kWDma; ++it) {
      uint32_t b = offW0;
      asm volatile("" : "+v"(b));                    // formed per issue, not held as 8 addresses
      const uint32_t o = min(b + static_cast<uint32_t>(it * 8 * NW) * static_cast<uint32_t>(p.K), capW);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(wres, (lds_void_t*)(bw + (it * 8 * NW + wave * 8) * kBK), 16,
                                               static_cast<int>(o), so, 0, 0);
    }
  };

  // ---- A: lane (row ri = lane / 8 of a group of 8 rows, c = lane % 8)
  // holds chunks ca and ca + cd of the row's 16 chunks of 8 BF16; wave w
  // quantises tile rows R w .. R w + R - 1, R = kRowsPerWave (row group j:
  // rows R w + 8j + ri)
  const int ri = lane >> 3, c = lane & 7;
  const int cd = p.cd;
  const int ca = (c / cd) * 2 * cd + (c % cd);
  const int cb = ca + cd;
  const int arow0 = wave * kRowsPerWave + ri;     // tile row of row group 0
  // A goes through a buffer resource whose base is the tile's first row
  // (group g's columns) and whose size ends at row T: rows past T read
  // zeros (their outputs are never stored).  A lane's two offsets are fixed
  // for the tile; the row group and the stage enter as the scalar offset, so
  // a load costs no address arithmetic.  Offsets stay below 2^32: at most
  // 255 rows of H*D < 2^23 BF16 plus one group's 2 K bytes.
  const uint32_t row_bytes = static_cast<uint32_t>(L) * 2;
  const uint64_t valid_bytes = static_cast<uint64_t>(p.T - t0) * row_bytes;
  const __amdgpu_buffer_rsrc_t xres = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(p.x + static_cast<size_t>(t0) * L + static_cast<size_t>(g) * p.K), 0,
      static_cast<int>(min(valid_bytes, static_cast<uint64_t>(0xFFFFFFFFu))), kBufferFlags);
  const uint32_t voff_a = static_cast<uint32_t>(arow0) * row_bytes + static_cast<uint32_t>(ca) * 16;
  const uint32_t voff_b = voff_a + static_cast<uint32_t>(cd) * 16;
  uint4 av[NG][2];
  auto stage_soff = [&](int kb) __attribute__((always_inline)) {
    return static_cast<uint32_t>(real_stage(kb)) * (2 * kBK);
  };
  // row group j of the stage at scalar offset soff into av[j]
  auto load_group = [&](int j, uint32_t soff) __attribute__((always_inline)) {
    const uint32_t so = soff + static_cast<uint32_t>(8 * j) * row_bytes;
    const v4u a0 = __builtin_amdgcn_raw_buffer_load_b128(xres, static_cast<int>(voff_a), static_cast<int>(so), 0);
    const v4u a1 = __builtin_amdgcn_raw_buffer_load_b128(xres, static_cast<int>(voff_b), static_cast<int>(so), 0);
    av[j][0] = make_uint4(a0.x, a0.y, a0.z, a0.w);
    av[j][1] = make_uint4(a1.x, a1.y, a1.z, a1.w);
  };
  auto load_a = [&](int kb) __attribute__((always_inline)) {
    const uint32_t soff = stage_soff(kb);
#pragma unroll
    for (int j = 0; j < NG; ++j) load_group(j, soff);
  };

  // rows of the lane's row groups whose position is outside the table (bit j)
  uint32_t bad_rows = 0;
  const int R = p.R;
  const int half = R >> 1;
  // bit kb: loop stage kb holds the last 128 dims of a head (the rotated
  // slice).  Taken once per tile into a scalar register, so that the choice
  // of rotating code per stage is a uniform branch.
  uint32_t rope_bits = 0;
  if constexpr (ROPE) {
    for (int kb = 0; kb < KB; ++kb) {
      const int colg = g * p.K + real_stage(kb) * kBK;
      rope_bits |= ((colg + kBK) % p.D == 0 ? 1u : 0u) << kb;
    }
    rope_bits = __builtin_amdgcn_readfirstlane(rope_bits);
  }
  auto rope_stage = [&](int kb) __attribute__((always_inline)) { return ROPE && ((rope_bits >> kb) & 1u); };

  // ---- quantise the stage in av[] into buffer `buf` (A region) and asc[sb]
  // LDS byte offsets of the lane's two 8-byte code pieces in row group 0:
  // row tr = arow0 + 8j is at + 1024 j, and its swizzle swz8(tr) depends on
  // tr % 16 only (kRowsPerWave is a multiple of 16), so it is swz8(ri) for
  // even j and swz8(ri) ^ 4 for odd j
  const int szr = swz8(ri);
  auto piece_off = [&](int ch, int sz) __attribute__((always_inline)) { return (((ch >> 1) ^ sz) << 4) + (ch & 1) * 8; };
  const uint32_t qoff[2][2] = {
      {static_cast<uint32_t>(arow0 * kBK + piece_off(ca, szr)), static_cast<uint32_t>(arow0 * kBK + piece_off(ca, szr ^ 4))},
      {static_cast<uint32_t>(arow0 * kBK + piece_off(cb, szr)), static_cast<uint32_t>(arow0 * kBK + piece_off(cb, szr ^ 4))}};
  // asc byte of tile row tr = arow0 + 8j (A tile tr / 32 = wave R / 32 + j / 4
  // is tile (tr / 32) % NJ of wave row (tr / 32) / NJ): [wave row][tr % 32][tile]
  auto sc_index = [&](int j) __attribute__((always_inline)) {
    const int blk = wave * (kRowsPerWave / 32) + (j >> 2);
    return (blk / NJ) * 128 + (8 * (j & 3) + ri) * 4 + blk % NJ;
  };
  // ---- rotation tables of a rope stage: the cos and sin rows of the tile's
  // tokens go by LDS-DMA into the A region of the stage's buffer (free until
  // the stage's codes are written there), each at the 128 bytes its token's
  // codes will take: cos[R/2] then sin[R/2] (R <= 64).  A wave loads and
  // reads only its own rows, and a row's codes are written after its
  // rotation has read its tables, so no barrier is involved.  Two DMA
  // instructions per row group (cos, then sin R bytes further on),
  // 8 rows, the R/16 lanes of a row's pieces enabled.  The tables are read
  // through buffer resources (the host keeps max_pos * R below 2^31).
  const uint32_t tab_bytes = static_cast<uint32_t>(p.max_pos * R);
  const __amdgpu_buffer_rsrc_t cres =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(p.cos), 0, static_cast<int>(tab_bytes), kBufferFlags);
  const __amdgpu_buffer_rsrc_t sres =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(p.sin), 0, static_cast<int>(tab_bytes), kBufferFlags);
  auto issue_cs = [&](uint8_t* ba, int kb) __attribute__((always_inline)) {
    if (!ROPE || !rope_stage(kb)) return;
    uint8_t* dst = ba + wave * kRowsPerWave * kBK;
    const int piece = lane & 7;
    const int npc = R >> 4;                          // 16-byte pieces per table row
#pragma unroll
    for (int k = 0; k < NG; ++k) {
      int tr = wave * kRowsPerWave + k * 8 + (lane >> 3);   // tile row
      asm volatile("" : "+v"(tr));                   // read here, not hoisted as 8 live positions
      const int pj = max(spos[tr], 0);               // outside the table: row 0 (its codes are NaN)
      const int off = pj * R + piece * 16;
      if (piece < npc) {
        __builtin_amdgcn_raw_ptr_buffer_load_lds(cres, (lds_void_t*)(dst + k * 1024), 16, off, 0, 0, 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(sres, (lds_void_t*)(dst + k * 1024 + npc * 16), 16, off, 0, 0, 0);
      }
    }
  };

  // rotation of one row group's two chunks (local copies), from the tables
  // at `tab`: a chunk outside the rotated slice reads pair 0 and keeps its
  // own value
  const int first_rot = (kBK - R) / 8;             // first rotated chunk of a head's last stage
  const bool rot_a = ca >= first_rot;
  const bool rot_b = NEOX ? ca >= first_rot : cb >= first_rot;
  const int ti_a = NEOX ? (rot_a ? (ca - first_rot) * 8 : 0) : (rot_a ? (ca - first_rot) * 4 : 0);
  const int ti_b = NEOX ? ti_a : (rot_b ? (cb - first_rot) * 4 : 0);
  // all-ones where the chunk is rotated: the rotated value is blended in
  // with these (opaque to the compiler, which otherwise turned the choice
  // into divergent branches around the rotation)
  uint32_t rmask_a = rot_a ? ~0u : 0u, rmask_b = rot_b ? ~0u : 0u;
  asm volatile("" : "+v"(rmask_a), "+v"(rmask_b));
  auto blend = [](uint4 v, const uint4 r, uint32_t msk) __attribute__((always_inline)) {
    v.x = (r.x & msk) | (v.x & ~msk);
    v.y = (r.y & msk) | (v.y & ~msk);
    v.z = (r.z & msk) | (v.z & ~msk);
    v.w = (r.w & msk) | (v.w & ~msk);
    return v;
  };
  auto rotate2 = [&](const uint8_t* tab, uint4& v0, uint4& v1) __attribute__((always_inline)) {
    const uint16_t* crow = reinterpret_cast<const uint16_t*>(tab);
    const uint16_t* srow = crow + half;
    if constexpr (!NEOX) {
      // pairs (2i, 2i+1) of the rotated slice: a chunk's 4 dwords are 4 pairs
      auto rot_chunk = [&](const uint4 v, const uint2 cc, const uint2 ss) __attribute__((always_inline)) {
        float xr, yr;
        uint4 r;
        inv_rotate(bf16_lo(v.x), bf16_hi(v.x), bf16_lo(cc.x), bf16_lo(ss.x), xr, yr);
        r.x = pk_bf16(xr, yr);
        inv_rotate(bf16_lo(v.y), bf16_hi(v.y), bf16_hi(cc.x), bf16_hi(ss.x), xr, yr);
        r.y = pk_bf16(xr, yr);
        inv_rotate(bf16_lo(v.z), bf16_hi(v.z), bf16_lo(cc.y), bf16_lo(ss.y), xr, yr);
        r.z = pk_bf16(xr, yr);
        inv_rotate(bf16_lo(v.w), bf16_hi(v.w), bf16_hi(cc.y), bf16_hi(ss.y), xr, yr);
        r.w = pk_bf16(xr, yr);
        return r;
      };
      // a lane's first chunk (ca = c < 8) lies before the rotated slice,
      // which starts at chunk (128 - R) / 8 >= 8 for R <= 64: only the
      // second chunk can be rotated
      const uint4 rb = rot_chunk(v1, *reinterpret_cast<const uint2*>(crow + ti_b),
                                 *reinterpret_cast<const uint2*>(srow + ti_b));
      v1 = blend(v1, rb, rmask_b);
    } else {
      // pairs (i, i + R/2): chunk ca holds x of pairs i0 .. i0+7, chunk cb their y
      const uint4 cc = *reinterpret_cast<const uint4*>(crow + ti_a);
      const uint4 ss = *reinterpret_cast<const uint4*>(srow + ti_a);
      const uint32_t xw[4] = {v0.x, v0.y, v0.z, v0.w};
      const uint32_t yw[4] = {v1.x, v1.y, v1.z, v1.w};
      const uint32_t cw[4] = {cc.x, cc.y, cc.z, cc.w};
      const uint32_t sw4[4] = {ss.x, ss.y, ss.z, ss.w};
      uint32_t xo[4], yo[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        float x0, y0, x1, y1;
        inv_rotate(bf16_lo(xw[k]), bf16_lo(yw[k]), bf16_lo(cw[k]), bf16_lo(sw4[k]), x0, y0);
        inv_rotate(bf16_hi(xw[k]), bf16_hi(yw[k]), bf16_hi(cw[k]), bf16_hi(sw4[k]), x1, y1);
        xo[k] = pk_bf16(x0, x1);
        yo[k] = pk_bf16(y0, y1);
      }
      v0 = blend(v0, make_uint4(xo[0], xo[1], xo[2], xo[3]), rmask_a);
      v1 = blend(v1, make_uint4(yo[0], yo[1], yo[2], yo[3]), rmask_a);
    }
  };

  // quantise row group j of the stage in av[] into buffer `buf` (A region)
  // and asc[sb], rotating it first if `rs` (a rope stage; a uniform branch
  // around the rotation alone, so that no MFMA is on either side of it).
  // The 8 lanes of a row hold the same scale byte and all of them store it.
  // `between(k)`, k = 0..3, runs at four fixed points of the work (the
  // stage loop puts one MFMA there); the order is pinned by scheduling
  // barriers, so that each MFMA runs beside the vector work after it.
  // The waits for the group's loads are the compiler's (before the first
  // use of a loaded register).  The table DMA of a rope stage is waited for
  // here, before the first group rotates: `tab_wait` is the number of
  // vector-memory instructions this wave issued after it (0: already waited).
  auto quant_group = [&](bool rs, auto jc, uint8_t* ba, int sb, auto tab_wait, auto&& between)
                         __attribute__((always_inline)) {
    constexpr int j = decltype(jc)::value;
    uint4 v0 = av[j][0], v1 = av[j][1];
    if (ROPE && rs) {
      if constexpr (j == 0 && decltype(tab_wait)::value > 0)
        __builtin_amdgcn_s_waitcnt(wait_vm_only(decltype(tab_wait)::value));
      rotate2(ba + (arow0 + 8 * j) * kBK, v0, v1);
    }
    uint32_t m = max(amax_bits8(v0), amax_bits8(v1));
    if (ROPE && ((bad_rows >> j) & 1)) m = 0x7F80u;   // position outside the table: NaN scale
    between(ic<0>{});
    m = max8(m);
    const bool finite = m < 0x7F80u;
    // the E8M0 byte, e8m0_exponent<8>(m) + 127 for a finite amax, in three
    // operations: with 0x1F added the mantissa field carries into the
    // exponent field exactly when it exceeds 0x60, so the byte is
    // ((m + 0x1F) >> 7) - 8, clamped at 0; the subtraction of 8 << 7 goes
    // first and the shift is arithmetic
    const int eb = max(static_cast<int>(m - 0x3E1u) >> 7, 0);
    const float sbits = __uint_as_float(static_cast<uint32_t>(eb) << 23);
    between(ic<1>{});
    uint2 q0 = encode8(v0, sbits), q1 = encode8(v1, sbits);
    // a non-finite group: codes 0x7F (a blend with an opaque mask, which the
    // compiler does not turn into a branch)
    uint32_t fin = finite ? ~0u : 0u;
    asm volatile("" : "+v"(fin));
    q0.x = (q0.x & fin) | (0x7F7F7F7Fu & ~fin);
    q0.y = (q0.y & fin) | (0x7F7F7F7Fu & ~fin);
    q1.x = (q1.x & fin) | (0x7F7F7F7Fu & ~fin);
    q1.y = (q1.y & fin) | (0x7F7F7F7Fu & ~fin);
    between(ic<2>{});
    *reinterpret_cast<uint2*>(ba + qoff[0][j & 1] + j * 8 * kBK) = q0;
    *reinterpret_cast<uint2*>(ba + qoff[1][j & 1] + j * 8 * kBK) = q1;
    (&asc[sb][0][0][0])[sc_index(j)] = static_cast<uint8_t>(finite ? eb : 0xFF);
    between(ic<3>{});
  };
  auto quantise = [&](int kb, uint8_t* ba, int sb) __attribute__((always_inline)) {
    const bool rs = rope_stage(kb);
    static_for<0, NG>([&](auto jc) __attribute__((always_inline)) { quant_group(rs, jc, ba, sb, ic<0>{}, [](auto) {}); });
  };

  // ---- fragments (as bmm_large_kernel): row wn*128 + 32i + lane%32 of W,
  // wt*32*NJ + 32j + lane%32 of A; lane group q2 takes logical chunks 4h + q2
  // and 4h + q2 + 2 of 64-K half h
  const int r32 = lane & 31;
  const int q2 = lane >> 5;
  const int rdW = (wn * 128 + r32) * kBK;
  const int rdA = (wt * 32 * NJ + r32) * kBK;
  const int sz = swz8(r32);
  const int ch0[2] = {(q2 ^ sz) << 4, ((4 + q2) ^ sz) << 4};
  const int ch1[2] = {((q2 + 2) ^ sz) << 4, ((6 + q2) ^ sz) << 4};
  auto read_frag = [&](const uint8_t* q, int h) __attribute__((always_inline)) {
    return make_v8i(*reinterpret_cast<const uint4*>(q + ch0[h]), *reinterpret_cast<const uint4*>(q + ch1[h]));
  };

  v16f acc[4][NJ];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  // One stage: the kMfmas MFMAs of stage kb (two K-halves of fragments, the
  // second read when the first half's MFMAs are issued).
  // MODE 1 and 2 quantise stage kb+1 (av[] into `na`) alongside them: the
  // first kPure MFMAs run alone, then each row group goes with kPerGroup
  // MFMAs placed at fixed points of its work (scheduling barriers and opaque
  // accumulator copies pin the order, so each MFMA runs beside the vector
  // work after it).  The first use of av[] waits for every load and DMA in
  // flight -- the compiler's rule while LDS-DMA is outstanding -- so the MFMAs
  // before it give the previous iteration's weight DMA that much more time.
  // MODE 2 also reloads each row group's registers with stage kb+2's BF16 as
  // soon as they are free.
  auto step = [&](auto mode, const uint8_t* cw, const uint8_t* ca, uint8_t* na, int kb) __attribute__((always_inline)) {
    constexpr int MODE = decltype(mode)::value;
    const uint32_t swv = *reinterpret_cast<const uint32_t*>(&wsc[real_stage(kb)][wn][r32][0]);
    const uint32_t sav = *reinterpret_cast<const uint32_t*>(&asc[kb & 1][wt][r32][0]);
    const bool rs = MODE >= 1 && rope_stage(kb + 1);
    const uint32_t nb = MODE == 2 ? stage_soff(kb + 2) : 0u;
    v8i fw[4], fa[NJ];
    auto read_w = [&](int i, int h) __attribute__((always_inline)) { fw[i] = read_frag(cw + rdW + i * 32 * kBK, h); };
    auto read_a = [&](int h) __attribute__((always_inline)) {
#pragma unroll
      for (int j = 0; j < NJ; ++j) fa[j] = read_frag(ca + rdA + j * 32 * kBK, h);
    };
    auto pin_all = [&]() __attribute__((always_inline)) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j) asm volatile("" : "+a"(acc[i][j]));
    };
    auto mfma_at = [&](auto mc) __attribute__((always_inline)) {   // MFMA m of the stage
      constexpr int m = decltype(mc)::value, K = m % (4 * NJ), I = K / NJ;
      __builtin_amdgcn_sched_barrier(0);
      // the second half's fragments: A and W tiles 0 and 1 at its first MFMA,
      // then W tile I + 1 at the first MFMA of W tile I (two W tiles live at
      // a time, while the quantisation runs beside these MFMAs)
      if constexpr (m == 4 * NJ) {
        pin_all();
        read_a(1);
        read_w(0, 1);
        read_w(1, 1);
      } else if constexpr (m > 4 * NJ && K % NJ == 0 && I + 1 < 4) {
        read_w(I + 1, 1);
      }
      asm volatile("" : "+a"(acc[K / NJ][K % NJ]));
      mfma_range<K, K + 1, NJ>(acc, fw, fa, swv, sav);
      asm volatile("" : "+a"(acc[K / NJ][K % NJ]));
      __builtin_amdgcn_sched_barrier(0);
    };
    read_a(0);
#pragma unroll
    for (int i = 0; i < 4; ++i) read_w(i, 0);
    if constexpr (MODE == 0) {
      static_for<0, kMfmas>(mfma_at);
    } else {
      static_for<0, kPure>(mfma_at);
      static_for<0, NG>([&](auto gc) __attribute__((always_inline)) {
        constexpr int g = decltype(gc)::value;
        // the tables of stage kb+1 came before its W DMA; in MODE 2 that is
        // the last DMA issued (MODE 1 waited for everything at its start)
        quant_group(rs, gc, na, (kb + 1) & 1, ic<MODE == 2 ? kWDma : 0>{}, [&](auto kc) __attribute__((always_inline)) {
          static_for<0, kPerGroup>([&](auto qc) __attribute__((always_inline)) {
            constexpr int q = decltype(qc)::value;
            if constexpr (hook_of(kPerGroup, q) == decltype(kc)::value) mfma_at(ic<kPure + g * kPerGroup + q>{});
          });
        });
        if constexpr (MODE == 2) load_group(g, nb);
      });
    }
    pin_all();
    __builtin_amdgcn_sched_barrier(0);
  };

  // ---- prologue: positions, the tile's W scales, stage 0 quantised, stage 1 on its way
  if (tid < kTile) {
    if constexpr (ROPE) {
      const int64_t pp = p.pos[min(t0 + tid, p.T - 1)];
      spos[tid] = (pp >= 0 && pp < p.max_pos) ? static_cast<int32_t>(pp) : -1;
    }
    // thread tid stages W row tid's scale bytes of all stages
    const uint8_t* scw = p.sw + (static_cast<size_t>(g) * p.N + n0 + min(tid, limW)) * KB;
    for (int s = 0; s < KB; ++s) wsc[s][tid >> 7][tid & 31][(tid >> 5) & 3] = scw[s];
  }
  __builtin_amdgcn_s_waitcnt(kWaitVmMax);
  stage_barrier();                                   // spos is written
  if constexpr (ROPE) {
#pragma unroll
    for (int j = 0; j < NG; ++j) bad_rows |= (spos[arow0 + 8 * j] < 0 ? 1u : 0u) << j;
  }
  load_a(0);
  issue_cs(sa0, 0);
  issue_w(sw0, 0);
  __builtin_amdgcn_s_waitcnt(wait_vm(0));
  stage_barrier();
  quantise(0, sa0, 0);
  if (KB > 1) {                                      // stage 1 into the unused buffer
    load_a(1);
    issue_cs(sa1, 1);
    issue_w(sw1, 1);
  }
  __builtin_amdgcn_s_waitcnt(kWaitVmMax);
  stage_barrier();                                   // stage 0's codes are in st0

  // ---- stage loop.  On entry to iteration kb: buffer kb%2 holds stage kb
  // (W and the quantised A); this wave's loads of stage kb+1's BF16, its
  // rotation tables and then the DMA of its W (into the other buffer) may be
  // in flight.  The last two stages are peeled (no reload, then no
  // quantisation).  (Every lambda is inlined and no iteration skips the
  // MFMAs: with a first iteration that did, or with the quantiser as a
  // called function, the register allocator moved the accumulators through
  // scratch memory on every stage.)
  // One loop iteration with its buffers named: kb even reads st0 and fills
  // st1, kb odd the reverse.  With the buffers fixed per call (the loop runs
  // two stages per trip) the compiler can tell the fragment reads from the
  // DMA into the other buffer; with a run-time choice it made every stage
  // wait for all outstanding loads first.
  auto iter = [&](uint8_t* cw, uint8_t* ca, uint8_t* na, int kb) __attribute__((always_inline)) {
    step(ic<2>{}, cw, ca, na, kb);
    // stage kb+1's W has landed once at most stage kb+2's loads are pending
    __builtin_amdgcn_s_waitcnt(wait_vm(kALoads));
    stage_barrier();                                 // everyone is done with stage kb's buffers; stage kb+1 is in the other
    issue_cs(ca, kb + 2);
    issue_w(cw, kb + 2);
  };
  int kb = 0;
  for (; kb + 3 < KB; kb += 2) {
    iter(sw0, sa0, sa1, kb);
    iter(sw1, sa1, sa0, kb + 1);
  }
  if (kb + 2 < KB) {                                 // kb even
    iter(sw0, sa0, sa1, kb);
    ++kb;
  }
  if (kb + 1 < KB) {                                 // kb = KB - 2
    // stage kb+1's BF16 and tables have landed once at most its W DMA is pending
    __builtin_amdgcn_s_waitcnt(wait_vm(kWDma));
    step(ic<1>{}, (kb & 1) ? sw1 : sw0, (kb & 1) ? sa1 : sa0, (kb & 1) ? sa0 : sa1, kb);
    __builtin_amdgcn_s_waitcnt(wait_vm(0));
    stage_barrier();
    ++kb;
  }
  step(ic<0>{}, (kb & 1) ? sw1 : sw0, (kb & 1) ? sa1 : sa0, nullptr, kb);   // kb = KB - 1
  __builtin_amdgcn_s_waitcnt(wait_vm(0));          // no DMA outlives the workgroup

  // ---- epilogue straight from the accumulators (as bmm_large_kernel)
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const int t = t0 + wt * 32 * NJ + j * 32 + r32;
    uint16_t* orow = p.out + (static_cast<size_t>(t) * p.G + g) * p.N;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      // the block's 16 values, each read out of its AGPR here (as plain
      // reads the allocator moved accumulators into VGPRs and spilled)
      float v[16];
#pragma unroll
      for (int k = 0; k < 16; ++k) asm volatile("v_accvgpr_read_b32 %0, %1" : "=v"(v[k]) : "a"(acc[i][j][k]));
#pragma unroll
      for (int pp = 0; pp < 2; ++pp) {
        const uint32_t x0 = pack_bf16x2(v[8 * pp + 0], v[8 * pp + 1]), x1 = pack_bf16x2(v[8 * pp + 2], v[8 * pp + 3]);
        const uint32_t y0 = pack_bf16x2(v[8 * pp + 4], v[8 * pp + 5]), y1 = pack_bf16x2(v[8 * pp + 6], v[8 * pp + 7]);
        const auto s0 = __builtin_amdgcn_permlane32_swap(x0, y0, false, false);
        const auto s1 = __builtin_amdgcn_permlane32_swap(x1, y1, false, false);
        const int n = n0 + wn * 128 + i * 32 + pp * 16 + q2 * 8;
        if (t < p.T && n < p.N) *reinterpret_cast<uint4*>(orow + n) = make_uint4(s0[0], s1[0], s0[1], s1[1]);
      }
      // one accumulator block at a time: read out of the AGPRs as it is stored
      __builtin_amdgcn_sched_barrier(0);
    }
  }
}

}  // namespace

// Fused wo_a dispatch (arguments validated by the caller: K % 128 == 0,
// K <= 4096, D % 128 == 0, R <= 64 and R % 16 == 0 (R in {16, 32, 64} for
// split halves), N % 16 == 0, T >= 1).
mx_status launch_woa_fused(const void* x, const int64_t* positions, const void* cos, const void* sin,
                           int64_t max_pos, int64_t T, int32_t H, int32_t D, int32_t rope_dim, int32_t style,
                           const uint8_t* w, const uint8_t* w_scale, void* out, int32_t G, int32_t N,
                           hipStream_t stream) {
  FusedArgs p;
  p.x = static_cast<const uint16_t*>(x);
  p.pos = positions;
  p.cos = static_cast<const uint16_t*>(cos);
  p.sin = static_cast<const uint16_t*>(sin);
  p.max_pos = max_pos;
  p.w = w;
  p.sw = w_scale;
  p.out = static_cast<uint16_t*>(out);
  p.T = static_cast<int>(T);
  p.G = G;
  p.N = N;
  p.K = static_cast<int>(static_cast<int64_t>(H) * D / G);
  p.D = D;
  p.R = rope_dim;
  const bool neox = style == MX_ROPE_NEOX && rope_dim > 0;
  p.cd = neox ? rope_dim / 16 : 8;
  p.tiles_t = static_cast<int>((T + kTile - 1) / kTile);
  p.tiles_n = (N + kTile - 1) / kTile;
  p.total_tiles = p.tiles_t * p.tiles_n * G;
  p.per_xcd = (p.total_tiles + 7) / 8;
  const int grid = p.per_xcd * 8;
  constexpr int nw = 8;   // two waves per SIMD (4 waves of 128 x 128: about 12% slower)
  if (rope_dim == 0)
    woa_fused_kernel<nw, false, false><<<grid, 64 * nw, 0, stream>>>(p);
  else if (neox)
    woa_fused_kernel<nw, true, true><<<grid, 64 * nw, 0, stream>>>(p);
  else
    woa_fused_kernel<nw, true, false><<<grid, 64 * nw, 0, stream>>>(p);
  return launch_status("mx_wo_a_fused");
}

}  // namespace mx
