// Fused inverse RoPE + per-token group E8M0 FP8 quantisation (gfx950).
//
// "[ROCm][DSV4][Perf] Use FP8 WO_A output projection", Summary item 1: the
// attention output is inverse-rotated and quantised per token to FP8 with one
// E8M0 scale per group of 128 consecutive elements, in one pass.  The FP8 byte
// flavour (OCP, or FNUZ capped at 224) follows "[ROCm][DSv4] Functional fixes
// for DeepSeek V4 on MI300X/MI325X", Purpose.
//
// Memory-bound design: every lane owns 8 consecutive BF16 (one 16-byte load);
// a quantisation group of 128 is 16 consecutive lanes = one DPP row, so its
// amax is reduced with four row rotations and no LDS; the scale exponent is
// computed with integer ops on the BF16 bits of the amax; the codes come from
// the hardware OCP converter (round to nearest even) on r * 2^-e, which is
// exact because |r * 2^-e| <= 448; each lane stores 8 packed codes (8 bytes).
// The rotation is fp32 with separately rounded products and sums (this file is
// built with -ffp-contract=off), then rounded to BF16 before the amax.
#include "common.hpp"

namespace mx {

namespace {

constexpr int kThreads = 256;
constexpr int kUnroll = 4;                       // chunks of 8 elements per lane
constexpr int kChunksPerBlock = kThreads * kUnroll;

struct QuantArgs {
  const uint4* x;             // [T, L] BF16 as 16-byte chunks
  const int64_t* pos;         // [T]
  const uint16_t* cos;        // [max_pos, R/2]
  const uint16_t* sin;
  int64_t max_pos;
  uint32_t total_chunks;      // T * L / 8 (this launch)
  DivU32 row_div;             // chunks per row = L / 8
  DivU32 head_div;            // chunks per head = D / 8
  uint32_t rope_chunk0;       // (D - R) / 8: first rotated chunk of a head
  uint32_t half_pairs;        // R / 2
  uint2* q;                   // [T, L] codes as 8-byte chunks
  uint8_t* scale;             // [T, L / group]
};

template <int CTRL>
__device__ __forceinline__ uint32_t dpp(uint32_t v) {
  return static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), CTRL, 0xF, 0xF, false));
}

// max over the lanes of one group: 16 lanes (a DPP row) for group 128, 4 lanes
// (a quad) for group 32.
template <int GROUP>
__device__ __forceinline__ uint32_t group_max(uint32_t m) {
  if constexpr (GROUP == 128) {
    m = max(m, dpp<0x128>(m));   // row_ror:8
    m = max(m, dpp<0x124>(m));   // row_ror:4
    m = max(m, dpp<0x122>(m));   // row_ror:2
    m = max(m, dpp<0x121>(m));   // row_ror:1
  } else {
    m = max(m, dpp<0xB1>(m));    // quad_perm [1,0,3,2]
    m = max(m, dpp<0x4E>(m));    // quad_perm [2,3,0,1]
  }
  return m;
}

// (x, y) -> (x*c + y*s, y*c - x*s), every operation rounded to fp32.
__device__ __forceinline__ void inv_rotate(float x, float y, float c, float s, float& xr, float& yr) {
  const float xc = x * c, ys = y * s, yc = y * c, xs = x * s;
  xr = xc + ys;
  yr = yc - xs;
}

__device__ __forceinline__ uint32_t amax_bits8(const uint4 v) {
  const uint32_t a = v.x & 0x7FFF7FFFu, b = v.y & 0x7FFF7FFFu, c = v.z & 0x7FFF7FFFu, d = v.w & 0x7FFF7FFFu;
  const uint32_t m0 = max(max(a & 0xFFFFu, a >> 16), max(b & 0xFFFFu, b >> 16));
  const uint32_t m1 = max(max(c & 0xFFFFu, c >> 16), max(d & 0xFFFFu, d >> 16));
  return max(m0, m1);
}

// Rotates the chunk `v` (8 BF16) in place if it lies in a rotated slice.
// Returns false if the token's position is out of range.
template <int STYLE>
__device__ __forceinline__ bool rope_chunk(const QuantArgs& a, uint32_t c, uint32_t row, uint32_t hchunk,
                                           int64_t p, uint4& v) {
  if (hchunk < a.rope_chunk0) return true;
  if (p < 0 || p >= a.max_pos) return false;
  const uint32_t j = (hchunk - a.rope_chunk0) * 8;   // dim offset inside the rotated slice
  const uint16_t* crow = a.cos + p * a.half_pairs;
  const uint16_t* srow = a.sin + p * a.half_pairs;
  uint32_t w[4] = {v.x, v.y, v.z, v.w};
  if constexpr (STYLE == MX_ROPE_INTERLEAVED) {
    // the 8 elements are pairs i0..i0+3, each dword one (x, y) pair
    const uint32_t i0 = j / 2;
    const uint2 cc = *reinterpret_cast<const uint2*>(crow + i0);
    const uint2 ss = *reinterpret_cast<const uint2*>(srow + i0);
    const uint32_t cw[4] = {cc.x, cc.x >> 16, cc.y, cc.y >> 16};
    const uint32_t sw[4] = {ss.x, ss.x >> 16, ss.y, ss.y >> 16};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      float xr, yr;
      inv_rotate(bf16_lo(w[k]), bf16_hi(w[k]), bf16_lo(cw[k]), bf16_lo(sw[k]), xr, yr);
      w[k] = pack_bf16x2(xr, yr);
    }
  } else {
    // split halves: this chunk holds one component of pairs i..i+7, the
    // partner chunk half_pairs/8 chunks away holds the other
    const bool first = j < a.half_pairs;
    const uint32_t i0 = first ? j : j - a.half_pairs;
    const uint32_t partner = first ? c + a.half_pairs / 8 : c - a.half_pairs / 8;
    const uint4 pv = a.x[partner];
    const uint4 cc = *reinterpret_cast<const uint4*>(crow + i0);
    const uint4 ss = *reinterpret_cast<const uint4*>(srow + i0);
    const uint32_t pw[4] = {pv.x, pv.y, pv.z, pv.w};
    const uint32_t cw[4] = {cc.x, cc.y, cc.z, cc.w};
    const uint32_t sw[4] = {ss.x, ss.y, ss.z, ss.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      float r0x, r0y, r1x, r1y;
      const float own0 = bf16_lo(w[k]), own1 = bf16_hi(w[k]);
      const float oth0 = bf16_lo(pw[k]), oth1 = bf16_hi(pw[k]);
      const float c0 = bf16_lo(cw[k]), c1 = bf16_hi(cw[k]);
      const float s0 = bf16_lo(sw[k]), s1 = bf16_hi(sw[k]);
      if (first) {
        inv_rotate(own0, oth0, c0, s0, r0x, r0y);
        inv_rotate(own1, oth1, c1, s1, r1x, r1y);
        w[k] = pack_bf16x2(r0x, r1x);
      } else {
        inv_rotate(oth0, own0, c0, s0, r0x, r0y);
        inv_rotate(oth1, own1, c1, s1, r1x, r1y);
        w[k] = pack_bf16x2(r0y, r1y);
      }
    }
  }
  v = make_uint4(w[0], w[1], w[2], w[3]);
  return true;
}

// Codes of 8 BF16 values scaled by 2^sh (exact), OCP rounding.
__device__ __forceinline__ uint2 encode8(const uint4 v, int sh) {
  int lo = 0, hi = 0;
  lo = cvt_fp8x2<false>(ldexpf(bf16_lo(v.x), sh), ldexpf(bf16_hi(v.x), sh), lo);
  lo = cvt_fp8x2<true>(ldexpf(bf16_lo(v.y), sh), ldexpf(bf16_hi(v.y), sh), lo);
  hi = cvt_fp8x2<false>(ldexpf(bf16_lo(v.z), sh), ldexpf(bf16_hi(v.z), sh), hi);
  hi = cvt_fp8x2<true>(ldexpf(bf16_lo(v.w), sh), ldexpf(bf16_hi(v.w), sh), hi);
  return make_uint2(static_cast<uint32_t>(lo), static_cast<uint32_t>(hi));
}

template <int GROUP, int FMT, int STYLE, bool ROPE>
__global__ __launch_bounds__(kThreads) void quant_kernel(QuantArgs a) {
  constexpr int kLanesPerGroup = GROUP / 8;
  constexpr int EM = FMT == MX_FP8_E4M3_OCP ? 8 : 7;
  const uint32_t base = blockIdx.x * kChunksPerBlock + threadIdx.x;
  uint4 v[kUnroll];
  uint32_t cidx[kUnroll];
  // issue all loads first; out-of-range chunks re-read the last valid chunk so
  // that every lane takes part in the group reductions
#pragma unroll
  for (int u = 0; u < kUnroll; ++u) {
    const uint32_t c = base + u * kThreads;
    cidx[u] = c < a.total_chunks ? c : a.total_chunks - 1;
    v[u] = a.x[cidx[u]];
  }
#pragma unroll
  for (int u = 0; u < kUnroll; ++u) {
    const uint32_t c = cidx[u];
    bool ok = true;
    if constexpr (ROPE) {
      const uint32_t row = div_u32(c, a.row_div);
      const uint32_t cin = c - row * a.row_div.d;
      const uint32_t hrow = div_u32(cin, a.head_div);
      const uint32_t hchunk = cin - hrow * a.head_div.d;
      const int64_t p = a.pos[row];
      if (p < 0 || p >= a.max_pos) ok = false;
      else ok = rope_chunk<STYLE>(a, c, row, hchunk, p, v[u]);
    }
    uint32_t m = amax_bits8(v[u]);
    if (!ok) m = 0x7F80u;                 // mark the whole group bad
    m = group_max<GROUP>(m);
    const bool finite = m < 0x7F80u;
    const int e = e8m0_exponent<EM>(finite ? m : 0);
    // FNUZ code of r*2^-e = OCP code of r*2^-(e-1)
    const int sh = FMT == MX_FP8_E4M3_OCP ? -e : 1 - e;
    uint2 codes = encode8(v[u], sh);
    if constexpr (FMT == MX_FP8_E4M3_FNUZ) {
      codes.x = ocp_negzero_to_fnuz(codes.x);
      codes.y = ocp_negzero_to_fnuz(codes.y);
    }
    if (!finite) {
      const uint32_t nan4 = FMT == MX_FP8_E4M3_OCP ? 0x7F7F7F7Fu : 0x80808080u;
      codes = make_uint2(nan4, nan4);
    }
    const uint32_t craw = base + u * kThreads;
    if (craw < a.total_chunks) {
      a.q[craw] = codes;
      if ((threadIdx.x & (kLanesPerGroup - 1)) == 0)
        a.scale[craw / kLanesPerGroup] = finite ? static_cast<uint8_t>(e + 127) : uint8_t(0xFF);
    }
  }
}

template <int GROUP, int FMT>
void launch_style(const QuantArgs& a, bool rope, int style, uint32_t blocks, hipStream_t s) {
  if (!rope)
    quant_kernel<GROUP, FMT, MX_ROPE_INTERLEAVED, false><<<blocks, kThreads, 0, s>>>(a);
  else if (style == MX_ROPE_INTERLEAVED)
    quant_kernel<GROUP, FMT, MX_ROPE_INTERLEAVED, true><<<blocks, kThreads, 0, s>>>(a);
  else
    quant_kernel<GROUP, FMT, MX_ROPE_NEOX, true><<<blocks, kThreads, 0, s>>>(a);
}

}  // namespace

// Launches the quantiser over rows [0, T) of x in slices whose chunk count
// fits 32-bit indexing.  Arguments were validated by the caller.
mx_status launch_quant(const void* x, const int64_t* positions, const void* cos, const void* sin,
                       int64_t max_pos, int64_t T, int32_t H, int32_t D, int32_t rope_dim, int32_t style,
                       int32_t group, int32_t fmt, uint8_t* q, uint8_t* scale, hipStream_t stream) {
  const int64_t L = static_cast<int64_t>(H) * D;
  const int64_t chunks_per_row = L / 8;
  // rows per launch: keep the chunk count below 2^31
  const int64_t max_rows = std::max<int64_t>(1, (int64_t(1) << 31) / chunks_per_row - 1);
  for (int64_t r0 = 0; r0 < T; r0 += max_rows) {
    const int64_t rows = std::min(max_rows, T - r0);
    QuantArgs a;
    a.x = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(x) + r0 * L);
    a.pos = positions ? positions + r0 : nullptr;
    a.cos = static_cast<const uint16_t*>(cos);
    a.sin = static_cast<const uint16_t*>(sin);
    a.max_pos = max_pos;
    a.total_chunks = static_cast<uint32_t>(rows * chunks_per_row);
    a.row_div = make_div(static_cast<uint32_t>(chunks_per_row));
    a.head_div = make_div(static_cast<uint32_t>(D / 8));
    a.rope_chunk0 = static_cast<uint32_t>((D - rope_dim) / 8);
    a.half_pairs = static_cast<uint32_t>(rope_dim / 2);
    a.q = reinterpret_cast<uint2*>(q + r0 * L);
    a.scale = scale + r0 * (L / group);
    const uint32_t blocks = static_cast<uint32_t>((a.total_chunks + kChunksPerBlock - 1) / kChunksPerBlock);
    const bool rope = rope_dim > 0;
    if (group == 128) {
      if (fmt == MX_FP8_E4M3_OCP) launch_style<128, MX_FP8_E4M3_OCP>(a, rope, style, blocks, stream);
      else launch_style<128, MX_FP8_E4M3_FNUZ>(a, rope, style, blocks, stream);
    } else {
      if (fmt == MX_FP8_E4M3_OCP) launch_style<32, MX_FP8_E4M3_OCP>(a, rope, style, blocks, stream);
      else launch_style<32, MX_FP8_E4M3_FNUZ>(a, rope, style, blocks, stream);
    }
    const mx_status st = launch_status("mx_inv_rope_group_quant");
    if (st != MX_OK) return st;
  }
  return MX_OK;
}

}  // namespace mx
