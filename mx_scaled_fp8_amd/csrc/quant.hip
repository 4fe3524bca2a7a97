// Fused inverse RoPE + per-token group E8M0 FP8 quantisation (gfx950).
//
// "[ROCm][DSV4][Perf] Use FP8 WO_A output projection", Summary item 1: the
// attention output is inverse-rotated and quantised per token to FP8 with one
// E8M0 scale per group of 128 consecutive elements, in one pass.  The FP8 byte
// flavour (OCP, or FNUZ capped at 224) follows "[ROCm][DSv4] Functional fixes
// for DeepSeek V4 on MI300X/MI325X", Purpose.
//
// Design (HBM-bound pass, 3 + 1/128 bytes per element):
//  * every lane owns 8 consecutive BF16 (one 16-byte load, one 8-byte store,
//    both non-temporal: each byte is touched once);
//    a group of 128 is 16 consecutive lanes = one DPP row, so its amax is four
//    row rotations of a packed-u16 max over the BF16 magnitudes, no LDS;
//  * the scale exponent is integer arithmetic on the BF16 bits of the amax;
//  * codes come from v_cvt_scalef32_pk_fp8_bf16, which converts two BF16
//    divided by an E8M0 scale to OCP e4m3 with round-to-nearest-even (checked
//    against the oracle on every BF16 pattern and scale 2^-127 .. 2^120); the
//    scale operand is built from its bits, byte << 23, so 2^-127 is exact;
//  * the rotation is fp32 with separately rounded products and sums (this
//    file is built with -ffp-contract=off), rounded to BF16 with
//    v_cvt_pk_bf16_f32 (nearest even) before the amax.
#include "common.hpp"

namespace mx {

namespace {

typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
typedef short v2s __attribute__((ext_vector_type(2)));
typedef unsigned short v2u16 __attribute__((ext_vector_type(2)));
typedef unsigned v4u_t __attribute__((ext_vector_type(4)));
typedef unsigned v2u_t __attribute__((ext_vector_type(2)));

constexpr int kThreads = 256;
// chunks of 8 elements per lane: 2 for large inputs (8192-token chunk: 252
// against 260 us with 4 and 274 with 8 per lane; 1 took 334); 1 when 2 would
// leave the chip with few workgroups (a decode batch, a linear's x)
constexpr int kUnrollLarge = 2, kUnrollSmall = 1;

struct QuantArgs {
  const uint4* x;             // [T, L] BF16 as 16-byte chunks
  const int64_t* pos;         // [T]
  const uint16_t* cos;        // [max_pos, R/2]
  const uint16_t* sin;
  int64_t max_pos;
  uint32_t total_chunks;      // T * L / 8 (this launch)
  DivU32 row_div;             // chunks per row = L / 8
  DivU32 head_div;            // chunks per head = D / 8
  int32_t row_shift;          // log2(L / 8) when a power of two, else -1
  int32_t head_shift;         // log2(D / 8) when a power of two, else -1
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

__device__ __forceinline__ uint32_t div_or_shift(uint32_t n, DivU32 d, int shift) {
  return shift >= 0 ? (n >> shift) : div_u32(n, d);
}

// Largest BF16 magnitude pattern of the 8 values in v (packed u16 max).
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

// (x, y) -> (x*c + y*s, y*c - x*s), every operation rounded to fp32.
__device__ __forceinline__ void inv_rotate(float x, float y, float c, float s, float& xr, float& yr) {
  const float xc = x * c, ys = y * s, yc = y * c, xs = x * s;
  xr = xc + ys;
  yr = yc - xs;
}

// Rotates the chunk `v` (8 BF16) in place; `j` is its dim offset inside the
// rotated slice of a head, `c` its chunk index, `p` the token position.
template <int STYLE>
__device__ __forceinline__ void rope_chunk(const QuantArgs& a, uint32_t c, uint32_t j, int64_t p, uint4& v) {
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
      w[k] = pk_bf16(xr, yr);
    }
  } else {
    // split halves: this chunk holds one component of pairs i0..i0+7, the
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
        w[k] = pk_bf16(r0x, r1x);
      } else {
        inv_rotate(oth0, own0, c0, s0, r0x, r0y);
        inv_rotate(oth1, own1, c1, s1, r1x, r1y);
        w[k] = pk_bf16(r0y, r1y);
      }
    }
  }
  v = make_uint4(w[0], w[1], w[2], w[3]);
}

// OCP codes of the 8 BF16 values of v divided by 2^e: `sbits` is the E8M0
// byte of 2^e placed in an FP32 exponent field (the converter reads the scale
// that way).
__device__ __forceinline__ uint2 encode8(const uint4 v, float sbits) {
  v2s lo = {0, 0}, hi = {0, 0};
  lo = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(lo, __builtin_bit_cast(v2bf, v.x), sbits, false);
  lo = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(lo, __builtin_bit_cast(v2bf, v.y), sbits, true);
  hi = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(hi, __builtin_bit_cast(v2bf, v.z), sbits, false);
  hi = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(hi, __builtin_bit_cast(v2bf, v.w), sbits, true);
  return make_uint2(__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi));
}

// Same codes through an exact FP32 rescale, for the one case the E8M0 scale
// operand cannot express (FNUZ with e = -127 needs a divisor of 2^-128).
__device__ __forceinline__ uint2 encode8_ldexp(const uint4 v, int sh) {
  int lo = 0, hi = 0;
  lo = cvt_fp8x2<false>(ldexpf(bf16_lo(v.x), sh), ldexpf(bf16_hi(v.x), sh), lo);
  lo = cvt_fp8x2<true>(ldexpf(bf16_lo(v.y), sh), ldexpf(bf16_hi(v.y), sh), lo);
  hi = cvt_fp8x2<false>(ldexpf(bf16_lo(v.z), sh), ldexpf(bf16_hi(v.z), sh), hi);
  hi = cvt_fp8x2<true>(ldexpf(bf16_lo(v.w), sh), ldexpf(bf16_hi(v.w), sh), hi);
  return make_uint2(static_cast<uint32_t>(lo), static_cast<uint32_t>(hi));
}

// Lane mapping: a wave is 4 DPP rows of 16 lanes; row r of wave w walks one
// segment of 64 consecutive chunks (4 groups of 128), chunk u*16 + lane%16 at
// unroll step u.  With 512-wide heads a segment is one head, so all its
// rotated chunks (the last 8) fall in step u = 3 and the rotation code runs
// in one step of four.
template <int GROUP, int FMT, int STYLE, bool ROPE, int U>
__global__ __launch_bounds__(kThreads) void quant_kernel(QuantArgs a) {
  constexpr int kLanesPerGroup = GROUP / 8;
  constexpr int EM = FMT == MX_FP8_E4M3_OCP ? 8 : 7;
  const uint32_t seg = blockIdx.x * (kThreads / 16) + (threadIdx.x >> 4);
  const uint32_t base = seg * (16 * U) + (threadIdx.x & 15);
  uint4 v[U];
  uint32_t cidx[U];
  // issue all loads first; out-of-range chunks re-read the last valid chunk so
  // that every lane takes part in the group reductions (a group is either all
  // in range or all out)
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const uint32_t c = base + u * 16;
    cidx[u] = c < a.total_chunks ? c : a.total_chunks - 1;
    // the input is read once and the codes written once: non-temporal
    // accesses (measured: 5.7 -> 6.2 TB/s on the 8192-token chunk)
    const v4u_t t = __builtin_nontemporal_load(reinterpret_cast<const v4u_t*>(a.x) + cidx[u]);
    v[u] = make_uint4(t[0], t[1], t[2], t[3]);
  }
  uint32_t row = 0, cin0 = 0;
  int64_t p = 0;
  bool ok = true;
  if constexpr (ROPE) {
    row = div_or_shift(cidx[0], a.row_div, a.row_shift);
    cin0 = cidx[0] - row * a.row_div.d;
    p = a.pos[row];
    ok = p >= 0 && p < a.max_pos;
  }
  uint32_t sword = 0;                   // group 128: the scale bytes of this row's U groups
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const uint32_t c = cidx[u];
    if constexpr (ROPE) {
      uint32_t cin = cin0 + u * 16;
      if (a.row_shift < 0 || cin >= a.row_div.d || c != cidx[0] + u * 16) {
        // the segment crosses a row (rows not a multiple of 512 elements) or
        // this chunk was clamped: locate it from scratch
        const uint32_t r = div_or_shift(c, a.row_div, a.row_shift);
        cin = c - r * a.row_div.d;
        if (r != row) {
          const int64_t pr = a.pos[r];
          ok = pr >= 0 && pr < a.max_pos;
          p = pr;
          row = r;
        }
      }
      const uint32_t hrow = div_or_shift(cin, a.head_div, a.head_shift);
      const uint32_t hchunk = cin - hrow * a.head_div.d;
      if (ok && hchunk >= a.rope_chunk0) rope_chunk<STYLE>(a, c, (hchunk - a.rope_chunk0) * 8, p, v[u]);
    }
    uint32_t m = amax_bits8(v[u]);
    if (!ok) m = 0x7F80u;                 // position outside the table: mark the group bad
    m = group_max<GROUP>(m);
    const bool finite = m < 0x7F80u;
    const int e = e8m0_exponent<EM>(finite ? m : 0);
    // FNUZ code of r*2^-e = OCP code of r*2^-(e-1)
    const int ecvt = FMT == MX_FP8_E4M3_OCP ? e : e - 1;
    uint2 codes;
    if (FMT == MX_FP8_E4M3_FNUZ && ecvt < -127)
      codes = encode8_ldexp(v[u], -ecvt);
    else
      codes = encode8(v[u], __uint_as_float(static_cast<uint32_t>(ecvt + 127) << 23));
    if constexpr (FMT == MX_FP8_E4M3_FNUZ) {
      codes.x = ocp_negzero_to_fnuz(codes.x);
      codes.y = ocp_negzero_to_fnuz(codes.y);
    }
    if (!finite) {
      const uint32_t nan4 = FMT == MX_FP8_E4M3_OCP ? 0x7F7F7F7Fu : 0x80808080u;
      codes = make_uint2(nan4, nan4);
    }
    const uint32_t craw = base + u * 16;
    const uint32_t sbyte = finite ? static_cast<uint32_t>(e + 127) : 0xFFu;
    if constexpr (GROUP == 128) sword |= sbyte << (8 * u);
    if (craw < a.total_chunks) {
      const v2u_t cw = {codes.x, codes.y};
      __builtin_nontemporal_store(cw, reinterpret_cast<v2u_t*>(a.q) + craw);
      if (GROUP != 128 && (threadIdx.x & (kLanesPerGroup - 1)) == 0)
        a.scale[craw / kLanesPerGroup] = static_cast<uint8_t>(sbyte);
    }
  }
  if constexpr (GROUP == 128) {
    // a row of 16 lanes quantised the U consecutive groups of its segment:
    // with U = 2 their scale bytes leave as one 2-byte store
    if ((threadIdx.x & 15) == 0) {
      uint8_t* dst = a.scale + base / 16;
      if (U == 2 && base + 16 < a.total_chunks && (reinterpret_cast<uintptr_t>(dst) & 1) == 0) {
        *reinterpret_cast<uint16_t*>(dst) = static_cast<uint16_t>(sword);
      } else {
#pragma unroll
        for (int u = 0; u < U; ++u)
          if (base + u * 16 < a.total_chunks) dst[u] = static_cast<uint8_t>(sword >> (8 * u));
      }
    }
  }
}

// ---------------------------------------------------------------- BF16 arm
//
// Inverse RoPE to BF16 with no quantisation: the first half of the BF16 wo_a
// path ("[ROCm][DSV4][Perf] Use FP8 WO_A output projection", Summary and
// Related work: an inverse RoPE followed by a BF16 grouped einsum, kept as
// the fallback).  Same rotation arithmetic as the quantiser.  The unit of
// work is 8 rotated pairs = 16 BF16 held in two 16-byte chunks (interleaved:
// two consecutive chunks; split halves: a chunk of first components and the
// chunk of their partners rope_dim/2 dims on), so a lane owns both members
// of each of its pairs and the pass can run in place.
//
//  * in place (out == x): one lane per unit; only the rotated slice of each
//    head is read and written (rope_dim/D of the tensor);
//  * out of place: one lane per 8-element chunk of the whole tensor; chunks
//    outside the rotated slice are copied, the first chunk of a unit
//    rotates the unit, the second is left to it.
// A token whose position is outside [0, max_pos) gets BF16 NaN (0x7FC0) in
// its rotated dims; the other dims pass through.

struct RopeArgs {
  const uint4* x;             // [T, L] BF16 as 16-byte chunks
  uint4* out;                 // [T, L]
  const int64_t* pos;         // [T]
  const uint16_t* cos;        // [max_pos, R/2]
  const uint16_t* sin;
  int64_t max_pos;
  uint32_t total;             // units (in place) or chunks (out of place) of this launch
  DivU32 row_div;             // units per row (H * R/16) or chunks per row (L/8)
  DivU32 head_div;            // units per head (R/16) or chunks per head (D/8)
  uint32_t head_chunks;       // D / 8
  uint32_t row_chunks;        // L / 8
  uint32_t rope_chunk0;       // (D - R) / 8
  uint32_t half_pairs;        // R / 2
};

// Rotates unit u of head slice starting at chunk `c0` (the head's first
// rotated chunk) of row `row`, reading from x and writing to out.
template <int STYLE>
__device__ __forceinline__ void rope_unit_bf16(const RopeArgs& a, uint32_t row, uint32_t c0, uint32_t u) {
  const uint32_t ca = c0 + (STYLE == MX_ROPE_INTERLEAVED ? 2 * u : u);
  const uint32_t cb = ca + (STYLE == MX_ROPE_INTERLEAVED ? 1 : a.half_pairs / 8);
  const uint4 va = a.x[ca], vb = a.x[cb];
  const int64_t p = a.pos[row];
  if (p < 0 || p >= a.max_pos) {
    const uint4 nan = make_uint4(0x7FC07FC0u, 0x7FC07FC0u, 0x7FC07FC0u, 0x7FC07FC0u);
    a.out[ca] = nan;
    a.out[cb] = nan;
    return;
  }
  const uint4 cc = *reinterpret_cast<const uint4*>(a.cos + p * a.half_pairs + 8 * u);
  const uint4 ss = *reinterpret_cast<const uint4*>(a.sin + p * a.half_pairs + 8 * u);
  const uint32_t cw[4] = {cc.x, cc.y, cc.z, cc.w};
  const uint32_t sw[4] = {ss.x, ss.y, ss.z, ss.w};
  uint32_t wa[4] = {va.x, va.y, va.z, va.w};
  uint32_t wb[4] = {vb.x, vb.y, vb.z, vb.w};
  if constexpr (STYLE == MX_ROPE_INTERLEAVED) {
    // dword k of the unit is pair k: (x, y) = (lo, hi)
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      float xr, yr;
      inv_rotate(bf16_lo(wa[k]), bf16_hi(wa[k]), bf16_lo(k & 1 ? cw[k >> 1] >> 16 : cw[k >> 1]),
                 bf16_lo(k & 1 ? sw[k >> 1] >> 16 : sw[k >> 1]), xr, yr);
      wa[k] = pk_bf16(xr, yr);
      inv_rotate(bf16_lo(wb[k]), bf16_hi(wb[k]), bf16_lo(k & 1 ? cw[2 + (k >> 1)] >> 16 : cw[2 + (k >> 1)]),
                 bf16_lo(k & 1 ? sw[2 + (k >> 1)] >> 16 : sw[2 + (k >> 1)]), xr, yr);
      wb[k] = pk_bf16(xr, yr);
    }
  } else {
    // element e of chunk a is the first component of pair e, of chunk b the second
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      float x0, y0, x1, y1;
      inv_rotate(bf16_lo(wa[k]), bf16_lo(wb[k]), bf16_lo(cw[k]), bf16_lo(sw[k]), x0, y0);
      inv_rotate(bf16_hi(wa[k]), bf16_hi(wb[k]), bf16_hi(cw[k]), bf16_hi(sw[k]), x1, y1);
      wa[k] = pk_bf16(x0, x1);
      wb[k] = pk_bf16(y0, y1);
    }
  }
  a.out[ca] = make_uint4(wa[0], wa[1], wa[2], wa[3]);
  a.out[cb] = make_uint4(wb[0], wb[1], wb[2], wb[3]);
}

template <int STYLE, bool COPY>
__global__ __launch_bounds__(kThreads) void rope_bf16_kernel(RopeArgs a) {
  const uint32_t i = blockIdx.x * kThreads + threadIdx.x;
  if (i >= a.total) return;
  const uint32_t row = div_u32(i, a.row_div);
  const uint32_t rem = i - row * a.row_div.d;
  const uint32_t head = div_u32(rem, a.head_div);
  const uint32_t hin = rem - head * a.head_div.d;
  const uint32_t c0 = row * a.row_chunks + head * a.head_chunks + a.rope_chunk0;
  if constexpr (!COPY) {
    rope_unit_bf16<STYLE>(a, row, c0, hin);
  } else {
    if (hin < a.rope_chunk0) {
      a.out[i] = a.x[i];
      return;
    }
    const uint32_t s = hin - a.rope_chunk0;      // chunk inside the rotated slice
    if (STYLE == MX_ROPE_INTERLEAVED) {
      if ((s & 1) == 0) rope_unit_bf16<STYLE>(a, row, c0, s >> 1);
    } else {
      if (s < a.half_pairs / 8) rope_unit_bf16<STYLE>(a, row, c0, s);
    }
  }
}

template <int GROUP, int FMT, int U>
void launch_style_u(const QuantArgs& a, bool rope, int style, hipStream_t s) {
  const uint32_t blocks = static_cast<uint32_t>((a.total_chunks + kThreads * U - 1) / (kThreads * U));
  if (!rope)
    quant_kernel<GROUP, FMT, MX_ROPE_INTERLEAVED, false, U><<<blocks, kThreads, 0, s>>>(a);
  else if (style == MX_ROPE_INTERLEAVED)
    quant_kernel<GROUP, FMT, MX_ROPE_INTERLEAVED, true, U><<<blocks, kThreads, 0, s>>>(a);
  else
    quant_kernel<GROUP, FMT, MX_ROPE_NEOX, true, U><<<blocks, kThreads, 0, s>>>(a);
}

constexpr uint32_t kSmallBlocks = 1024;
template <int GROUP, int FMT>
void launch_style(const QuantArgs& a, bool rope, int style, hipStream_t s) {
  // fewer than kSmallBlocks workgroups at kUnrollLarge chunks per lane: 1 chunk per lane
  if ((a.total_chunks + kThreads * kUnrollLarge - 1) / (kThreads * kUnrollLarge) < kSmallBlocks)
    launch_style_u<GROUP, FMT, kUnrollSmall>(a, rope, style, s);
  else
    launch_style_u<GROUP, FMT, kUnrollLarge>(a, rope, style, s);
}

int log2_if_pow2(uint32_t v) {
  if (v == 0 || (v & (v - 1)) != 0) return -1;
  int s = 0;
  while ((1u << s) != v) ++s;
  return s;
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
    a.row_shift = log2_if_pow2(static_cast<uint32_t>(chunks_per_row));
    a.head_shift = log2_if_pow2(static_cast<uint32_t>(D / 8));
    a.rope_chunk0 = static_cast<uint32_t>((D - rope_dim) / 8);
    a.half_pairs = static_cast<uint32_t>(rope_dim / 2);
    a.q = reinterpret_cast<uint2*>(q + r0 * L);
    a.scale = scale + r0 * (L / group);
    const bool rope = rope_dim > 0;
    if (group == 128) {
      if (fmt == MX_FP8_E4M3_OCP) launch_style<128, MX_FP8_E4M3_OCP>(a, rope, style, stream);
      else launch_style<128, MX_FP8_E4M3_FNUZ>(a, rope, style, stream);
    } else {
      if (fmt == MX_FP8_E4M3_OCP) launch_style<32, MX_FP8_E4M3_OCP>(a, rope, style, stream);
      else launch_style<32, MX_FP8_E4M3_FNUZ>(a, rope, style, stream);
    }
    const mx_status st = launch_status("mx_inv_rope_group_quant");
    if (st != MX_OK) return st;
  }
  return MX_OK;
}


// Inverse RoPE to BF16 over rows [0, T) (arguments validated by the caller;
// out == x runs in place).
mx_status launch_rope_bf16(const void* x, const int64_t* positions, const void* cos, const void* sin,
                           int64_t max_pos, int64_t T, int32_t H, int32_t D, int32_t rope_dim, int32_t style,
                           void* out, hipStream_t stream) {
  const int64_t L = static_cast<int64_t>(H) * D;
  const bool in_place = out == x;
  if (rope_dim == 0 && in_place) return MX_OK;
  const int64_t per_row = in_place ? static_cast<int64_t>(H) * (rope_dim / 16) : L / 8;
  const int64_t max_rows = std::max<int64_t>(1, (int64_t(1) << 31) / std::max<int64_t>(L / 8, 1) - 1);
  for (int64_t r0 = 0; r0 < T; r0 += max_rows) {
    const int64_t rows = std::min(max_rows, T - r0);
    RopeArgs a;
    a.x = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(x) + r0 * L);
    a.out = reinterpret_cast<uint4*>(static_cast<uint16_t*>(out) + r0 * L);
    a.pos = positions ? positions + r0 : nullptr;
    a.cos = static_cast<const uint16_t*>(cos);
    a.sin = static_cast<const uint16_t*>(sin);
    a.max_pos = max_pos;
    a.total = static_cast<uint32_t>(rows * per_row);
    a.row_div = make_div(static_cast<uint32_t>(per_row));
    a.head_div = make_div(static_cast<uint32_t>(in_place ? rope_dim / 16 : D / 8));
    a.head_chunks = static_cast<uint32_t>(D / 8);
    a.row_chunks = static_cast<uint32_t>(L / 8);
    a.rope_chunk0 = static_cast<uint32_t>((D - rope_dim) / 8);
    a.half_pairs = static_cast<uint32_t>(rope_dim / 2);
    const uint32_t blocks = (a.total + kThreads - 1) / kThreads;
    if (rope_dim == 0) {
      // nothing rotates: every chunk is copied (no position is read)
      a.rope_chunk0 = a.head_chunks;
      rope_bf16_kernel<MX_ROPE_INTERLEAVED, true><<<blocks, kThreads, 0, stream>>>(a);
    } else if (style == MX_ROPE_INTERLEAVED) {
      if (in_place) rope_bf16_kernel<MX_ROPE_INTERLEAVED, false><<<blocks, kThreads, 0, stream>>>(a);
      else rope_bf16_kernel<MX_ROPE_INTERLEAVED, true><<<blocks, kThreads, 0, stream>>>(a);
    } else {
      if (in_place) rope_bf16_kernel<MX_ROPE_NEOX, false><<<blocks, kThreads, 0, stream>>>(a);
      else rope_bf16_kernel<MX_ROPE_NEOX, true><<<blocks, kThreads, 0, stream>>>(a);
    }
    const mx_status st = launch_status("mx_inv_rope_bf16");
    if (st != MX_OK) return st;
  }
  return MX_OK;
}

}  // namespace mx
