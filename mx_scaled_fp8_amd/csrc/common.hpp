// Internal helpers shared by the HIP sources of libmxfp8 (not part of the ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mxfp8.h"

namespace mx {

// ------------------------------------------------------------------ host side

// Records a printf-style message as the calling thread's last error and
// returns `st`.
mx_status fail(mx_status st, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
// Clears the calling thread's last error.
void clear_error();
// True when mx_set_dry_run(1) is in force.
bool dry_run();
// Checks that the current HIP device is a gfx950 (cached per device).
mx_status require_gfx950();
// Compute units of the current device (known once require_gfx950() passed; 0 if not).
int device_cu_count();
// Maps a launch error to MX_ERR_HIP with a message naming `what`.
mx_status launch_status(const char* what);

enum Counter {
  C_QUANT = 0,
  C_BMM_LARGE,
  C_BMM_SMALL,
  C_DEQUANT,
  C_LINEAR_BF16,
  C_LINEAR_FP8,
  C_LINEAR_PERCALL,
  C_E8M0_DEVICE,
  C_E4M3_DEVICE,
  C_ROPE_BF16,
  C_BMM_BF16_LARGE,
  C_BMM_BF16_SMALL,
  C_EXPAND_SCALES,
  C_WOA_FUSED,
};
void count(Counter c);

inline bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

// Unsigned 32-bit division by a run-time constant d >= 1 through a 64-bit
// multiply-high: q = mulhi64(n, ceil(2^64 / d)) is exact for every n < 2^32
// (the rounding error of the reciprocal times n stays below 1/d).  d == 1 is
// special-cased because 2^64 does not fit.
struct DivU32 {
  uint64_t magic;
  uint32_t d;
};
inline DivU32 make_div(uint32_t d) {
  DivU32 r;
  r.d = d;
  if (d <= 1) {
    r.magic = 0;
  } else {
    // ceil(2^64 / d) = floor((2^64 - 1) / d) + 1 for d not dividing 2^64 - 1 ... and
    // in general floor((2^64-1)/d) + 1 >= 2^64/d with error < 1.
    r.magic = ~uint64_t(0) / d + 1;
  }
  return r;
}

// ---------------------------------------------------------------- device side

// s_waitcnt immediates (gfx9 encoding: vmcnt bits 3:0 and 15:14, expcnt
// bits 6:4, lgkmcnt bits 11:8).  wait_vm(n): at most n vector-memory
// instructions of this wave outstanding (they complete in issue order: loads,
// LDS-DMA and stores alike) and no LDS/scalar-memory instruction; expcnt is
// not waited on.  kWaitLgkmOnly: LDS/scalar memory only.
constexpr int wait_vm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4); }
constexpr int kWaitLgkmOnly = wait_vm(63) | 0xF;
// at most n vector-memory instructions outstanding; LDS and scalar memory not waited on
constexpr int wait_vm_only(int n) { return wait_vm(n) | 0x0F00; }
static_assert(wait_vm(0) == 0x0070 && wait_vm(16) == 0x4070 && wait_vm(18) == 0x4072 && wait_vm(24) == 0x4078 &&
                  wait_vm(32) == 0x8070 && kWaitLgkmOnly == 0xC07F && wait_vm_only(8) == 0x0F78,
              "s_waitcnt encoding");

// Word 3 of a raw buffer resource (gfx9 layout): 32-bit data format, no
// swizzle, no thread-id offset.  With stride 0 a load reads base + vector
// offset + scalar offset, and offsets at or past num_records read zeros.
constexpr int kBufferFlags = 0x00020000;

__device__ __forceinline__ uint32_t div_u32(uint32_t n, DivU32 dv) {
  return dv.magic == 0 ? n : static_cast<uint32_t>(__umul64hi(static_cast<uint64_t>(n), dv.magic));
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Two floats -> packed BF16 (low = lo), round to nearest even, NaN stays NaN:
// v_cvt_pk_bf16_f32 (checked bit-exact against integer RNE on 2^20 random
// FP32 patterns).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef __bf16 v2bf_t __attribute__((ext_vector_type(2)));
  const v2bf_t r = {static_cast<__bf16>(lo), static_cast<__bf16>(hi)};
  return __builtin_bit_cast(uint32_t, r);
}

// Scale exponent of a group from the BF16 pattern of its amax (sign cleared):
// e = ceil(log2(amax / M)) with M = 1.75 * 2^EM (EM = 8 for 448, 7 for 224).
// Writing amax = m * 2^E with m in [1, 2): e = E - EM + (m > 1.75), because
// M * 2^(E-EM) = 1.75 * 2^E.  On BF16 bits m > 1.75 means mantissa field > 0x60.
// Clamped to [-127, 127]; 0 gives -127.  amax must be finite (< 0x7F80).
// Branch-free: a zero or subnormal amax (exponent field 0) has E <= -127, so
// its e is below -127 whatever its mantissa and the clamp gives -127 -- the
// same as the formula on the raw fields; and a finite amax (field <= 254)
// gives at most 254 - 127 - 7 + 1 = 121, so the upper clamp never acts.
template <int EM>
__device__ __forceinline__ int e8m0_exponent(uint32_t amax_bits) {
  const int e = static_cast<int>(amax_bits >> 7) - 127 - EM + ((amax_bits & 0x7F) > 0x60 ? 1 : 0);
  return max(e, -127);
}

// Two floats -> two OCP e4m3 codes (round to nearest even) packed into the low
// (HI = false) or high (HI = true) 16 bits of `old`.  Inputs must be within
// [-448, 448] or NaN.
template <bool HI>
__device__ __forceinline__ int cvt_fp8x2(float a, float b, int old) {
  return __builtin_amdgcn_cvt_pk_fp8_f32(a, b, old, HI);
}

// In each byte of `w`, turn 0x80 (OCP -0) into 0x00 (FNUZ has no -0).
__device__ __forceinline__ uint32_t ocp_negzero_to_fnuz(uint32_t w) {
  const uint32_t t = w ^ 0x80808080u;                              // 0x80 bytes -> 0
  const uint32_t nz = (((t & 0x7F7F7F7Fu) + 0x7F7F7F7Fu) | t) & 0x80808080u;  // high bit: byte != 0
  return w ^ (~nz & 0x80808080u);
}

}  // namespace mx
