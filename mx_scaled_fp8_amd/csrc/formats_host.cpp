// Host-side format conversions of libmxfp8: FP32 -> E8M0 (lossless powers of
// two), FP32 -> e4m3 (OCP / FNUZ), and the decoders.
//
// FP32 -> E8M0: "[ROCm][DSV4][Perf] Use FP8 WO_A output projection",
// Implementation (positive power-of-two FP32 scales become biased E8M0 bytes
// without loss).  The e4m3 flavours and their bounds (448 OCP, 224 FNUZ):
// "[ROCm][DSv4] Functional fixes for DeepSeek V4 on MI300X/MI325X", Purpose.
#include <cmath>
#include <cstdint>
#include <cstring>

#include "mxfp8.h"

namespace mx {
mx_status fail(mx_status st, const char* fmt, ...);
void clear_error();
}  // namespace mx

namespace {

uint32_t bits_of(float f) {
  uint32_t u;
  std::memcpy(&u, &f, 4);
  return u;
}

// Exactly 2^n with -127 <= n <= 127?  On the FP32 pattern: a normal power of
// two has a zero mantissa field and sign 0; the only subnormal in range is
// 2^-127 = 0x00400000.  Returns the E8M0 byte or -1.
int pow2_byte(float f) {
  const uint32_t u = bits_of(f);
  if (u == 0x00400000u) return 0;
  const uint32_t ef = (u >> 23) & 0xFFu;
  if ((u >> 31) != 0 || (u & 0x7FFFFFu) != 0 || ef == 0 || ef == 0xFFu) return -1;
  return static_cast<int>(ef);  // 2^(ef-127) -> byte (ef-127)+127
}

// OCP e4m3 code of v: round to nearest, ties to even, saturating at 448.
// |v| = r * 2^(Eb-3) with Eb = max(E, -6) the exponent of |v| (or of the
// smallest normal for subnormal results) and r the rounded 3-bit-mantissa
// significand in units of that quantum; the code is ((Eb + 6) << 3) + r, which
// also covers subnormals (Eb = -6, r in 0..8) and a round-up into the next
// binade (r = 16).
uint8_t e4m3_ocp(float v) {
  const uint32_t u = bits_of(v);
  const uint32_t sign = (u >> 31) << 7;
  if (std::isnan(v)) return 0x7F;
  const double av = std::fabs(static_cast<double>(v));
  if (av >= 448.0) return static_cast<uint8_t>(sign | 0x7E);
  int code;
  if (av == 0.0) {
    code = 0;
  } else {
    int e2;
    std::frexp(av, &e2);               // av = m * 2^e2, m in [0.5, 1)
    int eb = e2 - 1;                   // exponent of av
    if (eb < -6) eb = -6;
    const double q = std::ldexp(av, 3 - eb);   // exact
    const double r = std::nearbyint(q);        // default mode: nearest, ties to even
    code = ((eb + 6) << 3) + static_cast<int>(r);
  }
  return static_cast<uint8_t>(sign | static_cast<uint32_t>(code));
}

// FNUZ e4m3: the FNUZ grid is the OCP grid halved (bias 8 vs 7), and 224 is
// half of 448, so the FNUZ code of v is the OCP code of 2v -- except that FNUZ
// has no -0 (0x80 is its NaN).
uint8_t e4m3_fnuz(float v) {
  if (std::isnan(v)) return 0x80;
  const double d = 2.0 * static_cast<double>(v);
  const float twice = std::fabs(d) >= 448.0 ? (d < 0 ? -448.0f : 448.0f) : static_cast<float>(d);
  const uint8_t c = e4m3_ocp(twice);
  return c == 0x80 ? 0x00 : c;
}

float e4m3_value(uint8_t c, int fmt) {
  const int bias = fmt == MX_FP8_E4M3_OCP ? 7 : 8;
  if (fmt == MX_FP8_E4M3_OCP && (c & 0x7F) == 0x7F) return NAN;
  if (fmt == MX_FP8_E4M3_FNUZ && c == 0x80) return NAN;
  const int ef = (c >> 3) & 0xF, mf = c & 7;
  const double mag = ef == 0 ? std::ldexp(mf / 8.0, 1 - bias) : std::ldexp(1.0 + mf / 8.0, ef - bias);
  return static_cast<float>((c & 0x80) ? -mag : mag);
}

}  // namespace

extern "C" {

mx_status mx_f32_pow2_to_e8m0(const float* in, uint8_t* out, int64_t n) {
  if (n < 0 || (n > 0 && (!in || !out))) return mx::fail(MX_ERR_INVALID_ARG, "mx_f32_pow2_to_e8m0: bad pointer or size");
  int64_t bad = 0, first_bad = -1;
  for (int64_t i = 0; i < n; ++i) {
    const int b = pow2_byte(in[i]);
    if (b < 0) {
      out[i] = 0xFF;
      if (bad++ == 0) first_bad = i;
    } else {
      out[i] = static_cast<uint8_t>(b);
    }
  }
  if (bad)
    return mx::fail(MX_ERR_NOT_LOSSLESS, "mx_f32_pow2_to_e8m0: %lld of %lld values are not powers of two in "
                    "[2^-127, 2^127] (first at index %lld)", (long long)bad, (long long)n, (long long)first_bad);
  mx::clear_error();
  return MX_OK;
}

mx_status mx_f32_to_e4m3_ocp(const float* in, uint8_t* out, int64_t n) {
  if (n < 0 || (n > 0 && (!in || !out))) return mx::fail(MX_ERR_INVALID_ARG, "mx_f32_to_e4m3_ocp: bad pointer or size");
  for (int64_t i = 0; i < n; ++i) out[i] = e4m3_ocp(in[i]);
  mx::clear_error();
  return MX_OK;
}

mx_status mx_f32_to_e4m3_fnuz(const float* in, uint8_t* out, int64_t n) {
  if (n < 0 || (n > 0 && (!in || !out))) return mx::fail(MX_ERR_INVALID_ARG, "mx_f32_to_e4m3_fnuz: bad pointer or size");
  for (int64_t i = 0; i < n; ++i) out[i] = e4m3_fnuz(in[i]);
  mx::clear_error();
  return MX_OK;
}

mx_status mx_e4m3_to_f32(const uint8_t* in, float* out, int64_t n, int32_t fmt) {
  if (n < 0 || (n > 0 && (!in || !out))) return mx::fail(MX_ERR_INVALID_ARG, "mx_e4m3_to_f32: bad pointer or size");
  if (fmt != MX_FP8_E4M3_OCP && fmt != MX_FP8_E4M3_FNUZ) return mx::fail(MX_ERR_INVALID_ARG, "mx_e4m3_to_f32: unknown format %d", fmt);
  for (int64_t i = 0; i < n; ++i) out[i] = e4m3_value(in[i], fmt);
  mx::clear_error();
  return MX_OK;
}

mx_status mx_e8m0_to_f32(const uint8_t* in, float* out, int64_t n) {
  if (n < 0 || (n > 0 && (!in || !out))) return mx::fail(MX_ERR_INVALID_ARG, "mx_e8m0_to_f32: bad pointer or size");
  for (int64_t i = 0; i < n; ++i) out[i] = in[i] == 0xFF ? NAN : std::ldexp(1.0f, static_cast<int>(in[i]) - 127);
  mx::clear_error();
  return MX_OK;
}

}  // extern "C"
