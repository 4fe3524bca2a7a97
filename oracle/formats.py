"""Number formats: BF16, e4m3 (OCP and FNUZ), E8M0 -- oracle, test infrastructure.

Every function here is written from the format definitions, not from any
implementation:

* BF16 is the upper half of an IEEE-754 binary32; rounding is to nearest, ties
  to even.
* OCP e4m3 (OCP 8-bit floating point specification): 1 sign, 4 exponent bits
  with bias 7, 3 mantissa bits, subnormals at exponent field 0, no infinities,
  NaN = S.1111.111, largest finite 448.  This is the byte format of the
  checkpoint's FP8 ``wo_a`` weight and of gfx950 activations ("[ROCm][DSV4][Perf]
  Use FP8 WO_A output projection", Summary; "[ROCm][DSv4] Functional fixes for
  DeepSeek V4 on MI300X/MI325X", Purpose).
* FNUZ e4m3: exponent bias 8, subnormals at exponent field 0, the only NaN is
  0x80, no negative zero, largest finite 240.  The pages cap its use at 224
  ("[ROCm][DSv4] Functional fixes ...", Purpose: FNUZ uses max value 224).
* E8M0 ("UE8M0", ``float8_e8m0fnu``): an unsigned biased exponent, value
  2**(b - 127), 0xFF = NaN ("[ROCm][DSV4][Perf] Use FP8 WO_A output projection",
  Implementation: native E8M0 bytes or lossless conversion of power-of-two
  FP32 scales to biased exponent bytes).
"""

from fractions import Fraction
import math

import numpy as np

OCP = "ocp"
FNUZ = "fnuz"

#: Saturation bound of each e4m3 flavour as the pages use it.
E4M3_MAX = {OCP: 448.0, FNUZ: 224.0}


# --------------------------------------------------------------------------- BF16

def bf16_to_f32(bits):
    """BF16 bit patterns (uint16) -> float32 values (exact)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32)


def bf16_to_f64(bits):
    """BF16 bit patterns (uint16) -> float64 values (exact)."""
    return bf16_to_f32(bits).astype(np.float64)


def f32_to_bf16_rne(x):
    """float32 -> BF16 bits, round to nearest, ties to even, on the bit pattern.

    The textbook integer form: add 0x7FFF plus the lowest kept bit, then drop the
    low 16 bits.  Because IEEE bit patterns of one sign are ordered like their
    values and the kept/dropped split is the same for normals and subnormals,
    this is exact RNE everywhere, and a carry out of the mantissa correctly
    bumps the exponent (to Inf past the largest finite).  NaNs are kept quiet
    (the quiet bit is forced so that truncation cannot turn them into Inf).
    """
    x = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    u = x.view(np.uint32).astype(np.uint64)
    nan = np.isnan(x)
    rounded = (u + np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16)
    quiet = (u >> np.uint64(16)) | np.uint64(0x0040)
    out = np.where(nan, quiet, rounded)
    return out.astype(np.uint16)


def f64_to_bf16_rne(x):
    """float64 -> BF16 bits, round to nearest, ties to even, by definition.

    Independent of :func:`f32_to_bf16_rne`: write |x| = m * 2**e with m in
    [0.5, 1); a BF16 keeps 8 significant bits down to the smallest normal
    2**-126 and a fixed quantum of 2**-133 below it.  Divide by the quantum,
    round half to even with ``np.rint`` and multiply back (all exact in fp64).
    Magnitudes that round to 2**128 or beyond become Inf.
    """
    x = np.asarray(x, dtype=np.float64)
    out = np.empty(x.shape, dtype=np.float64)
    finite = np.isfinite(x)
    xf = np.where(finite, x, 0.0)
    _, e = np.frexp(xf)
    quantum_exp = np.maximum(e - 8, -133)
    q = np.ldexp(np.ones_like(xf), quantum_exp)
    r = np.rint(xf / q) * q
    r = np.where(np.abs(r) >= 2.0 ** 128, np.copysign(np.inf, xf), r)
    out[...] = np.where(finite, r, x)
    # every value of `out` is now a BF16 value (or Inf/NaN), so the float32
    # conversion is exact and the upper half of its pattern is the answer
    f32 = out.astype(np.float32)
    bits = (np.ascontiguousarray(f32).view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    nan = np.isnan(x)
    bits = np.where(nan, (bits | np.uint16(0x0040)), bits)
    return bits.astype(np.uint16)


# --------------------------------------------------------------------------- e4m3

def e4m3_values(fmt):
    """The value of each of the 256 e4m3 codes (float64; NaN codes -> NaN)."""
    vals = np.empty(256, dtype=np.float64)
    bias = 7 if fmt == OCP else 8
    for code in range(256):
        sign = -1.0 if code & 0x80 else 1.0
        ef = (code >> 3) & 0xF
        mf = code & 0x7
        if ef == 0:
            mag = math.ldexp(mf / 8.0, 1 - bias)          # subnormal
        else:
            mag = math.ldexp(1.0 + mf / 8.0, ef - bias)
        vals[code] = sign * mag
    if fmt == OCP:
        vals[0x7F] = np.nan
        vals[0xFF] = np.nan
    elif fmt == FNUZ:
        vals[0x80] = np.nan                              # the single NaN; no -0
    else:
        raise ValueError(fmt)
    return vals


def e4m3_decode(codes, fmt):
    """e4m3 codes (uint8) -> float64 values."""
    return e4m3_values(fmt)[np.asarray(codes, dtype=np.uint8)]


def e4m3_encode(v, fmt):
    """Values (float64) -> e4m3 codes: nearest, ties to the even code, saturating.

    * NaN -> the format's NaN code (0x7F for OCP, 0x80 for FNUZ).
    * |v| above the saturation bound M (448 OCP, 224 FNUZ), Inf included,
      becomes +-M (code 0x7E / 0xFE in both flavours).
    * Otherwise the nearest of the finite magnitudes <= M is taken; on an exact
      tie the code whose lowest bit is 0 wins.
    * Zeros: OCP keeps the sign (a negative value that rounds to zero, or -0,
      gives 0x80); FNUZ has no negative zero and gives 0x00.
    """
    v = np.asarray(v, dtype=np.float64)
    m = E4M3_MAX[fmt]
    table = e4m3_values(fmt)
    # positive finite magnitudes up to M, indexed by their code (0x00 ...)
    pos = table[:0x80]
    ncodes = int(np.searchsorted(pos[~np.isnan(pos)], m, side="right"))
    mags = pos[:ncodes]
    assert np.all(np.diff(mags) > 0) and mags[-1] == m

    nan = np.isnan(v)
    neg = np.signbit(v)
    a = np.where(nan, 0.0, np.minimum(np.abs(v), m))
    hi = np.searchsorted(mags, a, side="left")           # mags[hi-1] < a <= mags[hi]
    hi = np.minimum(hi, ncodes - 1)
    lo = np.maximum(hi - 1, 0)
    d_lo = a - mags[lo]
    d_hi = mags[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    pick_hi |= a == mags[hi]
    mag_code = np.where(pick_hi, hi, lo).astype(np.int64)
    if fmt == OCP:
        code = np.where(neg, mag_code | 0x80, mag_code)
        code = np.where(nan, 0x7F, code)
    else:
        code = np.where(neg & (mag_code != 0), mag_code | 0x80, mag_code)
        code = np.where(nan, 0x80, code)
    return code.astype(np.uint8)


# --------------------------------------------------------------------------- E8M0

def e8m0_decode(b):
    """E8M0 bytes -> float64 values 2**(b-127); 0xFF -> NaN."""
    b = np.asarray(b, dtype=np.int64)
    out = np.ldexp(np.ones(b.shape), b - 127)
    return np.where(b == 255, np.nan, out)


def e8m0_exponent_for_amax(amax, fmt):
    """Scale exponent for one group, by the definition (exact rational arithmetic).

    The quantiser picks the E8M0 scale 2**e with e = ceil(log2(amax / M)), M the
    saturation bound of the FP8 flavour; equivalently e is the smallest integer
    with amax <= M * 2**e.  It is clamped to the E8M0 range [-127, 127].  An
    all-zero group (amax = 0) takes the clamp, -127.  Returns the integer e, or
    None when amax is not finite (the scale byte is then NaN, 0xFF).
    """
    if not math.isfinite(amax):
        return None
    if amax == 0:
        return -127
    a = Fraction(amax)
    mm = Fraction(E4M3_MAX[fmt])
    # start from a float estimate and correct it with exact comparisons
    e = math.ceil(math.log2(amax / E4M3_MAX[fmt]))
    while a > mm * Fraction(2) ** e:
        e += 1
    while a <= mm * Fraction(2) ** (e - 1):
        e -= 1
    return max(-127, min(127, e))


_E8M0_TABLES = {}


def e8m0_table_for_bf16_amax(fmt):
    """Scale byte for every non-negative BF16 amax pattern 0x0000..0x7FFF."""
    if fmt not in _E8M0_TABLES:
        vals = bf16_to_f64(np.arange(0x8000, dtype=np.uint16))
        tab = np.empty(0x8000, dtype=np.uint8)
        for i, a in enumerate(vals):
            e = e8m0_exponent_for_amax(float(a), fmt)
            tab[i] = 0xFF if e is None else e + 127
        _E8M0_TABLES[fmt] = tab
    return _E8M0_TABLES[fmt]


def f32_pow2_to_e8m0(x):
    """Lossless FP32 -> E8M0 conversion of power-of-two scales.

    ("[ROCm][DSV4][Perf] Use FP8 WO_A output projection", Implementation:
    positive power-of-two FP32 scales become biased E8M0 exponent bytes without
    loss.)  A value converts iff it is exactly 2**n with -127 <= n <= 127 (2**-127
    is an FP32 subnormal and is accepted); its byte is n + 127.  Returns
    (bytes uint8, ok bool); bytes are 0 where ok is False.
    """
    x = np.asarray(x, dtype=np.float32).astype(np.float64)
    out = np.zeros(x.shape, dtype=np.uint8)
    ok = np.zeros(x.shape, dtype=bool)
    for idx, v in np.ndenumerate(x):
        if not math.isfinite(v) or v <= 0:
            continue
        mant, exp = math.frexp(v)          # v = mant * 2**exp, mant in [0.5, 1)
        if mant != 0.5:
            continue
        n = exp - 1
        if -127 <= n <= 127:
            out[idx] = n + 127
            ok[idx] = True
    return out, ok
