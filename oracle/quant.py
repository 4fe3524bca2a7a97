"""Per-token group E8M0 FP8 quantisation -- oracle, test infrastructure.

"[ROCm][DSV4][Perf] Use FP8 WO_A output projection" (Summary, item 1): the
attention output is inverse-rotated and quantised per token to FP8 with one
E8M0 scale per group of 128 consecutive elements.  The FP8 byte flavour is OCP
on gfx950 and FNUZ (saturating at 224) on gfx942 ("[ROCm][DSv4] Functional
fixes for DeepSeek V4 on MI300X/MI325X", Purpose).  For each group:

1. amax = max |r| over the group (r already rounded to BF16);
2. e = the smallest integer with amax <= M * 2**e, i.e. ceil(log2(amax/M)),
   clamped to [-127, 127]; scale byte = e + 127 (0xFF if the group holds a
   NaN or an Inf);
3. every element becomes the e4m3 code nearest to r * 2**-e (exact in fp64),
   ties to the even code, saturating at +-M.  A group whose scale is NaN gets
   the format's NaN code everywhere.

Pins: exhaustive scale table against the closed form on BF16 bits, hand
cases, the power-of-two shift invariant, the OCP/FNUZ byte relation
(tests/test_oracle_quant.py).
"""

import numpy as np

from .formats import (bf16_to_f64, e4m3_encode, e8m0_table_for_bf16_amax,
                      OCP, FNUZ)
from .rope import inverse_rope, INTERLEAVED


def group_quant(r_bits, group, fmt):
    """Quantise rows of BF16 bits [R, L] in groups of ``group`` along L.

    Returns (codes uint8 [R, L], scales uint8 [R, L/group]).
    """
    r_bits = np.asarray(r_bits, dtype=np.uint16)
    R, L = r_bits.shape
    assert L % group == 0
    vals = bf16_to_f64(r_bits).reshape(R, L // group, group)
    mag = np.abs(vals)
    nonfinite = ~np.all(np.isfinite(vals), axis=2)
    amax = np.where(nonfinite, 0.0, np.max(mag, axis=2, initial=0.0))
    # amax is one of the group's BF16 magnitudes, so its BF16 pattern indexes
    # the exact scale table
    amax_bits = (amax.astype(np.float32).view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    scales = e8m0_table_for_bf16_amax(fmt)[amax_bits]
    scales = np.where(nonfinite, np.uint8(0xFF), scales).astype(np.uint8)
    e = scales.astype(np.int64) - 127
    v = np.ldexp(vals, -e[:, :, None])
    codes = e4m3_encode(v, fmt)
    nan_code = 0x7F if fmt == OCP else 0x80
    codes = np.where(nonfinite[:, :, None], np.uint8(nan_code), codes)
    return codes.reshape(R, L).astype(np.uint8), scales


def inv_rope_group_quant(x_bits, positions, cos_bits, sin_bits, H, D, rope_dim,
                         style=INTERLEAVED, group=128, fmt=OCP):
    """The fused step of the path, unfused: inverse RoPE then group quant.

    x [T, H*D] BF16 bits -> (codes uint8 [T, H*D], scales uint8 [T, H*D/group]).
    """
    r = inverse_rope(x_bits, positions, cos_bits, sin_bits, H, D, rope_dim, style)
    return group_quant(r, group, fmt)


__all__ = ["group_quant", "inv_rope_group_quant", "OCP", "FNUZ"]
