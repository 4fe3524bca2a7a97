"""Inverse rotary position embedding -- oracle, test infrastructure.

"[ROCm][DSV4][Perf] Use FP8 WO_A output projection" (Summary, item 1) fuses an
inverse RoPE into the quantiser that feeds ``wo_a``; its Implementation section
caches contiguous BF16 cosine/sine tables once after weight load.  The pages do
not spell the rotation out, so the readings taken here are:

* the rotated slice is the last ``rope_dim`` dims of every head of size D;
* "inverse" is the rotation by -pos*omega_i: a pair (x, y) becomes
  (x*c + y*s, y*c - x*s) with c = cos, s = sin read from the BF16 tables at
  [pos, i] -- multiplication by the complex conjugate of exp(i*pos*omega_i);
* pairs are either interleaved, (2i, 2i+1) of the slice (RoFormer's pairing,
  the default), or split halves, (i, i + rope_dim/2) ("neox");
* arithmetic is fp32 with every product and sum rounded on its own (no fused
  multiply-add), in the order written above, and the result is rounded to BF16
  (nearest, ties to even) before anything else reads it.  "[ROCm][DSv4]
  Functional fixes ..." (Purpose) shows the unfused reference materialising
  BF16 here.

Pins (tests/test_oracle_rope.py): position 0 is the identity; a hand-computed
rotation at position 1; the conjugate-multiplication form in fp64 complex
arithmetic; forward after inverse returns the input within the table's
precision; the split-half pairing is the interleaved one up to a permutation
of the rotated dims; and inputs derived in exact rationals
(tests/golden/rope_rounding_cases.txt) whose BF16 result is fixed by the fp32
rounding of the sum -- an fp64 rotation rounded once gives other bits there.
Products of two BF16 values are exact in fp32, so whether the products are
rounded on their own or fused into the sum cannot change any result.
"""

import numpy as np

from .formats import bf16_to_f32, f32_to_bf16_rne

INTERLEAVED = "interleaved"
NEOX = "neox"


def pair_indices(D, rope_dim, style):
    """Within-head dim indices (first, second) of every rotated pair i."""
    base = D - rope_dim
    half = rope_dim // 2
    i = np.arange(half)
    if style == INTERLEAVED:
        return base + 2 * i, base + 2 * i + 1
    if style == NEOX:
        return base + i, base + half + i
    raise ValueError(style)


def inverse_rope(x_bits, positions, cos_bits, sin_bits, H, D, rope_dim, style=INTERLEAVED):
    """Inverse RoPE of x [T, H*D] (BF16 bits) -> rotated BF16 bits [T, H*D].

    ``positions`` int64 [T]; ``cos_bits``/``sin_bits`` BF16 bits [P, rope_dim/2].
    Dims outside the rotated slice pass through unchanged.  rope_dim = 0 is
    the identity.
    """
    x_bits = np.asarray(x_bits, dtype=np.uint16)
    T = x_bits.shape[0]
    assert x_bits.shape == (T, H * D)
    out = x_bits.copy()
    if rope_dim == 0 or T == 0:
        return out
    assert rope_dim % 2 == 0 and rope_dim <= D
    pos = np.asarray(positions, dtype=np.int64)
    c = bf16_to_f32(np.asarray(cos_bits)[pos])          # [T, rope_dim/2] f32
    s = bf16_to_f32(np.asarray(sin_bits)[pos])
    i0, i1 = pair_indices(D, rope_dim, style)
    xv = bf16_to_f32(x_bits).reshape(T, H, D)
    ov = out.reshape(T, H, D)
    for h in range(H):
        x = xv[:, h, i0]
        y = xv[:, h, i1]
        # numpy float32 ufuncs round each operation on its own
        xc = (x * c).astype(np.float32)
        ys = (y * s).astype(np.float32)
        yc = (y * c).astype(np.float32)
        xs = (x * s).astype(np.float32)
        xr = (xc + ys).astype(np.float32)
        yr = (yc - xs).astype(np.float32)
        ov[:, h, i0] = f32_to_bf16_rne(xr)
        ov[:, h, i1] = f32_to_bf16_rne(yr)
    return out
