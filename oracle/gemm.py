"""Scaled GEMMs, MXFP8 dequantisation and the MXFP8 linear -- oracle, test infrastructure.

* Batched a8w8 MX-scale GEMM ("[ROCm][DSV4][Perf] Use FP8 WO_A output
  projection", Summary item 2): out[t, g, n] = sum_k A[t,g,k] * W[g,n,k] where
  each FP8 operand is decoded and multiplied by its E8M0 block scale
  2**(s-127), one scale per 128 consecutive k.  Computed here in fp64 with
  numpy's float64 matmul; the result is left unrounded.
* MXFP8 -> BF16 dequantisation ("[ROCm][DSv4.1][Perf] Dequantize the MXFP8
  weight once when dot_scaled cannot be used", Purpose): w_bf16[n, k] =
  bf16(decode(w[n,k]) * 2**(s[n, k/block] - 127)), rounded to nearest even
  from the exact fp64 product.
* The BF16 arm of ``wo_a`` ("[ROCm][DSV4][Perf] Use FP8 WO_A output
  projection", Summary and Related work: the path the FP8 one replaces and
  keeps as its fallback -- an inverse RoPE, then a BF16 grouped einsum over a
  BF16 copy of the weight made once at load): out[t, g, n] = sum_k
  x[t,g,k] * W[g,n,k] on BF16 operands, in fp64, unrounded.  The BF16 weight
  is the group-128 dequantisation of the FP8 checkpoint weight.
* The MXFP8 linear (same page, Purpose and review thread): when K % 128 != 0
  the weight is used as BF16 (dequantised once at load, or per call when it
  was not prepared) and x stays BF16; when K % 128 == 0 the block-scaled FP8
  product is used, for which x is first quantised to MXFP8 (OCP, block 32).
"""

import numpy as np

from .formats import bf16_to_f64, e4m3_decode, e8m0_decode, f64_to_bf16_rne, OCP
from .quant import group_quant
from .rope import INTERLEAVED, inverse_rope

#: The alignment that decides the MXFP8 linear's branch ("[ROCm][DSv4.1][Perf]
#: Dequantize ...", Purpose: dot_scaled needs K % 128 == 0).
LINEAR_K_ALIGN = 128


def scaled_operand(codes, scales, block, fmt=OCP):
    """Decode FP8 codes [..., K] with E8M0 scales [..., K/block] -> fp64 [..., K]."""
    codes = np.asarray(codes, dtype=np.uint8)
    scales = np.asarray(scales, dtype=np.uint8)
    K = codes.shape[-1]
    assert scales.shape[-1] * block == K
    s = np.repeat(e8m0_decode(scales), block, axis=-1)
    return e4m3_decode(codes, fmt) * s


def bmm_a8w8_mxscale(a, a_scale, w, w_scale, a_fmt=OCP, block=128):
    """A u8 [T,G,K], a_scale u8 [T,G,K/block], W u8 OCP [G,N,K], w_scale u8
    [G,N,K/block] -> out fp64 [T,G,N] (unrounded)."""
    a = np.asarray(a, dtype=np.uint8)
    T, G, K = a.shape
    Gw, N, Kw = w.shape
    assert (Gw, Kw) == (G, K)
    out = np.empty((T, G, N), dtype=np.float64)
    for g in range(G):
        af = scaled_operand(a[:, g, :], a_scale[:, g, :], block, a_fmt)    # [T, K]
        wf = scaled_operand(w[g], w_scale[g], block, OCP)                  # [N, K]
        out[:, g, :] = af @ wf.T
    return out


def bmm_bf16(x_bits, w_bits):
    """x BF16 bits [T,G,K], W BF16 bits [G,N,K] -> out fp64 [T,G,N] (unrounded)."""
    x_bits = np.asarray(x_bits, dtype=np.uint16)
    w_bits = np.asarray(w_bits, dtype=np.uint16)
    T, G, K = x_bits.shape
    Gw, N, Kw = w_bits.shape
    assert (Gw, Kw) == (G, K)
    out = np.empty((T, G, N), dtype=np.float64)
    for g in range(G):
        out[:, g, :] = bf16_to_f64(x_bits[:, g, :]) @ bf16_to_f64(w_bits[g]).T
    return out


def wo_a_bf16(x_bits, positions, cos_bits, sin_bits, H, D, rope_dim, w_bits, style=INTERLEAVED):
    """The BF16 arm end to end: inverse RoPE of x [T, H*D] to BF16, viewed as
    [T, G, K], times the BF16 weight [G, N, K] -> fp64 [T, G, N]."""
    G, _, K = np.asarray(w_bits).shape
    xr = inverse_rope(x_bits, positions, cos_bits, sin_bits, H, D, rope_dim, style)
    return bmm_bf16(xr.reshape(xr.shape[0], G, K), w_bits)


def dequant_mxfp8_to_bf16(w, w_scale, block=32):
    """W u8 OCP [N,K] + scales u8 [N,K/block] -> BF16 bits [N,K]."""
    return f64_to_bf16_rne(scaled_operand(w, w_scale, block, OCP))


def linear_uses_bf16(K):
    """The MXFP8 linear's branch predicate: the BF16 path iff K % 128 != 0."""
    return K % LINEAR_K_ALIGN != 0


def linear_bf16(x_bits, w_bf16_bits):
    """x BF16 [M,K] @ W BF16 [N,K]^T in fp64 -> [M,N]."""
    return bf16_to_f64(x_bits) @ bf16_to_f64(w_bf16_bits).T


def linear_mxfp8(x_bits, w, w_scale, block=32):
    """The block-scaled FP8 branch: x is quantised to OCP MXFP8 (block 32) and
    multiplied by the MXFP8 weight in fp64 -> [M,N]."""
    xq, xs = group_quant(x_bits, block, OCP)
    return scaled_operand(xq, xs, block, OCP) @ scaled_operand(w, w_scale, block, OCP).T


def mx_linear(x_bits, w, w_scale, block=32):
    """The MXFP8 linear on an FP8 weight [N,K] with E8M0 scales [N,K/block]:
    the branch is chosen by K % 128 -> fp64 [M,N]."""
    K = np.asarray(w).shape[1]
    if linear_uses_bf16(K):
        return linear_bf16(x_bits, dequant_mxfp8_to_bf16(w, w_scale, block))
    return linear_mxfp8(x_bits, w, w_scale, block)
