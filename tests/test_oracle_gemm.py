"""Pins of the oracle's GEMMs, dequantisation and the MXFP8 linear.

* Batched GEMM on the tiny wo_a problem against an exact integer evaluation:
  every e4m3 value is an integer times 2**-9 (OCP) or 2**-10 (FNUZ), so each
  128-element block of products sums exactly in int64, and blocks are combined
  with exact rationals.
* All codes 1.0 with unit scales give K; a one-hot W column reproduces the
  dequantised A column (catches transposed operands and index slips).
* Dequantisation against torch's float8_e4m3fn decode times 2**(s-127) cast to
  BF16 (a library routine); it is exact for the scale range in use.
* The MXFP8 linear's branch table as printed on the pages, and both branches
  on small inputs against exact evaluation.
* The BF16 arm: the grouped BF16 product against exact rational sums (BF16
  decoded by torch), a one-hot W per (g, n), equality with the FP8 product of
  the group-128 dequantised operands; the end-to-end BF16 arm reduces to the
  plain product at position 0 and lies within the FP8 quantisation error
  bound of the FP8 arm.
"""

from fractions import Fraction

import numpy as np
import pytest
import torch

import workloads
from conftest import read_golden
from oracle import formats as F
from oracle import gemm as Gm
from oracle.quant import group_quant


def _int_and_exp(codes, fmt):
    """e4m3 codes -> (integer numerator, exponent) with value = num * 2**exp."""
    step = -9 if fmt == F.OCP else -10
    v = F.e4m3_decode(codes, fmt)
    num = np.ldexp(v, -step)
    assert np.all(num == np.round(num))
    return num.astype(np.int64), step


def _exact_bmm(a, sa, w, sw, a_fmt=F.OCP):
    T, G, K = a.shape
    N = w.shape[1]
    ia, ea = _int_and_exp(a, a_fmt)
    iw, ew = _int_and_exp(w, F.OCP)
    out = np.empty((T, G, N), dtype=object)
    nb = K // 128
    for g in range(G):
        # block sums, exact in int64: |ia*iw| < 2^36, 128 terms < 2^43
        blk = np.einsum("tbk,nbk->tnb", ia[:, g].reshape(T, nb, 128).astype(np.int64),
                        iw[g].reshape(N, nb, 128).astype(np.int64), optimize=False)
        for t in range(T):
            for n in range(N):
                acc = Fraction(0)
                for b in range(nb):
                    ex = int(sa[t, g, b]) - 127 + int(sw[g, n, b]) - 127 + ea + ew
                    acc += Fraction(int(blk[t, n, b])) * Fraction(2) ** ex
                out[t, g, n] = acc
    return out


@pytest.mark.parametrize("a_fmt", [F.OCP, F.FNUZ])
def test_bmm_tiny_exact(a_fmt):
    p = workloads.tiny()
    cos, sin = workloads.rope_tables(rows=16)
    from oracle.quant import inv_rope_group_quant
    a, sa = inv_rope_group_quant(p.x, p.positions, cos, sin, p.H, p.D, 64, fmt=a_fmt)
    a = a.reshape(p.T, p.G, p.K)
    sa = sa.reshape(p.T, p.G, p.K // 128)
    ours = Gm.bmm_a8w8_mxscale(a, sa, p.w, p.w_scale, a_fmt=a_fmt)
    exact = _exact_bmm(a, sa, p.w, p.w_scale, a_fmt)
    ex = np.vectorize(float)(exact)
    scale = np.abs(ours).max()
    assert np.all(np.abs(ours - ex) <= 1e-13 * scale)


def test_bmm_fnuz_equals_ocp_run():
    """The same activations quantised to FNUZ and to OCP give the same product."""
    p = workloads.tiny()
    cos, sin = workloads.rope_tables(rows=16)
    from oracle.quant import inv_rope_group_quant
    outs = []
    for fmt in (F.OCP, F.FNUZ):
        a, sa = inv_rope_group_quant(p.x, p.positions, cos, sin, p.H, p.D, 64, fmt=fmt)
        outs.append(Gm.bmm_a8w8_mxscale(a.reshape(p.T, p.G, p.K), sa.reshape(p.T, p.G, -1),
                                         p.w, p.w_scale, a_fmt=fmt))
    assert np.array_equal(outs[0], outs[1])


def test_bmm_all_ones():
    T, G, N, K = 3, 2, 5, 384
    a = np.full((T, G, K), 0x38, np.uint8)
    w = np.full((G, N, K), 0x38, np.uint8)
    sa = np.full((T, G, K // 128), 127, np.uint8)
    sw = np.full((G, N, K // 128), 127, np.uint8)
    assert np.all(Gm.bmm_a8w8_mxscale(a, sa, w, sw) == K)


def test_bmm_one_hot_and_orientation():
    T, G, N, K = 4, 3, 6, 256
    a, sa, _, _ = workloads.gemm_operands(7, T, G, N, K)
    w = np.zeros((G, N, K), np.uint8)
    sw = np.full((G, N, K // 128), 127, np.uint8)
    picks = np.arange(N) * 37 % K
    for g in range(G):
        for n in range(N):
            w[g, n, picks[n]] = 0x38
    out = Gm.bmm_a8w8_mxscale(a, sa, w, sw)
    for g in range(G):
        for n in range(N):
            k = picks[n]
            want = F.e4m3_decode(a[:, g, k], F.OCP) * F.e8m0_decode(sa[:, g, k // 128])
            assert np.array_equal(out[:, g, n], want)


def test_dequant_matches_torch_decode():
    data = workloads.mxfp8_linear()
    for K in (288, 576):
        _, w, ws, _ = data[K]
        w, ws = w[:512], ws[:512]
        ours = Gm.dequant_mxfp8_to_bf16(w, ws, 32)
        dec = torch.from_numpy(w.copy()).view(torch.float8_e4m3fn).to(torch.float32)
        sc = torch.from_numpy(np.repeat(F.e8m0_decode(ws), 32, axis=1)).to(torch.float32)
        ref = (dec * sc).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        assert np.array_equal(ours, ref)


@pytest.mark.parametrize("row", read_golden("mxfp8_linear_dispatch.txt"), ids=lambda r: r[0])
def test_linear_dispatch_table(row):
    K, residue, branch = int(row[0]), int(row[1]), row[2]
    assert K % 128 == residue
    assert Gm.linear_uses_bf16(K) == (branch == "bf16")


def _exact_dot(xv, wv):
    return sum(Fraction(float(a)) * Fraction(float(b)) for a, b in zip(xv, wv))


@pytest.mark.parametrize("K", [288, 1152])
def test_mx_linear_both_branches_exact(K):
    x, w, ws, _ = workloads.mxfp8_linear()[K]
    x, w, ws = x[:3], w[:4], ws[:4]
    out = Gm.mx_linear(x, w, ws, 32)
    if Gm.linear_uses_bf16(K):
        xv = F.bf16_to_f64(x)
        wv = F.bf16_to_f64(Gm.dequant_mxfp8_to_bf16(w, ws, 32))
    else:
        xq, xs = group_quant(x, 32, F.OCP)
        xv = F.e4m3_decode(xq, F.OCP) * np.repeat(F.e8m0_decode(xs), 32, axis=1)
        wv = F.e4m3_decode(w, F.OCP) * np.repeat(F.e8m0_decode(ws), 32, axis=1)
    for m in range(3):
        for n in range(4):
            ex = float(_exact_dot(xv[m], wv[n]))
            assert abs(out[m, n] - ex) <= 1e-12 * max(1.0, abs(ex))


# ---- the BF16 arm: bmm_bf16 and wo_a_bf16


def _torch_bf16_values(bits):
    """BF16 bit patterns -> float64 through torch's own BF16 decode."""
    t = torch.from_numpy(np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16)).view(torch.bfloat16)
    return t.to(torch.float64).numpy()


def test_bmm_bf16_against_exact_rationals():
    rng = np.random.default_rng(11)
    T, G, N, K = 3, 2, 5, 40
    x = workloads.activations(rng, T * G, K).reshape(T, G, K)
    w = workloads.activations(rng, G * N, K).reshape(G, N, K)
    out = Gm.bmm_bf16(x, w)
    xv, wv = _torch_bf16_values(x), _torch_bf16_values(w)
    for t in range(T):
        for g in range(G):
            for n in range(N):
                exact = sum(Fraction(float(a)) * Fraction(float(b)) for a, b in zip(xv[t, g], wv[g, n]))
                mag = float(np.sum(np.abs(xv[t, g] * wv[g, n])))
                assert abs(Fraction(out[t, g, n]) - exact) <= Fraction(K * mag) * Fraction(2) ** -52


def test_bmm_bf16_one_hot_and_orientation():
    rng = np.random.default_rng(12)
    T, G, N, K = 4, 3, 6, 64
    x = workloads.activations(rng, T * G, K).reshape(T, G, K)
    w = np.zeros((G, N, K), np.uint16)
    picks = (np.arange(N)[None, :] * 11 + 7 * np.arange(G)[:, None] + 5) % K     # per (g, n)
    for g in range(G):
        for n in range(N):
            w[g, n, picks[g, n]] = 0x3F80       # BF16 1.0
    out = Gm.bmm_bf16(x, w)
    xv = _torch_bf16_values(x)
    for g in range(G):
        for n in range(N):
            assert np.array_equal(out[:, g, n], xv[:, g, picks[g, n]])


def test_bmm_bf16_equals_fp8_product_of_dequantised_operands():
    # every scaled e4m3 value with scale exponents in [-12, -2] is a BF16 value,
    # so the group-128 dequantisations carry the FP8 operands exactly and the two
    # grouped products are the same fp64 computation
    T, G, N, K = 5, 2, 7, 256
    a, sa, w, sw = workloads.gemm_operands(13, T, G, N, K)
    ab = Gm.dequant_mxfp8_to_bf16(a.reshape(T * G, K), sa.reshape(T * G, K // 128), 128).reshape(T, G, K)
    wb = Gm.dequant_mxfp8_to_bf16(w.reshape(G * N, K), sw.reshape(G * N, K // 128), 128).reshape(G, N, K)
    assert np.array_equal(Gm.bmm_bf16(ab, wb), Gm.bmm_a8w8_mxscale(a, sa, w, sw))


def test_wo_a_bf16_position_zero_is_the_plain_product():
    p = workloads.tiny()
    cos, sin = workloads.rope_tables(rows=64)
    wb = workloads.activations(np.random.default_rng(14), p.G * p.N, p.K).reshape(p.G, p.N, p.K)
    zero = np.zeros(p.T, np.int64)
    out = Gm.wo_a_bf16(p.x, zero, cos, sin, p.H, p.D, 64, wb)
    assert np.array_equal(out, Gm.bmm_bf16(p.x.reshape(p.T, p.G, p.K), wb))


def test_wo_a_bf16_within_fp8_quantisation_error_of_the_fp8_arm():
    # The FP8 arm differs from the BF16 arm only by the activation quantisation:
    # |q(r) - r| <= 2^-4 |r| + 2^(e-10) per element (e4m3 round to nearest,
    # subnormal step 2^(e-9) with the group exponent e), so the two outputs
    # differ by at most sum_k (2^-4 |r_k| + 2^(e_k-10)) |w_k|.
    from oracle.quant import inv_rope_group_quant
    from oracle.rope import inverse_rope
    p = workloads.tiny()
    cos, sin = workloads.rope_tables(rows=64)
    wb = Gm.dequant_mxfp8_to_bf16(p.w.reshape(p.G * p.N, p.K), p.w_scale.reshape(p.G * p.N, -1), 128)
    wb = wb.reshape(p.G, p.N, p.K)
    bf = Gm.wo_a_bf16(p.x, p.positions, cos, sin, p.H, p.D, 64, wb)
    q, s = inv_rope_group_quant(p.x, p.positions, cos, sin, p.H, p.D, 64)
    fp8 = Gm.bmm_a8w8_mxscale(q.reshape(p.T, p.G, p.K), s.reshape(p.T, p.G, -1), p.w, p.w_scale)
    r = _torch_bf16_values(inverse_rope(p.x, p.positions, cos, sin, p.H, p.D, 64)).reshape(p.T, p.G, p.K)
    e = np.repeat(s.reshape(p.T, p.G, -1).astype(np.int64) - 127, 128, axis=2)
    per = 2.0 ** -4 * np.abs(r) + np.ldexp(1.0, e - 10)
    wv = np.abs(_torch_bf16_values(wb))
    bound = np.einsum("tgk,gnk->tgn", per, wv)
    assert np.all(np.abs(fp8 - bf) <= bound)
    assert np.any(fp8 != bf)                   # the arms do differ
