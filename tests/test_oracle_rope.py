"""Pins of the oracle's inverse RoPE.

* Position 0 has cos = 1 and sin = 0 exactly, so the rotation is the identity.
* Hand case at position 1, pair 0 (angle 1 rad): the BF16 table entries are
  cos = 0.5390625 (0x3F0A) and sin = 0.83984375 (0x3F57) -- cos(1) = 0.5403...
  and sin(1) = 0.8414... rounded to 8 significant bits -- and the inverse
  rotation takes (1, 0) to (c, -s) and (0, 1) to (s, c) exactly.
* The inverse rotation is multiplication by exp(-i*theta): checked in fp64
  complex arithmetic within fp32 + BF16 rounding.
* Forward rotation after the inverse returns the input within the tables'
  precision.
* Interleaved and split-half pairings touch the dims they should.
"""

import numpy as np
import pytest

import workloads
from conftest import read_golden
from oracle import formats as F
from oracle.rope import inverse_rope, pair_indices, INTERLEAVED, NEOX

COS, SIN = workloads.rope_tables(rows=4096)


def _rand_x(T, H, D, seed):
    rng = np.random.default_rng(seed)
    return workloads.to_bf16_bits(rng.standard_normal((T, H * D), dtype=np.float32))


def test_table_hand_values():
    assert COS[0, 0] == 0x3F80 and SIN[0, 0] == 0x0000
    assert COS[1, 0] == 0x3F0A and SIN[1, 0] == 0x3F57


@pytest.mark.parametrize("style", [INTERLEAVED, NEOX])
def test_position_zero_is_identity(style):
    x = _rand_x(8, 2, 128, 1)
    out = inverse_rope(x, np.zeros(8, np.int64), COS, SIN, 2, 128, 64, style)
    assert np.array_equal(out, x)


@pytest.mark.parametrize("style", [INTERLEAVED, NEOX])
def test_hand_case_position_one(style):
    H, D, R = 1, 128, 64
    i0, i1 = pair_indices(D, R, style)
    x = np.zeros((2, D), np.uint16)
    x[0, i0[0]] = 0x3F80            # (1, 0)
    x[1, i1[0]] = 0x3F80            # (0, 1)
    out = inverse_rope(x, np.array([1, 1]), COS, SIN, H, D, R, style)
    assert (out[0, i0[0]], out[0, i1[0]]) == (0x3F0A, 0xBF57)
    assert (out[1, i0[0]], out[1, i1[0]]) == (0x3F57, 0x3F0A)
    # nothing else moved
    mask = np.ones(D, bool); mask[[i0[0], i1[0]]] = False
    assert not out[:, mask].any()


def test_pairing_layouts():
    i0, i1 = pair_indices(512, 64, INTERLEAVED)
    assert (i0[0], i1[0], i0[-1], i1[-1]) == (448, 449, 510, 511)
    i0, i1 = pair_indices(512, 64, NEOX)
    assert (i0[0], i1[0], i0[-1], i1[-1]) == (448, 480, 479, 511)


@pytest.mark.parametrize("style", [INTERLEAVED, NEOX])
def test_conjugate_multiplication(style):
    T, H, D, R = 64, 3, 128, 64
    x = _rand_x(T, H, D, 2)
    pos = np.random.default_rng(3).integers(0, 4096, T)
    out = F.bf16_to_f64(inverse_rope(x, pos, COS, SIN, H, D, R, style)).reshape(T, H, D)
    xv = F.bf16_to_f64(x).reshape(T, H, D)
    i0, i1 = pair_indices(D, R, style)
    c = F.bf16_to_f64(COS[pos])[:, None, :]
    s = F.bf16_to_f64(SIN[pos])[:, None, :]
    z = (xv[:, :, i0] + 1j * xv[:, :, i1]) * (c - 1j * s)
    mag = np.abs(xv[:, :, i0]) + np.abs(xv[:, :, i1])
    tol = 2.0 ** -8 * np.maximum(np.abs(z.real), np.abs(z.imag)) + 4 * 2.0 ** -24 * mag
    assert np.all(np.abs(out[:, :, i0] - z.real) <= tol)
    assert np.all(np.abs(out[:, :, i1] - z.imag) <= tol)
    # dims before the rotated slice pass through
    keep = np.setdiff1d(np.arange(D), np.concatenate([i0, i1]))
    assert np.array_equal(out[:, :, keep], xv[:, :, keep])


@pytest.mark.parametrize("style", [INTERLEAVED, NEOX])
def test_forward_after_inverse_is_identity(style):
    T, H, D, R = 32, 2, 128, 64
    x = _rand_x(T, H, D, 4)
    pos = np.random.default_rng(5).integers(0, 4096, T)
    r = F.bf16_to_f64(inverse_rope(x, pos, COS, SIN, H, D, R, style)).reshape(T, H, D)
    i0, i1 = pair_indices(D, R, style)
    c = F.bf16_to_f64(COS[pos])[:, None, :]
    s = F.bf16_to_f64(SIN[pos])[:, None, :]
    fx = r[:, :, i0] * c - r[:, :, i1] * s
    fy = r[:, :, i0] * s + r[:, :, i1] * c
    xv = F.bf16_to_f64(x).reshape(T, H, D)
    nrm = np.hypot(xv[:, :, i0], xv[:, :, i1])
    # BF16 tables: c^2 + s^2 = 1 within ~2^-7; BF16 result rounding 2^-9
    assert np.all(np.abs(fx - xv[:, :, i0]) <= 2.0 ** -6 * nrm + 1e-30)
    assert np.all(np.abs(fy - xv[:, :, i1]) <= 2.0 ** -6 * nrm + 1e-30)


def test_rope_dim_zero_is_identity():
    x = _rand_x(4, 2, 128, 6)
    assert np.array_equal(inverse_rope(x, np.arange(4), COS, SIN, 2, 128, 0), x)


# --------------------------------------------------------------- fp32 rounding
#
# tests/golden/rope_rounding_cases.txt holds inputs whose BF16 result depends on
# the fp32 rounding of the rotation's sum (derived in exact rationals by
# tests/golden/make_rope_rounding_cases.py).  Products of BF16 values are exact
# in fp32, so a fused multiply-add cannot differ from separately rounded
# products; what these cases fix is that the sum is rounded to fp32 before the
# BF16 rounding, not rotated in fp64 and rounded once.

ROUNDING = read_golden("rope_rounding_cases.txt")


def _case_input(row, D, R, style):
    pos, i = int(row[0]), int(row[1])
    xb, yb = int(row[4], 16), int(row[5], 16)
    i0, i1 = pair_indices(D, R, style)
    x = np.zeros((1, D), np.uint16)
    x[0, i0[i]], x[0, i1[i]] = xb, yb
    return x, np.array([pos], np.int64), i0[i], i1[i]


@pytest.mark.parametrize("style", [INTERLEAVED, NEOX])
@pytest.mark.parametrize("row", ROUNDING, ids=lambda r: f"pos{r[0]}-i{r[1]}-{r[10][0]}")
def test_fp32_sum_rounding_golden(row, style):
    pos, i = int(row[0]), int(row[1])
    assert (COS[pos, i], SIN[pos, i]) == (int(row[2], 16), int(row[3], 16))
    D = R = 64
    x, p, a, b = _case_input(row, D, R, style)
    out = inverse_rope(x, p, COS, SIN, 1, D, R, style)
    assert (out[0, a], out[0, b]) == (int(row[6], 16), int(row[7], 16))


@pytest.mark.parametrize("row", ROUNDING, ids=lambda r: f"pos{r[0]}-i{r[1]}-{r[10][0]}")
def test_fp64_rotation_fails_the_rounding_pin(row):
    """A rotation in fp64 rounded once to BF16 -- the plausible mistake the
    golden cases are there to catch -- gives a different BF16 result."""
    pos, i = int(row[0]), int(row[1])
    c = float(F.bf16_to_f64(COS[pos, i]))
    s = float(F.bf16_to_f64(SIN[pos, i]))
    x = float(F.bf16_to_f64(np.uint16(int(row[4], 16))))
    y = float(F.bf16_to_f64(np.uint16(int(row[5], 16))))
    # exact in fp64: 16-bit products, sums within 53 bits
    mx = F.f64_to_bf16_rne(np.array([x * c + y * s, y * c - x * s]))
    assert (int(mx[0]), int(mx[1])) == (int(row[8], 16), int(row[9], 16))
    assert (int(mx[0]), int(mx[1])) != (int(row[6], 16), int(row[7], 16))


def test_products_of_bf16_are_exact_in_fp32():
    """Why no FMA variant can differ: a product of two BF16 values has at most
    16 significant bits, so fp32 holds it exactly (checked on every pair of
    positive mantissas; the exponent only shifts the product)."""
    m = np.arange(128, 256, dtype=np.int64)
    prod = m[:, None] * m[None, :]                 # < 2^16
    assert prod.max() < 2 ** 16
    a = (m.astype(np.float32) / 128)[:, None] * (m.astype(np.float32) / 128)[None, :]
    assert np.array_equal(a.astype(np.float64) * 2 ** 14, prod.astype(np.float64))


@pytest.mark.parametrize("R", [16, 64, 128])
def test_interleaved_is_neox_up_to_a_permutation(R):
    """Moving interleaved pair i, dims (2i, 2i+1) of the rotated slice, to the
    split-half dims (i, i + R/2) and rotating with the split-half pairing gives
    the interleaved rotation, moved the same way."""
    T, H, D = 16, 3, 128
    x = _rand_x(T, H, D, 7)
    pos = np.random.default_rng(8).integers(0, 4096, T)
    base, half = D - R, R // 2
    perm = np.arange(D)                     # neox dim j takes interleaved dim perm[j]
    perm[base:base + half] = base + 2 * np.arange(half)
    perm[base + half:] = base + 2 * np.arange(half) + 1
    xv = x.reshape(T, H, D)
    xn = np.ascontiguousarray(xv[:, :, perm]).reshape(T, H * D)
    cos, sin = workloads.rope_tables(rows=4096, rope_dim=R)
    ri = inverse_rope(x, pos, cos, sin, H, D, R, INTERLEAVED).reshape(T, H, D)
    rn = inverse_rope(xn, pos, cos, sin, H, D, R, NEOX).reshape(T, H, D)
    assert np.array_equal(rn, ri[:, :, perm])
    assert not np.array_equal(ri, xv)       # the rotation did something
