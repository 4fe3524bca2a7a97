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
