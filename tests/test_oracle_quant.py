"""Pins of the oracle's group quantiser.

* A hand-quantised group (tests/golden/quant_group_hand_case.txt) for both
  byte flavours.
* The error bound of round-to-nearest: every decoded value is within half a
  code step of r (and the group's largest magnitude is never saturated).
* Scaling a token by 2**k shifts every scale byte by k and keeps every code.
* Tokens are independent (permuting tokens permutes outputs).
* FNUZ bytes are OCP bytes with 0x80 -> 0x00 and scale + 1 (the FNUZ grid is
  the OCP grid halved, and M halves with it).
* All-zero, NaN and Inf groups.
"""

import numpy as np
import pytest

import workloads
from conftest import read_golden
from oracle import formats as F
from oracle.quant import group_quant, inv_rope_group_quant


def _x(T, L, seed, outliers=True):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((T, L), dtype=np.float32)
    if outliers:
        x[:, rng.choice(L, L // 100, replace=False)] *= 20
    return workloads.to_bf16_bits(x)


def test_hand_group():
    rows = read_golden("quant_group_hand_case.txt")
    r = np.zeros((1, 32), np.float32)
    r[0, :len(rows)] = [float(x[0]) for x in rows]
    bits = F.f32_to_bf16_rne(r)
    assert np.array_equal(F.bf16_to_f32(bits), r)        # the values are BF16 already
    for fmt, col, scale in ((F.OCP, 1, 120), (F.FNUZ, 2, 121)):
        q, s = group_quant(bits, 32, fmt)
        assert s.tolist() == [[scale]]
        want = [int(x[col], 16) for x in rows] + [0] * (32 - len(rows))
        assert q[0].tolist() == want, fmt


@pytest.mark.parametrize("fmt", [F.OCP, F.FNUZ])
@pytest.mark.parametrize("group", [32, 128])
def test_round_to_nearest_error_bound(fmt, group):
    x = _x(16, 1024, 1)
    q, s = group_quant(x, group, fmt)
    r = F.bf16_to_f64(x).reshape(16, -1, group)
    e = s.astype(np.int64)[:, :, None] - 127
    dq = F.e4m3_decode(q, fmt).reshape(16, -1, group) * np.ldexp(1.0, e)
    # step of the e4m3 grid around |r|*2^-e: 2^(floor(log2 v) - 3), at least the
    # subnormal step
    v = np.abs(r) * np.ldexp(1.0, -e)
    sub = 2.0 ** (-9 if fmt == F.OCP else -10)
    step = np.maximum(np.ldexp(1.0, np.floor(np.log2(np.maximum(v, 1e-300))).astype(int) - 3), sub)
    assert np.all(np.abs(dq - r) <= 0.5 * step * np.ldexp(1.0, e))
    # amax maps into [M/2, M]: the scale is the tightest power of two
    amax_v = np.max(v, axis=2)
    assert np.all(amax_v <= F.E4M3_MAX[fmt]) and np.all(amax_v > F.E4M3_MAX[fmt] / 2)


@pytest.mark.parametrize("k", [-5, 3, 9])
def test_power_of_two_shift(k):
    x = _x(8, 512, 2)
    q0, s0 = group_quant(x, 128, F.OCP)
    xs = F.f32_to_bf16_rne(np.ldexp(F.bf16_to_f32(x), k).astype(np.float32))
    q1, s1 = group_quant(xs, 128, F.OCP)
    assert np.array_equal(q1, q0)
    assert np.array_equal(s1.astype(int), s0.astype(int) + k)


def test_tokens_independent():
    x = _x(16, 512, 3)
    perm = np.random.default_rng(4).permutation(16)
    q, s = group_quant(x, 128, F.OCP)
    qp, sp = group_quant(x[perm], 128, F.OCP)
    assert np.array_equal(qp, q[perm]) and np.array_equal(sp, s[perm])


def test_fnuz_is_ocp_with_shifted_scale():
    x = _x(32, 1024, 5)
    qo, so = group_quant(x, 128, F.OCP)
    qf, sf = group_quant(x, 128, F.FNUZ)
    assert np.array_equal(sf.astype(int), so.astype(int) + 1)
    assert np.array_equal(qf, np.where(qo == 0x80, 0, qo))


def test_special_groups():
    x = np.zeros((1, 512), np.uint16)
    x[0, 128:256] = 0x8000                   # a group of -0.0
    x[0, 256] = 0x7FC0                       # NaN in group 2
    x[0, 384 + 5] = 0xFF80                   # -Inf in group 3
    x[0, 384 + 6] = 0x3F80
    for fmt, nan in ((F.OCP, 0x7F), (F.FNUZ, 0x80)):
        q, s = group_quant(x, 128, fmt)
        assert s[0].tolist() == [0, 0, 255, 255]
        assert not q[0, :128].any()
        assert np.all(q[0, 128:256] == (0x80 if fmt == F.OCP else 0))
        assert np.all(q[0, 256:] == nan)


def test_fused_equals_unfused_at_position_zero():
    cos, sin = workloads.rope_tables(rows=16)
    x = _x(4, 4 * 128, 6)
    q, s = inv_rope_group_quant(x, np.zeros(4, np.int64), cos, sin, 4, 128, 64)
    q0, s0 = group_quant(x, 128, F.OCP)
    assert np.array_equal(q, q0) and np.array_equal(s, s0)
