"""Pins of the oracle's number formats against things other than itself.

BF16: torch's CPU cast (a library routine) on every BF16 high half crossed with
the interesting low halves; the two independent BF16 encoders agree.
e4m3: hand-computed encodings (tests/golden/e4m3_hand_cases.txt), the decode
table's closed form per code, round trips of every finite code, torch's CPU
float8 casts inside the saturation bound.
E8M0: the exact rational definition against the closed form on BF16 bits
(exponent field, and whether the mantissa exceeds the 1.75 of 448 = 1.75*2^8 /
224 = 1.75*2^7), hand cases, the FNUZ = OCP + 1 relation.
FP32 -> E8M0: every power of two round-trips; hand cases.
"""

import math

import numpy as np
import pytest
import torch

from conftest import read_golden
from oracle import formats as F


def _all_bf16_crossed_with_low_halves():
    hi = np.arange(0x10000, dtype=np.uint32) << 16
    rng = np.random.default_rng(123)
    lows = np.concatenate([np.array([0, 1, 0x7FFF, 0x8000, 0x8001, 0xFFFF], np.uint32),
                           rng.integers(0, 0x10000, 6, dtype=np.uint32)])
    return (hi[:, None] | lows[None, :]).reshape(-1).view(np.float32)


def test_bf16_rne_matches_torch_cast():
    x = _all_bf16_crossed_with_low_halves()
    ours = F.f32_to_bf16_rne(x)
    ref = torch.from_numpy(x.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    nan = np.isnan(x)
    assert np.array_equal(ours[~nan], ref[~nan])
    # NaN stays NaN
    assert np.all(np.isnan(F.bf16_to_f32(ours[nan])))


def test_bf16_two_encoders_agree():
    x = _all_bf16_crossed_with_low_halves()
    a = F.f32_to_bf16_rne(x)
    b = F.f64_to_bf16_rne(x.astype(np.float64))
    nan = np.isnan(x)
    assert np.array_equal(a[~nan], b[~nan])


def test_bf16_hand_cases():
    cases = {1.0: 0x3F80, 1.0 + 2 ** -8: 0x3F80, 1.0 + 3 * 2 ** -8: 0x3F82,
             -2.0: 0xC000, 2.0 ** -133: 0x0001, 2.0 ** -134: 0x0000,
             3 * 2.0 ** -134: 0x0002, 3.0e38: 0x7F62, 3.4e38: 0x7F80}
    for v, bits in cases.items():
        assert int(F.f64_to_bf16_rne(np.array([v]))[0]) == bits, v
        assert int(F.f32_to_bf16_rne(np.array([v], np.float32))[0]) == bits, v


def test_e4m3_decode_closed_form_per_code():
    for fmt, bias in ((F.OCP, 7), (F.FNUZ, 8)):
        t = F.e4m3_values(fmt)
        for c in range(256):
            s, e, m = c >> 7, (c >> 3) & 15, c & 7
            if fmt == F.OCP and (c & 0x7F) == 0x7F:
                assert math.isnan(t[c]); continue
            if fmt == F.FNUZ and c == 0x80:
                assert math.isnan(t[c]); continue
            mag = (m / 8) * 2.0 ** (1 - bias) if e == 0 else (1 + m / 8) * 2.0 ** (e - bias)
            assert t[c] == (-mag if s else mag)
    assert F.e4m3_values(F.OCP)[0x7E] == 448 and F.e4m3_values(F.FNUZ)[0x7F] == 240
    assert F.e4m3_values(F.OCP)[0x01] == 2.0 ** -9 and F.e4m3_values(F.FNUZ)[0x01] == 2.0 ** -10


@pytest.mark.parametrize("row", read_golden("e4m3_hand_cases.txt"), ids=lambda r: f"{r[1]}:{r[0]}")
def test_e4m3_hand_cases(row):
    value, fmt, code = float(row[0]), row[1], int(row[2], 16)
    got = int(F.e4m3_encode(np.array([value]), fmt)[0])
    assert got == code, f"{value} {fmt}: got {got:#04x}, want {code:#04x}"


@pytest.mark.parametrize("fmt", [F.OCP, F.FNUZ])
def test_e4m3_round_trip_every_finite_code(fmt):
    t = F.e4m3_values(fmt)
    m = F.E4M3_MAX[fmt]
    codes = np.array([c for c in range(256) if not math.isnan(t[c]) and abs(t[c]) <= m], np.uint8)
    back = F.e4m3_encode(t[codes], fmt)
    if fmt == F.OCP:
        assert np.array_equal(back, codes)
    else:
        assert np.array_equal(back, codes)     # FNUZ has no -0 code to lose


@pytest.mark.parametrize("fmt,tdtype", [(F.OCP, torch.float8_e4m3fn), (F.FNUZ, torch.float8_e4m3fnuz)])
def test_e4m3_encode_matches_torch_cast_in_range(fmt, tdtype):
    # every BF16 pattern, scaled by several powers of two so that the whole
    # e4m3 range, its subnormals and underflow are covered
    base = F.bf16_to_f32(np.arange(0x10000, dtype=np.uint16)).astype(np.float64)
    m = F.E4M3_MAX[fmt]
    for k in (-130, -20, -12, -8, -4, 0, 4, 8):
        v = np.ldexp(base, k)
        keep = np.isfinite(v) & (np.abs(v) <= m)
        v = v[keep]
        ours = F.e4m3_encode(v, fmt)
        ref = torch.from_numpy(v.astype(np.float32)).to(tdtype).view(torch.uint8).numpy()
        # torch's FNUZ cast and ours agree on zero handling; compare all
        assert np.array_equal(ours, ref), (fmt, k, np.flatnonzero(ours != ref)[:5])


def test_e4m3_saturation_and_nan():
    for fmt in (F.OCP, F.FNUZ):
        m = F.E4M3_MAX[fmt]
        v = np.array([m * 1.01, np.inf, -np.inf, -m * 7, np.nan])
        c = F.e4m3_encode(v, fmt)
        assert list(c[:4]) == [0x7E, 0x7E, 0xFE, 0xFE]
        assert c[4] == (0x7F if fmt == F.OCP else 0x80)


def _closed_form_e8m0(bits, fmt):
    """Scale byte from BF16 amax bits: e = E - E_M + [mantissa > 0.75],
    E_M = 8 (448 = 1.75*2^8) or 7 (224 = 1.75*2^7); subnormal amax handled by
    its own exponent; clamp to [-127, 127]."""
    out = np.empty(bits.size, np.int64)
    em = 8 if fmt == F.OCP else 7
    for i, b in enumerate(bits.tolist()):
        ef, mf = (b >> 7) & 0xFF, b & 0x7F
        if ef == 0xFF:
            out[i] = 255; continue
        if b == 0:
            out[i] = 0; continue
        if ef == 0:                       # subnormal: value mf * 2^-133
            E = mf.bit_length() - 1 - 133
            mant_over = (mf / (1 << (mf.bit_length() - 1))) > 1.75
        else:
            E = ef - 127
            mant_over = mf > 0x60           # 1 + mf/128 > 1.75
        e = E - em + int(mant_over)
        out[i] = max(-127, min(127, e)) + 127
    return out


@pytest.mark.parametrize("fmt", [F.OCP, F.FNUZ])
def test_e8m0_table_equals_closed_form_on_all_bf16_amax(fmt):
    bits = np.arange(0x8000, dtype=np.int64)
    tab = F.e8m0_table_for_bf16_amax(fmt).astype(np.int64)
    assert np.array_equal(tab, _closed_form_e8m0(bits, fmt))


@pytest.mark.parametrize("row", read_golden("e8m0_hand_cases.txt"), ids=lambda r: f"{r[1]}:{r[0]}")
def test_e8m0_hand_cases(row):
    amax, fmt, byte = float(row[0]), row[1], int(row[2])
    e = F.e8m0_exponent_for_amax(amax, fmt)
    assert e + 127 == byte


def test_e8m0_fnuz_is_ocp_plus_one_away_from_clamps():
    ocp = F.e8m0_table_for_bf16_amax(F.OCP).astype(int)
    fnuz = F.e8m0_table_for_bf16_amax(F.FNUZ).astype(int)
    inner = (ocp >= 1) & (ocp <= 253)
    inner[0] = False
    assert np.all(fnuz[inner] == ocp[inner] + 1)


def test_e8m0_decode():
    assert F.e8m0_decode(np.array([127]))[0] == 1.0
    assert F.e8m0_decode(np.array([0]))[0] == 2.0 ** -127
    assert F.e8m0_decode(np.array([254]))[0] == 2.0 ** 127
    assert math.isnan(F.e8m0_decode(np.array([255]))[0])


@pytest.mark.parametrize("row", read_golden("e8m0_convert_cases.txt"), ids=lambda r: r[0])
def test_f32_pow2_to_e8m0_hand_cases(row):
    x = np.array([int(row[0], 16)], np.uint32).view(np.float32)
    b, ok = F.f32_pow2_to_e8m0(x)
    if row[1] == "reject":
        assert not ok[0]
    else:
        assert ok[0] and int(b[0]) == int(row[1])


def test_f32_pow2_to_e8m0_every_power():
    n = np.arange(-127, 128)
    x = np.ldexp(np.ones(n.size, np.float32), n).astype(np.float32)
    b, ok = F.f32_pow2_to_e8m0(x)
    assert ok.all()
    assert np.array_equal(b.astype(int), n + 127)
    # decode(encode(s)) == s
    assert np.array_equal(F.e8m0_decode(b), x.astype(np.float64))


@pytest.mark.parametrize("fmt,tdtype", [(F.OCP, torch.float8_e4m3fn), (F.FNUZ, torch.float8_e4m3fnuz)])
def test_e4m3_decode_table_matches_torch_cast(fmt, tdtype):
    """The decode table against a library routine: torch's float8 -> float32
    CPU cast of every one of the 256 codes (NaN codes compared as NaN)."""
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(tdtype).to(torch.float32).numpy().astype(np.float64)
    ours = F.e4m3_decode(np.arange(256, dtype=np.uint8), fmt)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])
    # signed zeros agree too
    assert np.array_equal(np.signbit(ours[~nan]), np.signbit(ref[~nan]))
