"""Writes tests/golden/rope_rounding_cases.txt: inverse-RoPE inputs whose BF16
result depends on the rotation's sum being rounded to fp32 first.

The rotation of a pair (x, y) by -pos*omega is x' = x*c + y*s, y' = y*c - x*s,
computed in fp32 with every operation rounded and the result then rounded to
BF16 (nearest, ties to even).  All four operands are BF16 values (8 significant
bits), so each product has at most 16 significant bits and is exact in fp32: a
fused multiply-add and separately rounded products give the same fp32 sum.
The only rounding before the final one is the fp32 rounding of the sum.  It
changes the BF16 result exactly when the exact sum lies within half an fp32
ulp of a BF16 midpoint (but not on it): fp32 then rounds onto the midpoint and
the tie goes to the even BF16 neighbour, while the exact sum would have gone to
the nearer one.  An oracle that rotated in fp64 (or in exact arithmetic) gives
the other BF16 value on every case in the file.

Candidates are found by a vectorised fp64 search (products and sums of the
magnitudes searched are exact in fp64); every case written is then re-derived
in exact rational arithmetic (fractions.Fraction) with the rounding rules
written out below, and the derivation is stored beside it.  The cos/sin
entries are the BF16 rotary tables of the tests (omega_i = 10000^(-2i/64),
angle in fp64, cos/sin -> fp32 -> BF16), read at the stated (pos, i).

Run from the repository root:  python tests/golden/make_rope_rounding_cases.py
"""

import os
import sys
from fractions import Fraction

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)

import workloads  # noqa: E402  (seeded inputs and the rotary tables only)

OUT = os.path.join(HERE, "rope_rounding_cases.txt")
TABLE_AT = [(1, 0), (1, 7), (2, 7), (3, 7)]   # (pos, pair) entries searched


def bf16_value(bits):
    """Exact value of a finite BF16 pattern."""
    sign = -1 if bits & 0x8000 else 1
    e = (bits >> 7) & 0xFF
    m = bits & 0x7F
    if e == 0:
        return sign * Fraction(m, 1 << 7) * Fraction(1, 1 << 126)
    return sign * (1 + Fraction(m, 128)) * (Fraction(2) ** (e - 127))


def round_rne(v, p):
    """Nearest value with p significant bits (normal range), ties to even."""
    if v == 0:
        return Fraction(0)
    sign = -1 if v < 0 else 1
    a = abs(v)
    e = 0
    while a >= 2:
        a /= 2
        e += 1
    while a < 1:
        a *= 2
        e -= 1
    q = Fraction(2) ** (e - p + 1)                # spacing of p-bit values at 2^e
    n = abs(v) / q
    lo = n.numerator // n.denominator
    rem = n - lo
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and lo % 2 == 1):
        lo += 1
    return sign * lo * q


def f32(v):
    return round_rne(v, 24)


def bf16(v):
    return round_rne(v, 8)


def bf16_bits(v):
    """Pattern of a value that is exactly a BF16 normal number."""
    x = np.array([float(v)], dtype=np.float32)
    assert Fraction(float(x[0])) == v
    return int(x.view(np.uint32)[0] >> 16)


def hexf(v):
    return float(v).hex()


def search():
    with np.errstate(invalid="ignore"):
        vals = (np.arange(0x10000, dtype=np.uint32) << 16).view(np.float32).astype(np.float64)
    bits = np.arange(0x10000, dtype=np.uint32)
    xsel = (vals >= 1) & (vals < 2)
    ysel = np.isfinite(vals) & (np.abs(vals) >= 2.0 ** -12) & (np.abs(vals) < 2.0 ** -1)
    xb, yb = bits[xsel], bits[ysel]
    X, Y = np.meshgrid(vals[xsel], vals[ysel], indexing="ij")
    XB, YB = np.meshgrid(xb, yb, indexing="ij")

    def bf16_64(S):
        _, e = np.frexp(S)
        q = np.ldexp(1.0, e - 8)
        return np.rint(S / q) * q

    cos, sin = workloads.rope_tables(rows=8)
    found = []
    for pos, i in TABLE_AT:
        cb, sb = int(cos[pos, i]), int(sin[pos, i])
        c, s = float(bf16_value(cb)), float(bf16_value(sb))
        for which, S in (("x", X * c + Y * s), ("y", Y * c - X * s)):
            d = np.argwhere(bf16_64(S) != bf16_64(S.astype(np.float32).astype(np.float64)))
            if len(d):
                # the candidate with the largest |y| (the least extreme inputs)
                k = d[np.argmax(np.abs(Y[tuple(d.T)]))]
                found.append((pos, i, cb, sb, int(XB[tuple(k)]), int(YB[tuple(k)]), which))
    return found


def derive(pos, i, cb, sb, xb, yb, which):
    c, s, x, y = bf16_value(cb), bf16_value(sb), bf16_value(xb), bf16_value(yb)
    xc, ys, yc, xs = x * c, y * s, y * c, x * s
    for p in (xc, ys, yc, xs):
        assert f32(p) == p                         # every product is exact in fp32
    sx, sy = xc + ys, yc - xs
    out = {}
    for name, S in (("x", sx), ("y", sy)):
        out[name] = (S, f32(S), bf16(f32(S)), bf16(S))
    S, S32, dbl, single = out[which]
    assert dbl != single, "not a double-rounding case"
    mid = (dbl + single) / 2
    assert S32 == mid and S != mid                 # fp32 lands on the BF16 midpoint
    text = (f"{which}' exact = {hexf(S)}; fp32 -> {hexf(S32)}, the midpoint of BF16 "
            f"{hexf(min(dbl, single))} and {hexf(max(dbl, single))}; tie to even -> {hexf(dbl)}; "
            f"rounding the exact sum once gives {hexf(single)}")
    return (bf16_bits(out["x"][2]), bf16_bits(out["y"][2]), bf16_bits(out["x"][3]),
            bf16_bits(out["y"][3]), text)


def main():
    rows = []
    for case in search():
        pos, i, cb, sb, xb, yb, which = case
        ox, oy, fx, fy, text = derive(*case)
        rows.append(f"{pos:<4d} {i:<3d} 0x{cb:04X} 0x{sb:04X} 0x{xb:04X} 0x{yb:04X} 0x{ox:04X} 0x{oy:04X} "
                    f"0x{fx:04X} 0x{fy:04X}  {text}")
    with open(OUT, "w") as f:
        f.write(__doc__.split("\n\n")[1].replace("\n", "\n# ").join(["# ", "\n"]))
        f.write("#\n# Written by tests/golden/make_rope_rounding_cases.py (exact rational derivation).\n"
                "# Columns: pos, pair i, cos bits, sin bits, x bits, y bits, then the BF16 result\n"
                "# (x', y') of the fp32 rotation, then (x', y') of an exact rotation rounded once.\n"
                "#\n")
        f.write("\n".join(rows) + "\n")
    print(f"wrote {len(rows)} cases to {OUT}")


if __name__ == "__main__":
    main()
