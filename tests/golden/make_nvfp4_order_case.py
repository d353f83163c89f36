"""Derives tests/golden/nvfp4_order_nonpow2_g.json with exact rational arithmetic.

Independent of the oracle: every quantity is a Python Fraction, and each fp32
operation of the NVFP4 block quantizer is written out as "exact result, then
IEEE 754 binary32 round-to-nearest-even" (fl32 below). The element formats come
from the OCP Microscaling Formats (MX) v1.0 definitions (E2M1 magnitudes 0, 0.5,
1, 1.5, 2, 3, 4, 6; E4M3 "FN": bias 7, 3 mantissa bits, largest finite 448),
rounded to nearest with ties to the even code and saturating.

The row has one global scale from its amax of 1.0, so g = fl32(1 / 2688) is
not a power of two and the order of the fp32 operations decides some codes.
Four orders are derived:
  reading8           s = a_b / (6 g), sf = E4M3(s), d = sf g, code = E2M1(v / d)
                     (each operation one fp32 rounding: the binding order)
  scale_div6_then_g  s = (a_b / 6) / g, the rest as reading8
  d_fp64             d = sf g kept exact (no fp32 rounding), code = E2M1(v / d)
                     with the quotient exact as well
  recip_mul          code = E2M1(v * fl32(1 / d))
The test checks that the oracle reproduces "reading8" and that every other
order changes at least one scale or code of this row.

Run: python tests/golden/make_nvfp4_order_case.py  (rewrites the JSON)
"""
from __future__ import annotations

import json
import os
from fractions import Fraction as F

HERE = os.path.dirname(os.path.abspath(__file__))
OUT = os.path.join(HERE, "nvfp4_order_nonpow2_g.json")


def fl32(q: F) -> F:
    """IEEE 754 binary32 round-to-nearest-even of an exact rational (finite
    results only; the values here are far from overflow)."""
    if q == 0:
        return F(0)
    sign = -1 if q < 0 else 1
    a = abs(q)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    while F(2) ** e > a:
        e -= 1
    while F(2) ** (e + 1) <= a:
        e += 1
    quantum = F(2) ** (max(e, -126) - 23)      # 24 significant bits; subnormal below 2^-126
    m = a / quantum
    lo = m.numerator // m.denominator
    rem = m - lo
    if rem > F(1, 2) or (rem == F(1, 2) and lo % 2 == 1):
        lo += 1
    return sign * lo * quantum


E2M1_MAG = [F(0), F(1, 2), F(1), F(3, 2), F(2), F(3), F(4), F(6)]


def e4m3_mag(c: int) -> F:
    e, m = (c >> 3) & 15, c & 7
    return F(m, 512) if e == 0 else (1 + F(m, 8)) * F(2) ** (e - 7)


E4M3_MAG = [e4m3_mag(c) for c in range(127)]          # 0x7F is NaN


def nearest_code(a: F, mags) -> int:
    """Index of the magnitude nearest to a (a >= 0), ties to the even index,
    saturating at the largest."""
    if a >= mags[-1]:
        return len(mags) - 1
    lo = max(i for i, v in enumerate(mags) if v <= a)
    if lo == len(mags) - 1:
        return lo
    below, above = a - mags[lo], mags[lo + 1] - a
    if above < below or (above == below and (lo + 1) % 2 == 0):
        return lo + 1
    return lo


def e2m1(u: F, negative: bool) -> int:
    return (8 if negative else 0) | nearest_code(abs(u), E2M1_MAG)


def e4m3(s: F) -> int:
    return nearest_code(abs(s), E4M3_MAG)


def quantize(row, order: str):
    """row: list of Fractions (fp32 values). Returns (g, scale codes, E2M1 codes)."""
    amax = max(abs(v) for v in row)
    g = fl32(amax / 2688)
    scales, codes = [], []
    for b in range(len(row) // 16):
        blk = row[b * 16:(b + 1) * 16]
        ab = max(abs(v) for v in blk)
        if order == "scale_div6_then_g":
            s = fl32(fl32(ab / 6) / g)
        else:
            s = fl32(ab / fl32(6 * g))
        sf = e4m3(s)
        scales.append(sf)
        if order == "d_fp64":
            d = E4M3_MAG[sf] * g
        else:
            d = fl32(E4M3_MAG[sf] * g)
        for v in blk:
            if order == "d_fp64":
                u = v / d
            elif order == "recip_mul":
                u = fl32(v * fl32(1 / d))
            else:
                u = fl32(v / d)
            codes.append(e2m1(u, v < 0))
    return g, scales, codes


# One row of 32 fp32 values (exact binary32 numbers written as hex floats).
# Block 0 holds the row amax 1.0 (so g = fl32(1/2688)) and ordinary values.
# Block 1: its largest magnitude 0x1.c92494p-3 ~ 0.2232 puts a_b / (6 g) within
# an fp32 rounding of the E4M3 midpoint between codes 108 and 109 (the two
# scale orders round it to different sides); 0x1.24924ap-7 and 0x1.b6db6ep-6
# lie next to the E2M1 midpoints 0.25 and 0.75 of that block's decode scale,
# where the fp32 quotient and the exact quotient round differently;
# 0x1.b6db6ep-6 and 0x1.6db6dep-5 also round differently under the
# reciprocal-multiply form.
ROW_HEX = [
    "0x1.0p+0", "-0x1.8p-1", "0x1.0p-1", "-0x1.0p-2", "0x1.5p-3", "0x1.2p-4", "-0x1.0p-5", "0x0.0p+0",
    "0x1.99999ap-2", "-0x1.333334p-3", "0x1.e00000p-2", "-0x1.c00000p-1", "0x1.0p-7", "-0x1.4p-1",
    "0x1.7p-2", "0x1.1p-6",
    "0x1.c92494p-3", "0x1.24924ap-7", "0x1.b6db6ep-6", "0x1.6db6dep-5", "-0x1.24924ap-7",
    "-0x1.b6db6ep-6", "0x1.0p-4", "-0x1.8p-4", "0x1.4p-5", "0x1.0p-3", "-0x1.6p-3", "0x0.0p+0",
    "0x1.0p-8", "-0x1.2p-4", "0x1.9p-4", "-0x1.92p-3",
]

ORDERS = ["reading8", "scale_div6_then_g", "d_fp64", "recip_mul"]


def row_fractions():
    return [F(float.fromhex(h)) for h in ROW_HEX]


def derive():
    row = row_fractions()
    out = {}
    for order in ORDERS:
        g, scales, codes = quantize(row, order)
        out[order] = {"g_hex": float(g).hex(), "scales": scales, "codes": codes}
    return out


def main():
    doc = {
        "source": "Derived by tests/golden/make_nvfp4_order_case.py with exact rationals "
                  "(fractions.Fraction) and IEEE 754 binary32 round-to-nearest-even written "
                  "out by hand; NVFP4 convention (E2M1 elements, E4M3 scale per 16, FP32 "
                  "global scale amax/(6*448)) and OCP MX v1.0 element formats. The binding "
                  "order is reading8; the other orders are plausible slips that this row "
                  "tells apart.",
        "row_hex": ROW_HEX,
        "orders": derive(),
    }
    with open(OUT, "w") as f:
        json.dump(doc, f, indent=1)
        f.write("\n")
    print(OUT)


if __name__ == "__main__":
    main()
