"""Derives tests/golden/nvfp4_4o6_blocks.json: the 4-over-6 NVFP4 block choice
with exact rational arithmetic, independently of the oracle.

Reading of the 4-over-6 per-token activation contract (FlashInfer PR #4366,
"Performance benchmark", which names it only by its environment switches):
global scale g = fl32(amax / 1536) (6 * 256: the usual block scales stay at or
below 256, so scales 1.5x larger still fit E4M3); each 16-block is quantized
twice with the usual fp32 operation order, once with the block max mapped to
the E2M1 maximum 6 and once to 4; the candidate with the smaller sum of
squared errors sum_i (v_i - code_i * d)^2 is kept, ties going to the max-to-6
candidate. Here the errors are exact rationals (the oracle accumulates them in
fp64; the blocks below are far from a tie).

Each fp32 operation is written as "exact result, then IEEE binary32
round-to-nearest-even" with the hand-written fl32 of make_nvfp4_order_case.py.

Run: python tests/golden/make_nvfp4_4o6_case.py  (rewrites the JSON)
"""
from __future__ import annotations

import importlib.util
import json
import os
from fractions import Fraction as F

HERE = os.path.dirname(os.path.abspath(__file__))
OUT = os.path.join(HERE, "nvfp4_4o6_blocks.json")

_spec = importlib.util.spec_from_file_location("make_nvfp4_order_case",
                                               os.path.join(HERE, "make_nvfp4_order_case.py"))
_mk = importlib.util.module_from_spec(_spec)
_spec.loader.exec_module(_mk)
fl32, e2m1, e4m3, E2M1_MAG, E4M3_MAG = _mk.fl32, _mk.e2m1, _mk.e4m3, _mk.E2M1_MAG, _mk.E4M3_MAG


def candidate(blk, g: F, top: int):
    """(scale code, codes, exact squared error) of one block, max mapped to top."""
    ab = max(abs(v) for v in blk)
    s = fl32(ab / fl32(top * g))
    sf = e4m3(s)
    d = fl32(E4M3_MAG[sf] * g)
    codes, err = [], F(0)
    for v in blk:
        if d == 0:
            c = 8 if v < 0 else 0
        else:
            c = e2m1(fl32(v / d), v < 0)
        codes.append(c)
        val = E2M1_MAG[c & 7] * d * (-1 if c & 8 else 1)
        err += (v - val) ** 2
    return sf, codes, err


def quantize_row(row):
    amax = max(abs(v) for v in row)
    g = fl32(amax / 1536)
    scales, codes, picks = [], [], []
    for b in range(len(row) // 16):
        blk = row[b * 16:(b + 1) * 16]
        if g == 0:
            scales.append(0)
            codes += [8 if v < 0 else 0 for v in blk]
            picks.append(6)
            continue
        s6, c6, e6 = candidate(blk, g, 6)
        s4, c4, e4 = candidate(blk, g, 4)
        four = e4 < e6
        scales.append(s4 if four else s6)
        codes += c4 if four else c6
        picks.append(4 if four else 6)
    return g, scales, codes, picks


# Three 16-blocks of one row (exact binary32 values as hex floats):
#  block 0: the row maximum 1.0 with values near 1/4-multiples of it, where
#           the finer grid of the max-to-4 candidate wins (pick 4);
#  block 1: maximum 0.625 with values where the max-to-6 grid wins (pick 6);
#  block 2: the row maximum 1.0 again among Gaussian-like values (pick 4).
ROW_HEX = [
    "0x1.0p+0", "-0x1.8p-1", "0x1.0p-1", "0x1.0p-2", "0x1.8p-3", "0x1.0p-3", "-0x1.0p-4", "0x0.0p+0",
    "0x1.0p-1", "-0x1.0p-2", "0x1.8p-2", "0x1.8p-1", "-0x1.0p+0", "0x1.0p-3", "0x1.0p-1", "0x1.8p-3",
    "0x1.8p-2", "0x1.0p-2", "0x1.0p-3", "0x1.4p-1", "-0x1.8p-2", "0x1.0p-3", "0x1.0p-4", "0x0.0p+0",
    "0x1.8p-3", "-0x1.0p-2", "0x1.0p-2", "0x1.0p-4", "-0x1.0p-3", "0x1.8p-3", "0x1.0p-3", "0x1.8p-4",
    "0x1.0p+0", "-0x1.6a09e6p-1", "0x1.333334p-2", "-0x1.99999ap-3", "0x1.d1745ep-2",
    "0x1.24924ap-3", "-0x1.c71c72p-2", "0x1.745d18p-4", "0x1.b6db6ep-1", "-0x1.0624dep-5",
    "0x1.47ae14p-2", "-0x1.eb851ep-3", "0x1.1eb852p-1", "0x1.4fdf3cp-6", "-0x1.f9db22p-2",
    "0x1.a5e354p-3",
]


# A row of two exact ties: row max 3 gives g = 3/1536 = 2^-9; block 0 (max 3)
# and block 1 (values +-12, +-6 and 0 times 2^-9) lie exactly on both the
# max-to-6 grid (scales 256 and 2) and the max-to-4 grid (scales 384 and 3),
# so both candidates have zero error and the tie rule decides (max-to-6).
TIE_ROW_HEX = [
    "0x1.8p+1", "0x0.0p+0", "-0x1.8p+0", "0x1.8p+1", "0x0.0p+0", "0x1.8p+0", "-0x1.8p+1", "0x0.0p+0",
    "0x0.0p+0", "0x1.8p+0", "0x0.0p+0", "0x0.0p+0", "-0x1.8p+0", "0x0.0p+0", "0x1.8p+1", "0x0.0p+0",
    "0x1.8p-6", "-0x1.8p-6", "0x1.8p-7", "0x0.0p+0", "0x1.8p-6", "-0x1.8p-7", "0x0.0p+0", "0x1.8p-6",
    "0x1.8p-7", "0x1.8p-6", "-0x1.8p-6", "0x0.0p+0", "0x1.8p-7", "0x1.8p-6", "0x0.0p+0", "-0x1.8p-7",
]


def row_fractions(hexes=None):
    return [F(float.fromhex(h)) for h in (ROW_HEX if hexes is None else hexes)]


def derive():
    out = {}
    for key, hexes in (("row", ROW_HEX), ("tie_row", TIE_ROW_HEX)):
        g, scales, codes, picks = quantize_row(row_fractions(hexes))
        out[key] = {"g_hex": float(g).hex(), "scales": scales, "codes": codes, "picks": picks}
    return out


def main():
    doc = {
        "source": "Derived by tests/golden/make_nvfp4_4o6_case.py with exact rationals "
                  "(fractions.Fraction) and hand-written IEEE binary32 rounding: the 4-over-6 "
                  "NVFP4 block choice (global scale amax/(6*256), per block the max-to-6 or the "
                  "max-to-4 candidate, whichever has the smaller exact sum of squared errors, "
                  "ties to max-to-6). OCP MX v1.0 element formats.",
        "row_hex": ROW_HEX,
        "tie_row_hex": TIE_ROW_HEX,
        "expected": derive(),
    }
    with open(OUT, "w") as f:
        json.dump(doc, f, indent=1)
        f.write("\n")
    print(OUT)


if __name__ == "__main__":
    main()
