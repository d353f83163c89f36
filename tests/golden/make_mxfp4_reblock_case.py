"""Derives tests/golden/mxfp4_reblock_blocks.json: NVFP4 blocks re-blocked to
MXFP4, with exact rational arithmetic, independently of the oracle.

Re-blocking (the other NVFP4 GEMM option: FP4 matrix units take one E8M0
scale per 32 elements, NVFP4 carries one E4M3 scale per 16): each 32-element
block's local NVFP4 values w = E2M1(code) * E4M3(sf) are re-quantized by the
OCP MX v1.0 rule for E2M1 elements, shared exponent X = floor(log2 max|w|) - 2
(2 = exponent of E2M1's largest normal, 6 = 1.5 * 2^2), clamped to
[-127, 127], element codes E2M1_RNE(w / 2^X) with ties to the even code and
saturation at 6, the sign kept (also for zeros); an all-zero block gets
X = -127. The global scale stays outside the block.

Run: python tests/golden/make_mxfp4_reblock_case.py  (rewrites the JSON)
"""
from __future__ import annotations

import importlib.util
import json
import os
from fractions import Fraction as F

HERE = os.path.dirname(os.path.abspath(__file__))
OUT = os.path.join(HERE, "mxfp4_reblock_blocks.json")

_spec = importlib.util.spec_from_file_location("make_nvfp4_order_case",
                                               os.path.join(HERE, "make_nvfp4_order_case.py"))
_mk = importlib.util.module_from_spec(_spec)
_spec.loader.exec_module(_mk)
e2m1, E2M1_MAG, E4M3_MAG = _mk.e2m1, _mk.E2M1_MAG, _mk.E4M3_MAG


def floor_log2(a: F) -> int:
    e = a.numerator.bit_length() - a.denominator.bit_length()
    while F(2) ** e > a:
        e -= 1
    while F(2) ** (e + 1) <= a:
        e += 1
    return e


def reblock(codes, scales):
    """codes: 32 NVFP4 codes (0..15), scales: 2 E4M3 codes. Returns (E8M0 code,
    32 MXFP4 codes)."""
    w = [E2M1_MAG[c & 7] * E4M3_MAG[scales[i // 16]] * (-1 if c & 8 else 1)
         for i, c in enumerate(codes)]
    amax = max(abs(v) for v in w)
    if amax == 0:
        return 0, [c & 8 for c in codes]
    X = max(-127, min(127, floor_log2(amax) - 2))
    out = []
    for v, c in zip(w, codes):
        out.append(e2m1(v / F(2) ** X, bool(c & 8)))
    return X + 127, out


# Blocks of 32 NVFP4 codes with the E4M3 scale codes of their two halves
# (scale values in parentheses); u = |w| / 2^X is what E2M1 rounds:
#  0: 0x38, 0x38 (1, 1): max 4, X = 0, every value already on the MXFP4 grid
#     (nothing changes);
#  1: 0x42, 0x38 (2.5, 1): max 15, X = 1; u = 7.5 saturates to 6, and exact
#     ties u = 0.25, 0.75, 1.25, 2.5, 5 go to the even neighbour;
#  2: 0x3C, 0x3A (1.5, 1.25): max 9, X = 1; ties u = 0.75, 1.25, 2.5;
#  3: 0x3F, 0x30 (1.875, 0.5): max 11.25, X = 1; ties u = 0.25, 0.75;
#  4: 0x4F, 0x48 (7.5, 4): max 45, X = 3; ties u = 0.25, 0.75;
#  5: all zeros of both signs: X = -127 (E8M0 code 0), sign-only codes.
BLOCKS = [
    ([0, 1, 2, 3, 4, 5, 6, 9, 10, 11, 12, 13, 14, 8, 0, 2,
      6, 14, 1, 9, 3, 11, 5, 13, 0, 8, 2, 10, 4, 12, 6, 7 - 1], [0x38, 0x38]),
    ([7, 3, 1, 9, 15, 11, 0, 8, 2, 10, 4, 12, 5, 13, 6, 14,
      1, 9, 1, 9, 0, 8, 2, 3, 4, 5, 6, 7, 10, 11, 12, 13], [0x42, 0x38]),
    ([7, 5, 15, 13, 3, 11, 2, 10, 1, 9, 4, 12, 6, 14, 0, 8,
      2, 10, 5, 13, 7, 15, 1, 9, 3, 11, 4, 12, 6, 14, 0, 8], [0x3C, 0x3A]),
    ([7, 6, 5, 4, 3, 2, 1, 0, 15, 14, 13, 12, 11, 10, 9, 8,
      7, 6, 5, 4, 3, 2, 1, 0, 15, 14, 13, 12, 11, 10, 9, 8], [0x3F, 0x30]),
    ([7, 6, 5, 4, 3, 2, 1, 0, 15, 14, 13, 12, 11, 10, 9, 8,
      7, 6, 5, 4, 3, 2, 1, 0, 15, 14, 13, 12, 11, 10, 9, 8], [0x4F, 0x48]),
    ([0, 8] * 16, [0x38, 0x00]),
]


def derive():
    return [list(reblock(c, s)) for c, s in BLOCKS]


def main():
    doc = {
        "source": "Derived by tests/golden/make_mxfp4_reblock_case.py with exact rationals "
                  "(fractions.Fraction): NVFP4 (E2M1 codes, E4M3 scale per 16) re-blocked to "
                  "MXFP4 (E2M1 codes, E8M0 scale per 32) by the OCP MX v1.0 rule, "
                  "X = floor(log2 max) - 2, E2M1 round to nearest even with saturation.",
        "blocks": [{"codes": c, "scales": s} for c, s in BLOCKS],
        "expected": [{"e8m0": e, "codes": c} for e, c in derive()],
    }
    with open(OUT, "w") as f:
        json.dump(doc, f, indent=1)
        f.write("\n")
    print(OUT)


if __name__ == "__main__":
    main()
