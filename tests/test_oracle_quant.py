"""Pins for the oracle's NVFP4 and MXFP8 block quantizers."""
import json
import os

import numpy as np
import pytest

from oracle import reference as R

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _num(v):
    return -0.0 if v == "-0" else float(v)


def test_nvfp4_worked_example():
    with open(os.path.join(GOLD, "nvfp4_worked_example.json")) as f:
        ex = json.load(f)
    b0 = [448.0 * _num(m) if m != "-0" else -0.0 for m in ex["block0_multipliers"]]
    row = np.array(b0 + [_num(v) for v in ex["block1_values"]], np.float32).reshape(1, 32)
    codes, sf, g = R.nvfp4_quantize(row, per_row=True)
    assert g[0] == np.float32(ex["expected_g"])
    assert list(sf[0]) == ex["expected_scales"]
    assert list(codes[0]) == ex["expected_codes"]
    # per-tensor scaling of a one-row tensor is the same computation
    c2, s2, g2 = R.nvfp4_quantize(row, per_row=False)
    assert np.array_equal(c2, codes) and np.array_equal(s2, sf) and g2[0] == g[0]


def _random_nvfp4_tensor(rng, rows, n, g):
    """Codes and scales whose dequantized tensor quantizes back to themselves:
    g is a power of two (so 6*g and sf*g are exact), every block holds a code of
    magnitude 6 (so its amax is 6*sf*g and s = sf exactly), and one block has
    sf = 448 (so the tensor amax is 2688*g and the global scale is g)."""
    nb = n // 16
    codes = rng.integers(0, 16, size=(rows, n)).astype(np.uint8)
    sf = rng.integers(1, 127, size=(rows, nb)).astype(np.uint8)
    for r in range(rows):
        for b in range(nb):
            codes[r, b * 16 + rng.integers(0, 16)] = 7 | (8 * rng.integers(0, 2))
    sf[0, 0] = 0x7E
    vals = np.array([[R.e2m1_decode(c) for c in row] for row in codes])
    scal = np.array([[R.e4m3_decode(s) for s in row] for row in sf])
    v = (vals * np.repeat(scal, 16, axis=1) * g).astype(np.float32)
    return v, codes, sf


@pytest.mark.parametrize("g", [1.0, 2.0 ** -10, 2.0 ** 6])
def test_nvfp4_roundtrip_per_tensor(g):
    rng = np.random.default_rng(3)
    v, codes, sf = _random_nvfp4_tensor(rng, 4, 64, g)
    c2, s2, g2 = R.nvfp4_quantize(v, per_row=False)
    assert g2[0] == np.float32(g)
    assert np.array_equal(s2, sf)
    assert np.array_equal(c2, codes)
    deq = R.nvfp4_dequant(c2, s2, g2, per_row=False)
    assert np.array_equal(deq, v.astype(np.float64))


def test_nvfp4_zero_tensor_and_zero_blocks():
    v = np.zeros((2, 32), np.float32)
    v[1, 3] = -0.0
    codes, sf, g = R.nvfp4_quantize(v, per_row=False)
    assert g[0] == 0 and not sf.any()
    assert codes[1, 3] == 8 and codes.sum() == 8
    v = np.zeros((1, 32), np.float32)
    v[0, 20] = 5.0
    v[0, 2] = -0.0
    codes, sf, g = R.nvfp4_quantize(v, per_row=True)
    assert sf[0, 0] == 0 and codes[0, 2] == 8 and codes[0, 20] == 7


def test_nvfp4_dequant_error_bound():
    """Every dequantized element is within half an E2M1 step of the input at its
    block's scale (the rounding bound), or saturated at 6*d."""
    rng = np.random.default_rng(4)
    v = rng.standard_normal((8, 256)).astype(np.float32)
    for per_row in (False, True):
        codes, sf, g = R.nvfp4_quantize(v, per_row)
        deq = R.nvfp4_dequant(codes, sf, g, per_row)
        gg = g[:, None].astype(np.float64) if per_row else float(g[0])
        d = np.array([[R.e4m3_decode(s) for s in row] for row in sf]) * gg
        d = np.repeat(d, 16, axis=1)
        err = np.abs(deq - v.astype(np.float64))
        # largest E2M1 gap is 2 (between 4 and 6): half of it, times d
        assert np.all(err <= 1.0 * d + 1e-12)
        # and relative to the block amax the error is small on average
        assert np.mean(err) / np.mean(np.abs(v)) < 0.15


def test_mxfp8_hand_blocks():
    with open(os.path.join(GOLD, "codec_cases.json")) as f:
        cases = json.load(f)["mxfp8_blocks"]
    for case in cases:
        vals = [_num(v) for v in case["values"]]
        row = np.zeros((1, 32), np.float32)
        row[0, :len(vals)] = vals
        codes, sc = R.mxfp8_quantize(row)
        assert sc[0, 0] == case["scale"], case["note"]
        assert list(codes[0, :len(vals)]) == case["codes"], case["note"]


def test_mxfp8_roundtrip():
    """E4M3 codes times 2^X quantize back to themselves when each block holds
    an element with exponent field 15 (|v| in [256, 448] * 2^X), which makes
    floor(log2(amax)) - 8 equal X."""
    rng = np.random.default_rng(5)
    rows, n = 3, 128
    codes = rng.integers(0, 256, size=(rows, n)).astype(np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0x12           # no NaN codes
    sc = rng.integers(100, 150, size=(rows, n // 32)).astype(np.uint8)
    for r in range(rows):
        for b in range(n // 32):
            codes[r, b * 32 + rng.integers(0, 32)] = 0x78 | rng.integers(0, 7) | (0x80 * rng.integers(0, 2))
    deq = R.mxfp8_dequant(codes, sc)
    c2, s2 = R.mxfp8_quantize(deq.astype(np.float32))
    assert np.array_equal(s2, sc) and np.array_equal(c2, codes)


def test_nvfp4_operation_order_non_power_of_two_g():
    """Pin of the fp32 operation order at a global scale that is not a power of
    two (g = fl32(1/2688)): the golden row was derived with exact rationals and
    hand-written IEEE binary32 rounding (tests/golden/make_nvfp4_order_case.py),
    independently of the oracle. Three plausible slips, s = (a_b/6)/g, d kept
    exact in fp64, and v * (1/d), each change a scale or code of this row, so
    the oracle matching the binding order rules them out."""
    import importlib.util
    spec = importlib.util.spec_from_file_location(
        "make_nvfp4_order_case", os.path.join(GOLD, "make_nvfp4_order_case.py"))
    mk = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mk)
    with open(os.path.join(GOLD, "nvfp4_order_nonpow2_g.json")) as f:
        ex = json.load(f)
    assert ex["orders"] == mk.derive(), "golden file out of date with its derivation"
    exp = ex["orders"]["reading8"]
    for order, alt in ex["orders"].items():
        if order != "reading8":
            assert alt["scales"] != exp["scales"] or alt["codes"] != exp["codes"], order
    row = np.array([float.fromhex(h) for h in ex["row_hex"]], np.float32).reshape(1, -1)
    g_exp = np.float32(float.fromhex(exp["g_hex"]))
    assert g_exp != np.float32(2.0 ** np.floor(np.log2(g_exp)))  # not a power of two
    for per_row in (True, False):
        codes, sf, g = R.nvfp4_quantize(row, per_row=per_row)
        assert g[0] == g_exp
        assert list(sf[0]) == exp["scales"]
        assert list(codes[0]) == exp["codes"]


def _load_golden_script(name):
    import importlib.util
    spec = importlib.util.spec_from_file_location(name, os.path.join(GOLD, name + ".py"))
    mk = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mk)
    return mk


def test_nvfp4_4o6_golden_row():
    """4-over-6 on a hand-derived row (exact rationals, no oracle call): the
    global scale amax/1536 and each block's choice between the max-to-6 and
    max-to-4 candidates (both occur)."""
    mk = _load_golden_script("make_nvfp4_4o6_case")
    with open(os.path.join(GOLD, "nvfp4_4o6_blocks.json")) as f:
        ex = json.load(f)
    assert ex["expected"] == mk.derive(), "golden file out of date with its derivation"
    assert set(ex["expected"]["row"]["picks"]) == {4, 6}
    # the tie row: both candidates exact, the tie goes to max-to-6 (scale 256
    # rather than 384 for the block of max 3, 2 rather than 3 for the other)
    assert ex["expected"]["tie_row"]["scales"] == [0x78, 0x40]
    for key, hexes in (("row", ex["row_hex"]), ("tie_row", ex["tie_row_hex"])):
        exp = ex["expected"][key]
        row = np.array([float.fromhex(h) for h in hexes], np.float32).reshape(1, -1)
        codes, sf, g = R.nvfp4_quantize(row, per_row=True, four_over_six=True)
        assert g[0] == np.float32(float.fromhex(exp["g_hex"])), key
        assert list(sf[0]) == exp["scales"], key
        assert list(codes[0]) == exp["codes"], key


def test_nvfp4_4o6_choice_matches_exact_argmin():
    """On seeded rows of several magnitudes, the oracle's 4-over-6 codes,
    scales and global scales equal the exact-rational derivation (every fp32
    step rounded by hand, the squared errors exact), i.e. each block keeps the
    candidate with the smaller error."""
    from fractions import Fraction as F
    mk = _load_golden_script("make_nvfp4_4o6_case")
    rng = np.random.default_rng(46)
    rows = (rng.standard_normal((6, 64)) * np.exp2(rng.integers(-8, 8, (6, 1)))).astype(np.float32)
    rows[2, 16:32] = 0.0                       # an all-zero block
    rows[3, :16] *= 1e-3                        # a block far below the row max
    codes, sf, g = R.nvfp4_quantize(rows, per_row=True, four_over_six=True)
    picks = []
    for r in range(rows.shape[0]):
        gg, scales, cc, pk = mk.quantize_row([F(float(v)) for v in rows[r]])
        assert g[r] == np.float32(float(gg)), r
        assert list(sf[r]) == scales, r
        assert list(codes[r]) == cc, r
        picks += pk
    assert 4 in picks and 6 in picks


def test_nvfp4_4o6_never_worse_than_max_to_6():
    """Per block, the 4-over-6 result's squared error is at most that of the
    usual max-to-6 quantization with the same global scale, and its result is
    one of the two candidates."""
    rng = np.random.default_rng(7)
    v = (rng.standard_normal((16, 128)) ** 3).astype(np.float32)
    c46, s46, g = R.nvfp4_quantize(v, per_row=True, four_over_six=True)
    L = R.lib()
    for r in range(v.shape[0]):
        c6 = np.empty(128, np.uint8)
        s6 = np.empty(8, np.uint8)
        L.orc_nvfp4_quantize(128, R._p(np.ascontiguousarray(v[r])), float(g[r]), R._p(c6), R._p(s6))
        d46 = R.nvfp4_dequant(c46[r:r + 1], s46[r:r + 1], g[r:r + 1], per_row=True)[0]
        d6 = R.nvfp4_dequant(c6[None], s6[None], g[r:r + 1], per_row=True)[0]
        e46 = ((d46 - v[r]) ** 2).reshape(8, 16).sum(1)
        e6 = ((d6 - v[r]) ** 2).reshape(8, 16).sum(1)
        assert np.all(e46 <= e6 * (1 + 1e-12))
        same6 = (s46[r] == s6)
        assert np.array_equal(c46[r].reshape(8, 16)[same6], c6.reshape(8, 16)[same6])


def test_nvfp4_4o6_roundtrip_on_max_to_4_grid():
    """Blocks whose values are code * sf * g with every code of magnitude at
    most 4 and a 4 in each block, g a power of two (the first block's scale
    384 puts the row max at 4 * 384 * 2^-9 = 3, so g = 3/1536 = 2^-9): the
    max-to-4 candidate is exact, so the dequantized row equals the input."""
    rng = np.random.default_rng(11)
    g = 2.0 ** -9
    for r in range(4):
        vals = []
        for b in range(6):
            sfv = 384.0 if b == 0 else R.e4m3_decode(int(rng.integers(1, 0x77)))
            codes = rng.choice([0, 1, 2, 3, 4, 5, 6, 8, 9, 10, 11, 12, 13, 14], size=16)
            codes[rng.integers(0, 16)] = 6 | (8 * int(rng.integers(0, 2)))   # code 6 = value 4
            vals += [R.e2m1_decode(int(c)) * sfv * g for c in codes]
        row = np.array(vals, np.float32)[None]
        assert np.float32(np.abs(row).max()) == np.float32(3.0)
        c, s, gg = R.nvfp4_quantize(row, per_row=True, four_over_six=True)
        assert gg[0] == np.float32(g)
        deq = R.nvfp4_dequant(c, s, gg, per_row=True)
        assert np.array_equal(deq, row.astype(np.float64))


def test_mxfp4_reblock_golden_blocks():
    """Re-blocking NVFP4 to MXFP4 on hand-chosen blocks (exact-rational
    derivation, no oracle call): round trip, saturation, exact ties, zero
    block with signed zeros."""
    mk = _load_golden_script("make_mxfp4_reblock_case")
    with open(os.path.join(GOLD, "mxfp4_reblock_blocks.json")) as f:
        ex = json.load(f)
    assert [[e["e8m0"], e["codes"]] for e in ex["expected"]] == mk.derive()
    for blk, exp in zip(ex["blocks"], ex["expected"]):
        codes = np.array(blk["codes"], np.uint8)[None]
        sf = np.array(blk["scales"], np.uint8)[None]
        mc, ms = R.mxfp4_reblock(codes, sf)
        assert int(ms[0, 0]) == exp["e8m0"]
        assert list(mc[0]) == exp["codes"]


def test_mxfp4_reblock_matches_exact_derivation_and_bounds():
    """Seeded NVFP4 rows re-blocked by the oracle equal the exact-rational
    derivation block for block; each re-blocked value is within half the E2M1
    gap at the block scale of the NVFP4 value (at most 2^X), or saturated
    (at most 2 * 2^X), and the dequantized row is code * 2^X exactly."""
    from fractions import Fraction as F
    mk = _load_golden_script("make_mxfp4_reblock_case")
    rng = np.random.default_rng(4)
    v = (rng.standard_normal((5, 128)) * np.exp2(rng.integers(-4, 4, (5, 1)))).astype(np.float32)
    codes, sf, g = R.nvfp4_quantize(v, per_row=True)
    mc, ms = R.mxfp4_reblock(codes, sf)
    for r in range(v.shape[0]):
        for b in range(v.shape[1] // 32):
            e8, cc = mk.reblock([int(c) for c in codes[r, 32 * b:32 * b + 32]],
                                [int(s) for s in sf[r, 2 * b:2 * b + 2]])
            assert int(ms[r, b]) == e8 and list(mc[r, 32 * b:32 * b + 32]) == cc
    w = R.nvfp4_dequant(codes, sf, np.ones(5, np.float32), per_row=True)   # local values
    rb = R.mxfp4_dequant(mc, ms)
    scale = np.repeat(np.exp2(ms.astype(np.float64) - 127), 32, axis=1)
    err = np.abs(rb - w)
    assert np.all(err <= 2.0 * scale)
    assert np.all(err[np.abs(w) <= 6.0 * scale] <= 1.0 * scale[np.abs(w) <= 6.0 * scale])


def test_mxfp4_reblock_round_trip_on_power_of_two_scales():
    """When both halves of every 32-block share one power-of-two E4M3 scale,
    NVFP4 values are already MXFP4 values: re-blocking keeps every value."""
    rng = np.random.default_rng(9)
    codes = rng.integers(0, 16, size=(3, 96)).astype(np.uint8)
    sf = np.empty((3, 6), np.uint8)
    for r in range(3):
        for b in range(3):
            e = int(rng.integers(1, 15))                # exponent field, mantissa 0
            sf[r, 2 * b] = sf[r, 2 * b + 1] = e << 3
    w = R.nvfp4_dequant(codes, sf, np.ones(3, np.float32), per_row=True)
    mc, ms = R.mxfp4_reblock(codes, sf)
    assert np.array_equal(R.mxfp4_dequant(mc, ms), w)
