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
