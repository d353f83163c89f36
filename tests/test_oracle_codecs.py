"""Pins for the oracle's element codecs (E2M1, E4M3, E8M0, bf16).

Pinned against hand-derived tables from the OCP MX v1.0 element definitions
(tests/golden/codec_cases.json) and against torch's own CPU casts where torch
implements the same format (float8_e4m3fn, bfloat16).
"""
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import reference as R

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _num(v):
    return -0.0 if v == "-0" else float(v)


@pytest.fixture(scope="module")
def cases():
    with open(os.path.join(GOLD, "codec_cases.json")) as f:
        return json.load(f)


def test_e2m1_decode_table(cases):
    for code, want in enumerate(cases["e2m1_decode"]):
        got = R.e2m1_decode(code)
        assert got == _num(want) and math.copysign(1, got) == math.copysign(1, _num(want))


def test_e2m1_roundtrip_all_codes():
    for code in range(16):
        assert R.e2m1_encode(R.e2m1_decode(code)) == code


def test_e2m1_ties_and_saturation(cases):
    for u, code in cases["e2m1_encode"]:
        assert R.e2m1_encode(_num(u)) == code, u


def test_e4m3_roundtrip_all_finite_codes():
    n = 0
    for code in range(256):
        if code & 0x7F == 0x7F:
            assert math.isnan(R.e4m3_decode(code))
            continue
        assert R.e4m3_encode(R.e4m3_decode(code)) == code
        n += 1
    assert n == 254


def test_e4m3_monotone():
    vals = [R.e4m3_decode(c) for c in range(127)]
    assert all(b > a for a, b in zip(vals, vals[1:]))
    assert vals[-1] == 448.0 and vals[1] == 2.0 ** -9


def test_e4m3_hand_cases(cases):
    for u, code in cases["e4m3_encode"]:
        assert R.e4m3_encode(u) == code, u


def test_e4m3_matches_torch_cast():
    """torch.float8_e4m3fn's CPU cast is RNE onto the same grid; compare on
    values below 464 (above, torch returns NaN where the method saturates)."""
    rng = np.random.default_rng(1)
    mags = np.concatenate([
        np.exp2(rng.uniform(-12, np.log2(463.9), 4000)),
        rng.uniform(0, 2.0 ** -6, 1000),          # subnormal range
    ]).astype(np.float32)
    # exact midpoints between adjacent codes (ties)
    grid = np.array([R.e4m3_decode(c) for c in range(127)])
    mids = ((grid[:-1] + grid[1:]) / 2).astype(np.float32)
    vals = np.concatenate([mags, -mags, mids, -mids])
    want = torch.from_numpy(vals).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = np.array([R.e4m3_encode(float(v)) for v in vals], np.uint8)
    assert np.array_equal(got, want)


def test_e8m0_decode(cases):
    for code, want in cases["e8m0_decode"]:
        assert R.e8m0_decode(code) == want
    assert math.isnan(R.e8m0_decode(255))


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(2)
    v = (rng.standard_normal(20000) * np.exp2(rng.uniform(-20, 20, 20000))).astype(np.float32)
    # exact ties: bf16 value plus half an ulp
    base = torch.from_numpy(v[:2000]).to(torch.bfloat16).to(torch.float32).numpy()
    ties = (base.view(np.uint32) | np.uint32(0x8000)).view(np.float32)
    v = np.concatenate([v, ties])
    want = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = R.f32_to_bf16_bits(v)
    assert np.array_equal(got, want)
