"""CPU checks of the parity helpers themselves: the MXFP8 FC2-input check
accepts the oracle's own quantization and rejects planted mistakes."""
import numpy as np
import pytest

from oracle import reference as R
from tests.helpers import check_a2_mxfp8


def _fake_ref(rows=6, cols=96, seed=3):
    rng = np.random.default_rng(seed)
    a = rng.standard_normal((rows, cols)) * np.exp2(rng.integers(-6, 6, (rows, 1)))
    a[1, :32] = 0.0                                 # an all-zero block
    a[2, 5] = 450.0 * 2.0 ** -8 * np.abs(a[2]).max()  # a large element in the row
    return {"a": a, "a_routes": np.arange(rows), "route_to_row": np.arange(rows)}


def test_mxfp8_check_accepts_oracle_quantization():
    ref = _fake_ref()
    codes, scales = R.mxfp8_quantize(ref["a"].astype(np.float32))
    check_a2_mxfp8(codes, scales, ref, "oracle")


def test_mxfp8_check_rejects_wrong_code():
    ref = _fake_ref()
    codes, scales = R.mxfp8_quantize(ref["a"].astype(np.float32))
    c = codes.copy()
    i = np.unravel_index(np.argmax(np.abs(ref["a"][3])), ref["a"][3].shape)[0]
    c[3, i] = (int(c[3, i]) & 0x80) | max((int(c[3, i]) & 0x7F) - 1, 0)  # one step toward zero
    with pytest.raises(AssertionError):
        check_a2_mxfp8(c, scales, ref, "planted code")


def test_mxfp8_check_rejects_wrong_scale():
    ref = _fake_ref()
    codes, scales = R.mxfp8_quantize(ref["a"].astype(np.float32))
    s = scales.copy()
    s[4, 1] += 1
    with pytest.raises(AssertionError):
        check_a2_mxfp8(codes, s, ref, "planted scale")


def test_mxfp8_check_rejects_swapped_columns():
    ref = _fake_ref()
    codes, scales = R.mxfp8_quantize(ref["a"].astype(np.float32))
    c = codes.copy()
    c[0, 0:16], c[0, 16:32] = codes[0, 16:32], codes[0, 0:16]
    with pytest.raises(AssertionError):
        check_a2_mxfp8(c, scales, ref, "planted swap")
