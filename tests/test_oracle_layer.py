"""Pins for the oracle's whole-layer forward.

Checks that do not reuse the oracle's own orchestration:
  - brute-force dense evaluation: every expert on every token with numpy
    matrix products, then selecting the routed pairs;
  - top-K = E with uniform weights equals the mean of the dense experts;
  - K = 1 reduces to the single chosen expert's output;
  - router-weight placement (FlashInfer PR #4366, "Description"): input- and
    output-side agree up to rounding when the FC2 input is not quantized
    (linearity of FC2), and bit-exactly in every mode when the weights are a
    power of two;
  - the pre-activation variant PR #4366 ("Existing SM120 status") criticises is
    detected: for ReLU2 with p = 1/2 it gives exactly half the correct result;
  - closed forms of the activations and an exact-rational spot check of FC1.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import reference as R
from synth_inputs import make_expert_weights, make_logits, make_x

MODES = ["w4a4_tensor", "w4a4_token", "w4a16", "mxfp8", "w4a4_token_4o6", "w4a4_token_mxfp4"]


def _setup(T=16, H=256, I=128, E=8, mode="w4a4_tensor", act="swiglu", seed=0, logits="normal"):
    N1 = 2 * I if act == "swiglu" else I
    x = make_x(seed, T, H).view(torch.int16).numpy().view(np.uint16)
    lg = make_logits(seed, T, E, logits).numpy()
    w1, w2 = make_expert_weights(seed, E, N1, H, I)
    w1, w2 = w1.numpy(), w2.numpy()
    W = R.QuantWeights(R.weight_format(mode), E, H, I, act, lambda e: (w1[e], w2[e]))
    return x, lg, W


def _dense(x, lg, W, K, mode, act, on_input):
    """Every expert on every token (dense matrix products), then pick routes."""
    T = x.shape[0]
    E, I = W.E, W.I
    ids, p = R.route(lg, K)
    xq = R.quantize_x(x, mode)
    X = np.stack([xq["deq"](t) for t in range(T)])
    W.ensure(range(E))
    deq = [W.dequant(e) for e in range(E)]
    acts = []
    for e in range(E):
        h = X @ deq[e][0].T
        if act == "swiglu":
            g, u = h[:, :I], h[:, I:]
            acts.append(g / (1.0 + np.exp(-g)) * u)
        else:
            acts.append(np.maximum(h, 0.0) ** 2)
    a = np.stack([acts[ids[t, k]][t] * (p[t, k] if on_input else 1.0)
                  for t in range(T) for k in range(K)])
    a32 = a.astype(np.float32)
    if mode == "w4a16":
        a2 = R.bf16_bits_to_f32(R.f32_to_bf16_bits(a32)).reshape(a.shape).astype(np.float64)
    elif mode == "mxfp8":
        a2 = R.mxfp8_dequant(*R.mxfp8_quantize(a32))
    else:
        per_row = mode in R.PER_ROW_MODES
        c, s, g = R.nvfp4_quantize(a32, per_row, four_over_six=mode == "w4a4_token_4o6")
        if mode == "w4a4_token_mxfp4":
            a2 = R.mxfp4_dequant(*R.mxfp4_reblock(c, s), g, per_row)
        else:
            a2 = R.nvfp4_dequant(c, s, g, per_row)
    y = np.zeros((T, x.shape[1]))
    for t in range(T):
        for k in range(K):
            o = a2[t * K + k] @ deq[ids[t, k]][1].T
            y[t] += (1.0 if on_input else p[t, k]) * o
    return y


def _rel(a, b):
    return np.max(np.abs(a - b)) / np.sqrt(np.mean(b * b))


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("act", ["swiglu", "relu2"])
@pytest.mark.parametrize("on_input", [False, True])
def test_forward_matches_dense_brute_force(mode, act, on_input):
    x, lg, W = _setup(mode=mode, act=act)
    K = 2
    ref = R.forward(x, lg, W, K, mode, act, on_input)["y"]
    dense = _dense(x, lg, W, K, mode, act, on_input)
    assert _rel(ref, dense) < 1e-12


@pytest.mark.parametrize("mode", MODES)
def test_topk_equals_E_uniform_is_mean_of_dense_experts(mode):
    E = 8
    x, _, W = _setup(mode=mode, E=E)
    lg = np.zeros((16, E), np.float32)          # equal logits -> p = 1/8 exactly
    y = R.forward(x, lg, W, E, mode, "swiglu", False)["y"]
    dense = _dense(x, lg, W, E, mode, "swiglu", False)
    assert _rel(y, dense) < 1e-12
    # and the weights really were uniform
    _, p = R.route(lg, E)
    assert np.all(p == 1.0 / E)


def test_k1_is_single_expert_output():
    x, lg, W = _setup(mode="w4a16")
    out = R.forward(x, lg, W, 1, "w4a16", "swiglu", False)
    assert np.all(out["p"] == 1.0)
    # y[t] is exactly the FC2 output of token t's route (weight 1)
    assert np.array_equal(out["y"], out["o"])


@pytest.mark.parametrize("act", ["swiglu", "relu2"])
def test_placement_linear_without_fc2_input_quantization(act):
    x, lg, W = _setup(mode="w4a4_token", act=act)
    yo = R.forward(x, lg, W, 2, "w4a4_token", act, False, fc2_input_quant=False)["y"]
    yi = R.forward(x, lg, W, 2, "w4a4_token", act, True, fc2_input_quant=False)["y"]
    assert _rel(yi, yo) < 1e-13
    # with quantization the two placements genuinely differ
    yq = R.forward(x, lg, W, 2, "w4a4_token", act, True)["y"]
    assert not np.array_equal(yq, yo)


@pytest.mark.parametrize("mode", MODES)
def test_placement_bit_exact_with_power_of_two_weights(mode):
    E = 8
    x, _, W = _setup(mode=mode, E=E)
    lg = np.zeros((16, E), np.float32)          # p = 1/8 for every route
    yo = R.forward(x, lg, W, E, mode, "swiglu", False)
    yi = R.forward(x, lg, W, E, mode, "swiglu", True)
    assert np.array_equal(yo["y"], yi["y"])
    if "a2q" in yo:
        assert np.array_equal(yo["a2q"]["codes"], yi["a2q"]["codes"])


def test_pre_activation_variant_is_detected():
    """ReLU(p z)^2 = p^2 ReLU(z)^2, not p ReLU(z)^2: with p = 1/2 the wrong
    variant yields exactly half of the correct input-side output."""
    E = 2
    x, _, W = _setup(mode="w4a16", act="relu2", E=E)
    lg = np.zeros((16, E), np.float32)
    good = R.forward(x, lg, W, E, "w4a16", "relu2", True)["y"]
    bad = R.forward(x, lg, W, E, "w4a16", "relu2", True, pre_act_variant=True)["y"]
    assert np.array_equal(bad, 0.5 * good)
    assert not np.allclose(bad, good)


def test_activation_closed_forms():
    L = R.lib()
    out = np.empty(3)
    h = np.array([0.0, 30.0, -30.0, 2.0, 5.0, 7.0])         # gates | ups
    L.orc_activation(0, 3, R._p(h), 0, 1.0, 0, R._p(out))
    assert out[0] == 0.0                                    # silu(0) = 0
    assert abs(out[1] - 30.0 * 5.0) < 1e-9                  # silu(z) -> z
    assert abs(out[2]) < 1e-10                              # silu(-30) ~ 0
    r = np.array([-3.0, 2.0, 0.0])
    out = np.empty(3)
    L.orc_activation(1, 3, R._p(r), 0, 1.0, 0, R._p(out))
    assert list(out) == [0.0, 4.0, 0.0] and not np.signbit(out[0])
    L.orc_activation(1, 3, R._p(r), 1, 0.25, 0, R._p(out))  # input side: times p
    assert list(out) == [0.0, 1.0, 0.0]


def test_fc1_exact_rational_spot_check():
    """fp64 FC1 sums against exact rational sums of the dequantized operands:
    the difference obeys the sequential-summation bound H * 2^-52 * sum|terms|."""
    x, lg, W = _setup(mode="w4a4_tensor")
    xq = R.quantize_x(x, "w4a4_tensor")
    W.ensure([0, 3])
    for e, t, n in [(0, 0, 0), (0, 5, 200), (3, 11, 17)]:
        h = W.fc1(e, xq["deq"](t))[n]
        (c, s, g), _ = W.q[e]
        xr = [Fraction(v) for v in xq["deq"](t)]
        wr = [Fraction(R.e2m1_decode(c[n, k])) * Fraction(R.e4m3_decode(s[n, k // 16]))
              * Fraction(float(g)) for k in range(W.H)]
        exact = sum(a * b for a, b in zip(xr, wr))
        bound = W.H * 2.0 ** -52 * float(sum(abs(a * b) for a, b in zip(xr, wr)))
        assert abs(h - float(exact)) <= bound


def test_tiny_workload_regression_fixture():
    import json
    import os
    import sys
    sys.path.insert(0, os.path.join(os.path.dirname(__file__), "golden"))
    import make_golden
    with open(os.path.join(os.path.dirname(__file__), "golden", "tiny_oracle_output.json")) as f:
        want = json.load(f)
    got = make_golden.summary(make_golden.compute())
    for k, v in got.items():
        assert want[k] == v, k


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("act", ["swiglu", "relu2"])
def test_batched_products_match_per_route_products(mode, act):
    """The per-expert matrix-product form of FC1 and FC2 (one fp64 product per
    expert over its routes) gives the per-route matrix-vector results up to the
    fp64 summation order, with identical FC2-input codes, on both placements
    and with several threads."""
    x, lg, W = _setup(T=24, E=6, mode=mode, act=act, logits="normal_bias")
    for on_input in (False, True):
        a = R.forward(x, lg, W, 3, mode, act, on_input)
        b = R.forward(x, lg, W, 3, mode, act, on_input, batched=True, threads=4)
        assert np.array_equal(a["a_routes"], b["a_routes"])
        assert _rel(b["a"], a["a"]) < 1e-13
        if "a2q" in a:
            for key in a["a2q"]:
                assert np.array_equal(a["a2q"][key], b["a2q"][key]), key
        assert _rel(b["y"], a["y"]) < 1e-13
        # a token subset gives the same rows as the full forward
        c = R.forward(x, lg, W, 3, mode, act, on_input, batched=True, tokens=[3, 0, 17])
        assert _rel(c["y"], a["y"][[3, 0, 17]]) < 1e-13
