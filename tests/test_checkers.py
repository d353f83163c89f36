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


# ---------------------------------------------------------------------------
# the layer-output check: accepts the oracle's own result, rejects planted
# mistakes of the kinds a GPU path could make
# ---------------------------------------------------------------------------
import torch  # noqa: E402

from synth_inputs import make_expert_weights, make_logits, make_x  # noqa: E402
from tests.helpers import Fc2Input, check_layer_output  # noqa: E402

LAYER_MODES = ["w4a4_tensor", "w4a4_token", "w4a16", "mxfp8", "w4a4_token_4o6", "w4a4_token_mxfp4"]


def _bf16(y):
    return torch.from_numpy(np.ascontiguousarray(y)).float().bfloat16().double().numpy()


def _layer(mode, on_input, T=12, H=256, I=128, E=4, K=2, seed=1):
    x = make_x(seed, T, H).view(torch.int16).numpy().view(np.uint16)
    lg = make_logits(seed, T, E, "normal").numpy()
    w1, w2 = make_expert_weights(seed, E, 2 * I, H, I)
    W = R.QuantWeights(R.weight_format(mode), E, H, I, "swiglu",
                       lambda e: (w1[e].numpy(), w2[e].numpy()))
    ref = R.forward(x, lg, W, K, mode, "swiglu", on_input)
    rt2row = ref["route_to_row"]
    Rn = T * K

    def perm(a):                       # route order -> permuted row order
        out = np.empty_like(a)
        out[rt2row] = a
        return out
    a32 = ref["a"].astype(np.float32)
    if mode == "w4a16":
        pre = R.bf16_bits_to_f32(R.f32_to_bf16_bits(a32)).reshape(Rn, I)
        gi = Fc2Input(mode, pre=perm(pre))
    elif mode == "mxfp8":
        gi = Fc2Input(mode, codes=perm(ref["a2q"]["codes"]), scales=perm(ref["a2q"]["scales"]))
    else:
        g = ref["a2q"]["g"]
        gi = Fc2Input(mode, pre=perm(a32), codes=perm(ref["a2q"]["codes"]),
                      scales=perm(ref["a2q"]["scales"]), g=perm(g) if mode in R.PER_ROW_MODES else g)
        if mode == "w4a4_token_mxfp4":
            gi.mx_codes, gi.mx_scales = perm(ref["a2q"]["mx_codes"]), perm(ref["a2q"]["mx_scales"])
    return W, ref, gi, K


def _finalize(ref, o_routes, K, on_input, p=None):
    p = ref["p"] if p is None else p
    T = len(ref["tokens"])
    y = np.zeros((T, o_routes.shape[1]))
    for t in range(T):
        for k in range(K):
            y[t] += (1.0 if on_input else p[t, k]) * o_routes[t * K + k]
    return y


@pytest.mark.parametrize("mode", LAYER_MODES)
@pytest.mark.parametrize("on_input", [False, True])
def test_layer_check_accepts_oracle_result(mode, on_input):
    W, ref, gi, K = _layer(mode, on_input)
    res = check_layer_output(_bf16(ref["y"]), gi, ref, W, K, on_input, "oracle")
    assert res["own"][0] <= 2.0 ** -8 * np.abs(ref["y"]).max() / np.sqrt(np.mean(ref["y"] ** 2)) + 1e-12
    check_layer_output(_bf16(ref["y"]), gi, ref, W, K, on_input, "oracle", round_allow=True)


@pytest.mark.parametrize("mode", LAYER_MODES)
def test_layer_check_rejects_missed_fc2_tile(mode):
    """An FC2 tile that never ran: 16 rows of one expert leave 64 output
    columns of their routes' contributions at zero."""
    W, ref, gi, K = _layer(mode, False)
    o = ref["o"].copy()                      # route order
    e = int(np.argmax(ref["counts"]))
    rows = np.arange(ref["offsets"][e], ref["offsets"][e + 1])[:16]
    routes = ref["row_to_route"][rows]
    o[np.ix_(routes, np.arange(64))] = 0.0
    y = _bf16(_finalize(ref, o, K, False))
    with pytest.raises(AssertionError):
        check_layer_output(y, gi, ref, W, K, False, "missed tile")


@pytest.mark.parametrize("mode", LAYER_MODES)
def test_layer_check_rejects_wrong_route_weight(mode):
    """One token's two router weights swapped in the finalize."""
    W, ref, gi, K = _layer(mode, False)
    p = ref["p"].copy()
    t = int(np.argmax(np.abs(p[:, 0] - p[:, 1])))
    p[t, 0], p[t, 1] = p[t, 1], p[t, 0]
    y = _bf16(_finalize(ref, ref["o"], K, False, p))
    with pytest.raises(AssertionError):
        check_layer_output(y, gi, ref, W, K, False, "swapped weight")


@pytest.mark.parametrize("mode", ["w4a4_tensor", "w4a4_token", "mxfp8", "w4a4_token_4o6",
                                  "w4a4_token_mxfp4"])
@pytest.mark.parametrize("consistent", [False, True])
def test_layer_check_rejects_wrong_fc2_input_code(mode, consistent):
    """One FC2-input code one step off (toward zero) in the largest element of
    a route. consistent=True: the output is recomputed from the wrong code too
    (a quantizer bug the GEMM faithfully used); False: only the view is off."""
    W, ref, gi, K = _layer(mode, False)
    row = 5
    j = int(np.argmax(np.abs(gi.dequant_row(row))))
    c = int(gi.codes[row, j])
    gi.codes[row, j] = (c & 0x80) | ((c & 0x7F) - 1) if mode == "mxfp8" else (c & 8) | ((c & 7) - 1)
    y = ref["y"]
    if consistent:
        r = int(ref["row_to_route"][row])
        e = int(ref["ids"].flat[r])
        o = ref["o"].copy()
        o[r] = W.fc2_rows(e, gi.dequant_row(row)[None])[0]
        y = _finalize(ref, o, K, False)
    with pytest.raises(AssertionError):
        check_layer_output(_bf16(y), gi, ref, W, K, False, "wrong code")


def test_layer_check_rejects_wrong_global_scale():
    """The per-tensor FC2-input global scale one fp32 ulp off, codes kept."""
    W, ref, gi, K = _layer("w4a4_tensor", True)
    gi.g = np.nextafter(gi.g, np.float32(1.0)).astype(np.float32)
    with pytest.raises(AssertionError):
        check_layer_output(_bf16(ref["y"]), gi, ref, W, K, True, "wrong g")


@pytest.mark.parametrize("mode", ["w4a4_tensor", "w4a4_token", "w4a4_token_4o6"])
def test_nvfp4_code_check_alone(mode):
    """check_a2_nvfp4 by itself (without the bit-exact quantizer check)
    accepts the oracle's codes and rejects a code one step off, a block scale
    one step off and a swapped pair of columns."""
    from tests.helpers import check_a2_nvfp4
    W, ref, gi, K = _layer(mode, True)
    check_a2_nvfp4(gi, ref, "oracle")
    row = 3
    j = int(np.argmax(np.abs(gi.dequant_row(row))))
    for plant in ("code", "scale", "swap"):
        _, ref2, g2, _ = _layer(mode, True)
        if plant == "code":
            g2.codes[row, j] = (g2.codes[row, j] & 8) | ((g2.codes[row, j] & 7) - 1)
        elif plant == "scale":
            g2.scales[row, j // 16] += 1
        else:
            a, b = g2.codes[row, j].copy(), g2.codes[row, j ^ 1].copy()
            if a == b:
                continue
            g2.codes[row, j], g2.codes[row, j ^ 1] = b, a
        with pytest.raises(AssertionError):
            check_a2_nvfp4(g2, ref2, plant)


def test_layer_check_rejects_wrong_reblocked_code():
    """Mode 5: one re-blocked MXFP4 FC2-input code one step off (the NVFP4 codes
    right), with the output recomputed from it."""
    W, ref, gi, K = _layer("w4a4_token_mxfp4", False)
    row = 7
    j = int(np.argmax(np.abs(gi.dequant_row(row))))
    gi.mx_codes[row, j] = (gi.mx_codes[row, j] & 8) | ((gi.mx_codes[row, j] & 7) - 1)
    r = int(ref["row_to_route"][row])
    o = ref["o"].copy()
    o[r] = W.fc2_rows(int(ref["ids"].flat[r]), gi.dequant_row(row)[None])[0]
    with pytest.raises(AssertionError):
        check_layer_output(_bf16(_finalize(ref, o, K, False)), gi, ref, W, K, False, "wrong mx code")
