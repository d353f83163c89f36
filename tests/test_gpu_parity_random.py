"""GPU parity over a seeded random sample of layer shapes and modes.

Each case draws T, E, K, H, I, the activation, the mode, the placement of the
router weight and the finalize variant from a fixed-seed generator, so the
sample reaches the launch configurations the fixed cases may miss: every
M-tile size (chosen from the mean rows per expert), weight column counts that
are and are not multiples of 256 and 512, ragged expert groups and empty
experts. Every case checks routing and permutation bit-exactly, the FC1-input
and FC2-input quantization, and the output against the oracle's bar applied
to the error beyond the output's own bf16 rounding: on some of these shapes
the heavy-tailed outputs make even the exactly rounded oracle miss the plain
max-error bar (its largest |y| reaches 9 rms), which the named workloads'
tests keep.
"""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

from tests.helpers import Inputs, check_layer  # noqa: E402
from tests.test_gpu_parity_small import check_routing, check_x_quant, run_layer  # noqa: E402
import block_scaled_fp4_top_amd as moe  # noqa: E402
from oracle import reference as R  # noqa: E402

MODES = ["w4a4_tensor", "w4a4_token", "w4a16", "mxfp8", "w4a4_token_4o6", "w4a4_token_mxfp4"]


def _cases(n=24, seed=20261202):
    """Small shapes: every M-tile size, ragged groups, empty experts."""
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        E = int(rng.choice([1, 3, 8, 17, 40, 64]))
        K = int(rng.integers(1, min(E, 8) + 1))
        T = int(rng.choice([1, 5, 33, 96, 200, 300]))
        H = int(rng.choice([128, 256, 384, 640]))
        I = int(rng.choice([128, 256, 384]))
        act = str(rng.choice(["swiglu", "relu2"]))
        mode = MODES[i % len(MODES)]
        on_input = bool(rng.integers(0, 2))
        det = bool(rng.integers(0, 4) != 0)  # mostly deterministic, some fused
        logits = str(rng.choice(["normal", "uniform", "zipf"]))
        out.append((i, T, H, I, E, K, act, mode, on_input, det, logits))
    return out


def _big_cases(n=8, seed=7):
    """Wider shapes: 128-row tiles with 512-column blocks (eight waves), skewed
    groups of several tiles."""
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        E = int(rng.choice([16, 32, 64]))
        K = int(rng.choice([4, 8]))
        T = int(rng.choice([512, 1024]))
        H = int(rng.choice([512, 768, 1024]))
        I = int(rng.choice([256, 512]))
        act = str(rng.choice(["swiglu", "relu2"]))
        mode = MODES[i % len(MODES)]
        on_input = bool(rng.integers(0, 2))
        det = bool(rng.integers(0, 4) != 0)
        logits = str(rng.choice(["normal", "zipf"]))
        out.append((100 + i, T, H, I, E, K, act, mode, on_input, det, logits))
    return out


def _route_cases(n=8, seed=11):
    """Many experts and routes: the multi-block permutation (more than 16384
    routes or more than 256 experts) and every routing width (E up to 1024)."""
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        E = int(rng.choice([128, 200, 256, 300, 512, 1024]))
        K = int(rng.choice([1, 2, 6, 9, 16]))
        T = int(rng.choice([64, 700, 2048, 2500]))
        H = int(rng.choice([128, 256]))
        I = int(rng.choice([128, 256]))
        act = str(rng.choice(["swiglu", "relu2"]))
        mode = MODES[i % len(MODES)]
        on_input = bool(rng.integers(0, 2))
        det = bool(rng.integers(0, 4) != 0)
        logits = str(rng.choice(["normal", "uniform", "zipf"]))
        out.append((200 + i, T, H, I, E, K, act, mode, on_input, det, logits))
    return out


@pytest.mark.parametrize("case", _cases() + _big_cases() + _route_cases(), ids=lambda c: f"case{c[0]}")
def test_random_shape(case):
    i, T, H, I, E, K, act, mode, on_input, det, logits = case
    what = f"case{i} T={T} H={H} I={I} E={E} K={K} {act} {mode} on_input={on_input} det={det} {logits}"
    print(what, flush=True)
    inp = Inputs(T, H, I, E, K, act, logits, seed=100 + i)
    d, blob, ws, y, ref, W = run_layer(inp, K, mode, on_input, det)
    check_routing(d, ws, T, K, mode, ref)
    check_x_quant(d, ws, T, K, mode, ref)
    check_layer(moe, d, ws, y, ref, W, T, K, mode, on_input, what, round_allow=True)


@pytest.mark.parametrize("case", _cases() + _big_cases() + _route_cases(), ids=lambda c: f"case{c[0]}")
def test_fused_equals_deterministic(case):
    """On every sampled shape and mode, the fused finalize (the FC2 block
    completing a token's routes reduces them) gives the deterministic
    finalize's bits: the arrival counts on every tile configuration (16- to
    128-row tiles, two or four strips per wave, four or eight waves)."""
    i, T, H, I, E, K, act, mode, on_input, _, logits = case
    what = f"case{i} T={T} H={H} I={I} E={E} K={K} {act} {mode} on_input={on_input} {logits}"
    print(what, flush=True)
    inp = Inputs(T, H, I, E, K, act, logits, seed=100 + i)
    d = moe.Dims(E, H, I, act, R.weight_format(mode))
    blob = moe.prepare_weights(d, inp.w1, inp.w2)
    y_d = moe.forward(d, blob, inp.x, inp.logits, K, mode, on_input, True)
    y_f = moe.forward(d, blob, inp.x, inp.logits, K, mode, on_input, False)
    torch.cuda.synchronize()
    ndiff = int((y_f.view(torch.int16) != y_d.view(torch.int16)).sum().item())
    assert ndiff == 0, f"{what}: fused and deterministic outputs differ in {ndiff} elements"


@pytest.mark.parametrize("mode", MODES)
def test_workspace_reuse_across_shapes(mode):
    """A workspace sized for a large batch, reused for a smaller one right after:
    the second forward matches a forward on a fresh workspace bit for bit
    (deterministic finalize) and the oracle, so no state leaks between calls."""
    E, K, H, I = 24, 4, 256, 128
    big = Inputs(300, H, I, E, K, "swiglu", "zipf", seed=7)
    small = Inputs(37, H, I, E, K, "swiglu", "normal", seed=8)
    d = moe.Dims(E, H, I, "swiglu", R.weight_format(mode))
    blob = moe.prepare_weights(d, small.w1, small.w2)
    ws = torch.empty(moe.workspace_bytes(d, 300, K, mode), dtype=torch.uint8, device="cuda")
    moe.forward(d, blob, big.x, big.logits, K, mode, True, True, workspace=ws)
    y_reused = moe.forward(d, blob, small.x, small.logits, K, mode, True, True, workspace=ws).clone()
    y_fresh = moe.forward(d, blob, small.x, small.logits, K, mode, True, True)
    torch.cuda.synchronize()
    assert torch.equal(y_reused.view(torch.int16), y_fresh.view(torch.int16)), f"{mode}: reused workspace differs"
    _, _, ws2, y, ref, W = run_layer(small, K, mode, True, True)
    assert torch.equal(y.view(torch.int16), y_fresh.view(torch.int16))
    check_layer(moe, d, ws2, y_reused, ref, W, 37, K, mode, True, f"reuse {mode}")


def test_concurrent_forwards_share_a_blob():
    """Two streams run forwards on one prepared blob with their own workspaces
    at the same time; each result equals the same forward run alone."""
    E, K, H, I, mode = 16, 2, 256, 128, "w4a4_tensor"
    a = Inputs(200, H, I, E, K, "swiglu", "normal", seed=21)
    b = Inputs(90, H, I, E, K, "swiglu", "zipf", seed=22)
    d = moe.Dims(E, H, I, "swiglu", "nvfp4")
    blob = moe.prepare_weights(d, a.w1, a.w2)
    ya0 = moe.forward(d, blob, a.x, a.logits, K, mode, False, True).clone()
    yb0 = moe.forward(d, blob, b.x, b.logits, K, mode, False, True).clone()
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    wa = torch.empty(moe.workspace_bytes(d, 200, K, mode), dtype=torch.uint8, device="cuda")
    wb = torch.empty(moe.workspace_bytes(d, 90, K, mode), dtype=torch.uint8, device="cuda")
    outs = []
    for _ in range(4):
        with torch.cuda.stream(s1):
            ya = moe.forward(d, blob, a.x, a.logits, K, mode, False, True, workspace=wa, stream=s1)
        with torch.cuda.stream(s2):
            yb = moe.forward(d, blob, b.x, b.logits, K, mode, False, True, workspace=wb, stream=s2)
        torch.cuda.synchronize()
        outs.append((ya.clone(), yb.clone()))
    for ya, yb in outs:
        assert torch.equal(ya.view(torch.int16), ya0.view(torch.int16))
        assert torch.equal(yb.view(torch.int16), yb0.view(torch.int16))
