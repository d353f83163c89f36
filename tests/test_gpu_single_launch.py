"""The single-launch layer kernel (small batches) against the multi-launch
sequence: the same tiles, quantizers and finalize arithmetic in another
schedule, so every intermediate and the output must agree bit for bit with the
deterministic multi-launch forward. The oracle parity of the single launch is
covered by the other GPU tests, whose small shapes take it by default."""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # collected on CPU runs too; every test is marked gpu
    pytest.skip("no GPU", allow_module_level=True)

import block_scaled_fp4_top_amd as moe  # noqa: E402
from oracle import reference as R  # noqa: E402
from tests.helpers import Inputs, check_layer  # noqa: E402

# The single launch is switched off for every shape: on the GPU its kernel
# finished (bit-identical to the multi-launch forward) in the per-tensor NVFP4
# mode, but did not finish in the per-row NVFP4 mode (first shape below,
# on_input=False) and then in the W4A16 mode (same shape); the cause is not
# found. Every test that launches it stays, skipped.
OFF = pytest.mark.skip(reason="single-launch layer switched off: it did not finish in two GPU "
                              "runs (per-row NVFP4, W4A16), cause not found")
SINGLE_MODES = ["w4a4_tensor", "w4a16", "mxfp8"]
MODE_PARAMS = SINGLE_MODES + ["w4a4_token", "w4a4_token_4o6"]


@pytest.fixture(autouse=True)
def _auto_path_afterwards():
    yield
    moe.set_forward_path("auto")


def _views(mode):
    v = ["topk_ids", "topk_w", "counts", "offsets", "row_to_route", "route_to_row", "o"]
    if mode in ("w4a4_tensor", "w4a4_token", "w4a4_token_4o6"):
        v += ["x_codes", "x_scales", "x_g", "a2_pre", "a2_codes", "a2_scales", "a2_g"]
    elif mode == "mxfp8":
        v += ["x_codes", "x_scales", "a2_codes", "a2_scales"]
    else:
        v += ["a2_pre"]
    return v


def _forward(path, d, blob, inp, K, mode, on_input, det):
    moe.set_forward_path(path)
    assert moe.forward_path(d, inp.T, K, mode) == path
    ws = torch.zeros(moe.workspace_bytes(d, inp.T, K, mode), dtype=torch.uint8, device="cuda")
    y = moe.forward(d, blob, inp.x, inp.logits, K, mode, on_input, det, workspace=ws)
    torch.cuda.synchronize()
    st = moe.forward_status(ws)
    # on a wait that gave up: the counter's word index, its target, its value
    assert st == 0, f"{path}: status {st}, wait record {ws[4:16].view(torch.int32).tolist()}"
    return y, ws


def compare_paths(inp, K, mode, on_input, what=""):
    d = moe.Dims(inp.E, inp.H, inp.I, inp.act, R.weight_format(mode))
    blob = moe.prepare_weights(d, inp.w1, inp.w2)
    y_m, ws_m = _forward("multi", d, blob, inp, K, mode, on_input, True)
    y_s, ws_s = _forward("single", d, blob, inp, K, mode, on_input, True)
    T = inp.T
    for name in _views(mode):
        a = moe.workspace_view(d, ws_m, T, K, mode, name)
        b = moe.workspace_view(d, ws_s, T, K, mode, name)
        if name in ("x_g", "a2_g") and mode == "w4a4_tensor":
            # one tensor-wide scale: the multi-launch path stores it once, the
            # single launch beside every row
            n = T if name == "x_g" else T * K
            assert torch.equal(b[:n], a[:1].expand(n)), f"{what} {name}"
        else:
            assert torch.equal(a, b), f"{what} {name}"
    assert torch.equal(y_m, y_s), f"{what}: single-launch y differs from the multi-launch y"
    # the finalize flag does not change the single launch's result
    y_f, _ = _forward("single", d, blob, inp, K, mode, on_input, False)
    assert torch.equal(y_f, y_s), f"{what}: finalize flag changed the single-launch y"
    return d, blob, y_s, ws_s


# (T, H, I, E, K, act, logits): tiles of 16 and 32 rows, one and several
# column blocks, ReLU2 widths that are not a multiple of 256 (MXFP8 FC1 with
# two strips per wave), K = E, a single token, the largest batch (T*K = 4096)
# and many empty experts.
SHAPES = [
    (16, 256, 128, 8, 2, "swiglu", "normal"),
    (100, 384, 256, 8, 2, "swiglu", "normal"),
    (60, 256, 384, 16, 4, "relu2", "zipf"),
    (12, 256, 128, 8, 8, "swiglu", "uniform"),
    (1, 512, 256, 32, 6, "swiglu", "normal"),
    (512, 256, 128, 128, 8, "relu2", "normal"),
    (5, 256, 256, 256, 3, "swiglu", "zipf"),
]


@OFF
@pytest.mark.parametrize("mode", MODE_PARAMS)
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "T{}_H{}_I{}_E{}_K{}_{}".format(*s[:6]))
def test_single_launch_matches_multi_launch(mode, shape):
    T, H, I, E, K, act, lg = shape
    inp = Inputs(T, H, I, E, K, act, lg, seed=T + E)
    for on_input in (False, True):
        compare_paths(inp, K, mode, on_input, f"{mode} {shape} on_input={on_input}")


@OFF
@pytest.mark.parametrize("mode", ["w4a4_tensor", "w4a16", "mxfp8"])
def test_single_launch_against_oracle(mode):
    """The single launch against the oracle, forced (not only by default)."""
    T, H, I, E, K = 48, 256, 256, 16, 4
    inp = Inputs(T, H, I, E, K, "swiglu", "normal", seed=3)
    d = moe.Dims(E, H, I, "swiglu", R.weight_format(mode))
    blob = moe.prepare_weights(d, inp.w1, inp.w2)
    y, ws = _forward("single", d, blob, inp, K, mode, False, True)
    W = inp.oracle_weights(R.weight_format(mode))
    ref = R.forward(inp.x_bits(), inp.logits_np(), W, K, mode, "swiglu", False, threads=8)
    check_layer(moe, d, ws, y, ref, W, T, K, mode, False, f"single {mode}", threads=8)


def test_path_selection():
    """While the single launch is off, every shape takes the multi-launch
    sequence under "auto" and is refused under "single"."""
    d = moe.Dims(64, 256, 128, "swiglu", "nvfp4")
    moe.set_forward_path("auto")
    for T, K, mode in ((256, 6, "w4a16"), (4096, 6, "w4a16"), (64, 8, "w4a4_tensor"),
                       (256, 6, "w4a4_token")):
        assert moe.forward_path(d, T, K, mode) == "multi"
    moe.set_forward_path("multi")
    assert moe.forward_path(d, 256, 6, "w4a16") == "multi"
    moe.set_forward_path("single")
    for T, K, mode in ((256, 6, "w4a16"), (4096, 6, "w4a16"), (256, 6, "w4a4_token")):
        with pytest.raises(moe.MoeError) as ei:
            moe.forward_path(d, T, K, mode)
        assert ei.value.code == 2


def test_forced_single_launch_refuses_large_batches_before_launch():
    T, H, I, E, K = 1100, 256, 128, 8, 4   # T*K = 4400 routes
    inp = Inputs(T, H, I, E, K, "swiglu", "normal")
    d = moe.Dims(E, H, I, "swiglu", "nvfp4")
    blob = moe.prepare_weights(d, inp.w1, inp.w2)
    moe.set_forward_path("single")
    y = torch.full((T, H), 3.0, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(moe.MoeError) as ei:
        moe.forward(d, blob, inp.x, inp.logits, K, "w4a16", out=y)
    assert ei.value.code == 2
    torch.cuda.synchronize()
    assert bool((y == 3.0).all())


@OFF
def test_single_launch_header_mismatch():
    """A blob prepared for another activation: the prologue flags it and the
    layer kernel writes nothing."""
    T, H, I, E, K = 16, 256, 128, 8, 2
    inp = Inputs(T, H, I, E, K, "swiglu", "normal")
    d_sw = moe.Dims(E, H, I, "swiglu", "nvfp4")
    d_r2 = moe.Dims(E, H, I, "relu2", "nvfp4")
    blob = moe.prepare_weights(d_sw, inp.w1, inp.w2)
    moe.set_forward_path("single")
    ws = torch.empty(moe.workspace_bytes(d_sw, T, K, "w4a16"), dtype=torch.uint8, device="cuda")
    y = torch.full((T, H), 3.0, dtype=torch.bfloat16, device="cuda")
    moe.forward(d_r2, blob, inp.x, inp.logits, K, "w4a16", workspace=ws, out=y)
    assert moe.forward_status(ws) == 1
    assert bool((y == 3.0).all())
    moe.forward(d_sw, blob, inp.x, inp.logits, K, "w4a16", workspace=ws, out=y)
    assert moe.forward_status(ws) == 0
    assert not bool((y == 3.0).any())


@OFF
def test_single_launch_workspace_reuse_and_repeat():
    """Counters are cleared per forward: repeated and interleaved forwards of
    two shapes on one workspace give the same outputs as fresh workspaces."""
    mode = "w4a16"
    a = Inputs(40, 256, 128, 8, 3, "swiglu", "normal", seed=1)
    b = Inputs(7, 256, 128, 8, 5, "swiglu", "zipf", seed=2)
    d = moe.Dims(8, 256, 128, "swiglu", "nvfp4")
    blob = moe.prepare_weights(d, a.w1, a.w2)
    moe.set_forward_path("single")
    ref_a = moe.forward(d, blob, a.x, a.logits, 3, mode)
    ref_b = moe.forward(d, blob, b.x, b.logits, 5, mode)
    ws = torch.empty(max(moe.workspace_bytes(d, 40, 3, mode), moe.workspace_bytes(d, 7, 5, mode)),
                     dtype=torch.uint8, device="cuda")
    for _ in range(3):
        ya = moe.forward(d, blob, a.x, a.logits, 3, mode, workspace=ws)
        yb = moe.forward(d, blob, b.x, b.logits, 5, mode, workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(ya, ref_a) and torch.equal(yb, ref_b)
