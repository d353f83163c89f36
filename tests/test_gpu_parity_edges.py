"""GPU parity on the degenerate and boundary cases of the layer: one token,
K = 1 and K = E, empty experts, every token on one expert (several M-tiles and
a ragged tail), expert group sizes on both sides of the M-tile boundaries,
hidden sizes that are not powers of two, and the largest E and K the library
accepts."""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import block_scaled_fp4_top_amd as moe  # noqa: E402
from tests.helpers import Inputs, check_layer  # noqa: E402
from tests.test_gpu_parity_small import check_routing, check_x_quant, run_layer  # noqa: E402


def _with_logits(inp: Inputs, logits: np.ndarray):
    inp.logits = torch.from_numpy(np.ascontiguousarray(logits, np.float32)).cuda()
    return inp


def _onehot_logits(assign, E, seed=0):
    """Token t's largest logit is on expert assign[t]; the rest are small noise."""
    rng = np.random.default_rng(seed)
    lg = rng.standard_normal((len(assign), E)).astype(np.float32) * 0.1
    lg[np.arange(len(assign)), assign] = 10.0
    return lg


def _run_and_check(inp, K, mode, on_input, det=True, what=""):
    d, blob, ws, y, ref, W = run_layer(inp, K, mode, on_input, det)
    check_routing(d, ws, inp.T, K, mode, ref)
    check_x_quant(d, ws, inp.T, K, mode, ref)
    return check_layer(moe, d, ws, y, ref, W, inp.T, K, mode, on_input, what)


@pytest.mark.parametrize("mode", ["w4a4_tensor", "w4a4_token", "w4a16", "mxfp8"])
def test_single_token(mode):
    inp = Inputs(1, 256, 128, 8, 2, "swiglu", "normal")
    _run_and_check(inp, 2, mode, False, what=f"T=1 {mode}")


@pytest.mark.parametrize("mode", ["w4a4_token", "mxfp8"])
def test_k1_and_k_equals_e(mode):
    inp = Inputs(20, 256, 128, 4, 1, "relu2", "normal")
    _run_and_check(inp, 1, mode, True, what="K=1")
    inp = Inputs(20, 256, 128, 4, 4, "relu2", "normal")
    _run_and_check(inp, 4, mode, False, what="K=E")


def test_many_empty_experts():
    inp = Inputs(8, 256, 128, 64, 2, "swiglu", "normal")
    d, blob, ws, y, ref, W = run_layer(inp, 2, "w4a16", False, True)
    assert (ref["counts"] == 0).sum() >= 40
    check_routing(d, ws, 8, 2, "w4a16", ref)
    check_layer(moe, d, ws, y, ref, W, 8, 2, "w4a16", False, "empty experts")


@pytest.mark.parametrize("mode", ["w4a4_tensor", "w4a16", "mxfp8"])
def test_all_tokens_on_one_expert(mode):
    T, E = 300, 8
    inp = _with_logits(Inputs(T, 256, 128, E, 1, "swiglu", "normal"),
                       _onehot_logits(np.full(T, 3), E))
    for det in (True, False):
        _run_and_check(inp, 1, mode, False, det, what=f"one expert {mode} det={det}")


@pytest.mark.parametrize("on_input", [False, True])
def test_group_sizes_across_tile_boundaries(on_input):
    sizes = [8, 15, 16, 17, 31, 32, 33, 63, 64, 65, 127, 128, 129, 192, 1]
    assign = np.concatenate([np.full(n, e) for e, n in enumerate(sizes)])
    rng = np.random.default_rng(3)
    rng.shuffle(assign)
    E = len(sizes) + 1  # the last expert stays empty
    inp = _with_logits(Inputs(len(assign), 384, 256, E, 1, "swiglu", "normal"),
                       _onehot_logits(assign, E))
    for mode in ("w4a4_token", "w4a16", "mxfp8"):
        for det in (True, False):
            _run_and_check(inp, 1, mode, on_input, det, what=f"tiles {mode} det={det}")


def test_top2_group_sizes_and_bm_choice():
    """K = 2 with expert loads straddling 16/32/64/128 rows under every M-tile
    size the launcher may pick (T chosen so R/E selects each tile size)."""
    for T, E in [(40, 8), (120, 8), (250, 8), (700, 8)]:
        inp = Inputs(T, 256, 128, E, 2, "swiglu", "normal_bias")
        _run_and_check(inp, 2, "w4a4_token", True, what=f"T={T}")


def test_largest_e_and_k():
    inp = Inputs(64, 256, 128, 1024, 8, "swiglu", "normal", gen_device="cuda")
    _run_and_check(inp, 8, "w4a16", False, what="E=1024")
    inp = Inputs(4, 256, 128, 64, 64, "relu2", "normal")
    _run_and_check(inp, 64, "w4a4_tensor", True, what="K=64")


@pytest.mark.parametrize("K", [12, 33, 64])
def test_fused_finalize_large_k(K):
    """The fused finalize with more routes than one read-back batch (K > 8)
    and with one token per read-back round (K > 32): against the oracle, and
    bit for bit against the deterministic finalize."""
    print(f"case fused K={K}", flush=True)
    inp = Inputs(6, 256, 128, 64, K, "relu2", "normal")
    _, _, _, y_f, _, _ = run_layer(inp, K, "w4a4_tensor", True, False)
    _run_and_check(inp, K, "w4a4_tensor", True, det=False, what=f"fused K={K}")
    _, _, _, y_d, _, _ = run_layer(inp, K, "w4a4_tensor", True, True)
    torch.cuda.synchronize()
    assert torch.equal(y_f, y_d), f"K={K}: fused and deterministic outputs differ"


def test_ties_in_logits():
    """Exactly equal logits: lower expert ids win; the permutation stays stable."""
    T, E = 48, 16
    lg = np.zeros((T, E), np.float32)
    lg[:, 5] = 1.0
    lg[::2, 9] = 1.0
    inp = _with_logits(Inputs(T, 256, 128, E, 3, "swiglu", "normal"), lg)
    _run_and_check(inp, 3, "mxfp8", False, what="ties")


def test_invalid_arguments_rejected_before_launch():
    inp = Inputs(4, 256, 128, 8, 2, "swiglu", "normal")
    d = moe.Dims(8, 256, 128, "swiglu", "nvfp4")
    blob = moe.prepare_weights(d, inp.w1, inp.w2)
    with pytest.raises(TypeError):
        moe.forward(d, blob, inp.x.float(), inp.logits, 2, "w4a16")
    with pytest.raises(TypeError):
        moe.forward(d, blob, inp.x, inp.logits.double(), 2, "w4a16")
    with pytest.raises(ValueError):
        moe.forward(d, blob, inp.x, inp.logits[:, :4].contiguous(), 2, "w4a16")
    with pytest.raises(ValueError):
        moe.forward(d, blob, inp.x, inp.logits.cpu(), 2, "w4a16")
    with pytest.raises(ValueError):
        moe.forward(d, blob, inp.x, inp.logits.t().contiguous().t(), 2, "w4a16")
    with pytest.raises(moe.MoeError):      # NVFP4 blob with the MXFP8 mode
        moe.forward(d, blob, inp.x, inp.logits, 2, "mxfp8")
    with pytest.raises(moe.MoeError):      # K > E
        moe.forward(d, blob, inp.x, inp.logits, 9, "w4a16")
    small = torch.empty(64, dtype=torch.uint8, device="cuda")
    with pytest.raises(moe.MoeError) as ei:
        moe.forward(d, blob, inp.x, inp.logits, 2, "w4a16", workspace=small)
    assert ei.value.code == 3
    d2 = moe.Dims(8, 256, 256, "swiglu", "nvfp4")
    with pytest.raises(moe.MoeError):      # blob prepared for other dims
        moe.check_prepared(d2, blob)


@pytest.mark.parametrize("det", [True, False])
def test_mismatched_blob_header_detected_on_device(det):
    """A blob prepared for other dimensions but large enough for the call (a
    SwiGLU blob used as a ReLU2 one): the forward's first kernel finds the
    header difference, no kernel writes y, and the status word says so; a
    matching forward on the same workspace then reports 0."""
    T, H, I, E, K = 16, 256, 128, 8, 2
    inp = Inputs(T, H, I, E, K, "swiglu", "normal")
    d_sw = moe.Dims(E, H, I, "swiglu", "nvfp4")
    d_r2 = moe.Dims(E, H, I, "relu2", "nvfp4")
    blob = moe.prepare_weights(d_sw, inp.w1, inp.w2)
    assert blob.numel() >= moe.prepared_bytes(d_r2)
    ws = torch.empty(moe.workspace_bytes(d_sw, T, K, "w4a4_tensor"), dtype=torch.uint8, device="cuda")
    y = torch.full((T, H), 3.0, dtype=torch.bfloat16, device="cuda")
    moe.forward(d_r2, blob, inp.x, inp.logits, K, "w4a4_tensor", False, det, workspace=ws, out=y)
    assert moe.forward_status(ws) == 1
    assert bool((y == 3.0).all()), "y written although the blob header did not match"
    moe.forward(d_sw, blob, inp.x, inp.logits, K, "w4a4_tensor", False, det, workspace=ws, out=y)
    assert moe.forward_status(ws) == 0
    assert not bool((y == 3.0).all())
