"""GPU parity at sizes the oracle finishes in seconds: every mode, activation,
router-weight placement and finalize variant; bit-exact routing, permutation,
quantized activations and prepared weights; tolerance on the layer output."""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # collected on CPU runs too; every test is marked gpu
    pytest.skip("no GPU", allow_module_level=True)

import block_scaled_fp4_top_amd as moe  # noqa: E402
from oracle import reference as R  # noqa: E402
from tests.helpers import (Inputs, TOPW_REL, assert_output_close,  # noqa: E402
                           bf16_to_f64, check_layer, unpack_expert, unpack_nibbles)

MODES = ["w4a4_tensor", "w4a4_token", "w4a16", "mxfp8", "w4a4_token_4o6", "w4a4_token_mxfp4"]


def _fmt(mode):
    return R.weight_format(mode)


def run_layer(inp: Inputs, K, mode, on_input, det, threads=8, tokens=None, batched=False):
    d = moe.Dims(inp.E, inp.H, inp.I, inp.act, _fmt(mode))
    blob = moe.prepare_weights(d, inp.w1, inp.w2)
    moe.check_prepared(d, blob)
    ws = torch.empty(moe.workspace_bytes(d, inp.T, K, mode), dtype=torch.uint8, device="cuda")
    y = moe.forward(d, blob, inp.x, inp.logits, K, mode, on_input, det, workspace=ws)
    torch.cuda.synchronize()
    W = inp.oracle_weights(_fmt(mode))
    ref = R.forward(inp.x_bits(), inp.logits_np(), W, K, mode, inp.act, on_input,
                    tokens=tokens, threads=threads, batched=batched)
    return d, blob, ws, y, ref, W


def view(d, ws, T, K, mode, name):
    return moe.workspace_view(d, ws, T, K, mode, name).cpu().numpy()


def check_routing(d, ws, T, K, mode, ref):
    assert np.array_equal(view(d, ws, T, K, mode, "topk_ids").reshape(T, K), ref["ids"])
    w = view(d, ws, T, K, mode, "topk_w").reshape(T, K).astype(np.float64)
    assert np.max(np.abs(w - ref["p"]) / ref["p"]) <= TOPW_REL
    assert np.array_equal(view(d, ws, T, K, mode, "counts"), ref["counts"])
    assert np.array_equal(view(d, ws, T, K, mode, "offsets"), ref["offsets"])
    assert np.array_equal(view(d, ws, T, K, mode, "row_to_route"), ref["row_to_route"])
    assert np.array_equal(view(d, ws, T, K, mode, "route_to_row"), ref["route_to_row"])


def check_x_quant(d, ws, T, K, mode, ref):
    if mode == "w4a16":
        return
    xq = ref["xq"]
    H = d.H
    if mode == "mxfp8":
        assert np.array_equal(view(d, ws, T, K, mode, "x_codes").reshape(T, H), xq["codes"])
        assert np.array_equal(view(d, ws, T, K, mode, "x_scales").reshape(T, H // 32), xq["scales"])
        return
    codes = unpack_nibbles(view(d, ws, T, K, mode, "x_codes"), H).reshape(T, H)
    assert np.array_equal(codes, xq["codes"])
    assert np.array_equal(view(d, ws, T, K, mode, "x_scales").reshape(T, H // 16), xq["scales"])
    g = view(d, ws, T, K, mode, "x_g")
    if mode in R.PER_ROW_MODES:
        assert np.array_equal(g[:T], xq["g"])
    else:
        assert g[0] == xq["g"][0]
    if mode == "w4a4_token_mxfp4":  # the GEMM operand: x re-blocked to MXFP4
        assert np.array_equal(unpack_nibbles(view(d, ws, T, K, mode, "x_mx_codes"), H).reshape(T, H),
                              xq["mx_codes"])
        assert np.array_equal(view(d, ws, T, K, mode, "x_mx_scales").reshape(T, H // 32),
                              xq["mx_scales"])


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("act", ["swiglu", "relu2"])
@pytest.mark.parametrize("on_input", [False, True])
@pytest.mark.parametrize("det", [True, False])
def test_tiny_layer(mode, act, on_input, det):
    T, H, I, E, K = 16, 256, 128, 8, 2
    print(f"case mode={mode} act={act} on_input={on_input} det={det}", flush=True)
    inp = Inputs(T, H, I, E, K, act, "normal")
    d, blob, ws, y, ref, W = run_layer(inp, K, mode, on_input, det)
    check_routing(d, ws, T, K, mode, ref)
    check_x_quant(d, ws, T, K, mode, ref)
    check_layer(moe, d, ws, y, ref, W, T, K, mode, on_input, f"{mode}/{act}/{on_input}/{det}")


@pytest.mark.parametrize("mode", MODES)
def test_prepared_weights_bit_exact(mode):
    act = "swiglu"
    T, H, I, E, K = 4, 384, 256, 4, 2
    inp = Inputs(T, H, I, E, K, act, "normal")
    d = moe.Dims(E, H, I, act, _fmt(mode))
    blob = moe.prepare_weights(d, inp.w1, inp.w2).cpu().numpy()
    W = inp.oracle_weights(_fmt(mode))
    W.ensure(range(E))
    for e in range(E):
        w1c, w1s, g1, w2c, w2s, g2 = unpack_expert(blob, e)
        (oc1, os1, og1), (oc2, os2, og2) = W.q[e]
        assert np.array_equal(w1c, oc1) and np.array_equal(w1s, os1)
        assert np.array_equal(w2c, oc2) and np.array_equal(w2s, os2)
        if mode != "mxfp8":
            assert g1 == og1 and g2 == og2


@pytest.mark.parametrize("act", ["swiglu", "relu2"])
def test_prepared_weights_relu2_and_swiglu_layout(act):
    T, H, I, E, K = 4, 256, 384, 3, 1
    inp = Inputs(T, H, I, E, K, act, "normal")
    for fmt in ("nvfp4", "mxfp8"):
        d = moe.Dims(E, H, I, act, fmt)
        blob = moe.prepare_weights(d, inp.w1, inp.w2).cpu().numpy()
        W = inp.oracle_weights(fmt)
        W.ensure(range(E))
        for e in range(E):
            w1c, w1s, _, w2c, w2s, _ = unpack_expert(blob, e)
            (oc1, os1, _), (oc2, os2, _) = W.q[e]
            assert np.array_equal(w1c, oc1) and np.array_equal(w1s, os1)
            assert np.array_equal(w2c, oc2) and np.array_equal(w2s, os2)


def _crafted_matrix(rows, cols, seed):
    """Seeded normal values with planted edge cases: exact E2M1 ties at the
    block scale, zeros and negative zeros, all-zero blocks, subnormals and a
    wide dynamic range across rows."""
    g = torch.Generator().manual_seed(seed)
    v = torch.randn(rows, cols, generator=g, dtype=torch.float32)
    v *= torch.exp2(torch.randint(-20, 20, (rows, 1), generator=g).float())
    v[0, :16] = torch.tensor([6, 0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5, -0.25, -0.75, -1.25,
                              -1.75, -2.5, -3.5, -5, 0.0])
    v[0, 16:32] = 0.0
    v[0, 17] = -0.0
    v[1, :32] = torch.tensor([1e-40, -3e-39] + [0.0] * 30)
    v[2, 32:64] = torch.tensor([448.0, 480.0, -500.0, 300.0] + [0.001] * 28)
    return v


@pytest.mark.parametrize("kind", ["nvfp4_tensor", "nvfp4_row", "mxfp8", "nvfp4_row_4o6"])
def test_quantizer_bit_exact(kind):
    # shapes reach every row-quantizer variant: few long rows (a block per
    # row, and rows split into chunks of 256 quantization blocks: 2 chunks for
    # NVFP4 at 7168 columns, 4 / 2 for NVFP4 / MXFP8 at 16384, partial last
    # chunks), short rows, and many long rows held in registers (1 and 7
    # blocks of 16 per lane, the latter with idle lanes)
    for rows, cols, seed in [(7, 256, 1), (33, 2048, 2), (3, 7168, 3), (2080, 1024, 4),
                             (2049, 7168, 5), (5, 16384, 6), (3, 12320, 7)]:
        v = _crafted_matrix(rows, cols, seed)
        codes, scales, g = moe.quantize(v.cuda(), kind)
        torch.cuda.synchronize()
        vn = v.numpy()
        if kind == "mxfp8":
            oc, osc = R.mxfp8_quantize(vn)
            assert np.array_equal(codes.cpu().numpy(), oc)
            assert np.array_equal(scales.cpu().numpy(), osc)
        else:
            oc, osf, og = R.nvfp4_quantize(vn, per_row=kind != "nvfp4_tensor",
                                           four_over_six=kind == "nvfp4_row_4o6")
            assert np.array_equal(unpack_nibbles(codes.cpu().numpy(), cols), oc)
            assert np.array_equal(scales.cpu().numpy(), osf)
            assert np.array_equal(g.cpu().numpy(), og)


def test_quantizer_zero_matrix():
    v = torch.zeros(4, 64, device="cuda")
    v[1, 5] = -0.0
    codes, scales, g = moe.quantize(v, "nvfp4_tensor")
    c = unpack_nibbles(codes.cpu().numpy(), 64)
    assert g.item() == 0.0 and not scales.cpu().numpy().any()
    assert c[1, 5] == 8 and c.sum() == 8


@pytest.mark.parametrize("mode", MODES)
def test_deterministic_repeat_and_graph_replay(mode):
    T, H, I, E, K = 24, 256, 128, 8, 3
    inp = Inputs(T, H, I, E, K, "swiglu", "normal")
    d = moe.Dims(E, H, I, "swiglu", _fmt(mode))
    blob = moe.prepare_weights(d, inp.w1, inp.w2)
    ws = torch.empty(moe.workspace_bytes(d, T, K, mode), dtype=torch.uint8, device="cuda")
    y = torch.empty(T, H, dtype=torch.bfloat16, device="cuda")
    moe.forward(d, blob, inp.x, inp.logits, K, mode, True, True, workspace=ws, out=y)
    torch.cuda.synchronize()
    y0, ws0 = y.clone(), ws.clone()
    for _ in range(3):
        moe.forward(d, blob, inp.x, inp.logits, K, mode, True, True, workspace=ws, out=y)
    torch.cuda.synchronize()
    assert torch.equal(y, y0)
    for name in ["topk_ids", "topk_w", "counts", "offsets", "row_to_route", "route_to_row", "o"]:
        assert torch.equal(moe.workspace_view(d, ws, T, K, mode, name),
                           moe.workspace_view(d, ws0, T, K, mode, name)), name
    # hipGraph capture and replay on a side stream
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        moe.forward(d, blob, inp.x, inp.logits, K, mode, True, True, workspace=ws, out=y)
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=s):
            moe.forward(d, blob, inp.x, inp.logits, K, mode, True, True, workspace=ws, out=y,
                        stream=s)
    torch.cuda.synchronize()
    for _ in range(3):
        y.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, y0)
    # the graph reads its inputs at replay time: new x and logits, eager work
    # in between, every replay against the eager result for the same inputs
    inp2 = Inputs(T, H, I, E, K, "swiglu", "uniform", seed=5, make_weights=False)
    x1, l1 = inp.x.clone(), inp.logits.clone()
    y2 = moe.forward(d, blob, inp2.x, inp2.logits, K, mode, True, True)
    torch.cuda.synchronize()
    for rep in range(4):
        src_x, src_l, ref = (inp2.x, inp2.logits, y2) if rep % 2 == 0 else (x1, l1, y0)
        inp.x.copy_(src_x)
        inp.logits.copy_(src_l)
        y.fill_(1.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, ref), f"replay {rep}"


@pytest.mark.parametrize("mode", ["w4a4_tensor", "mxfp8"])
def test_fused_graph_replay(mode):
    """Fused finalize under graph capture: the arrival counters are cleared
    by a kernel inside the graph on every replay."""
    T, H, I, E, K = 24, 256, 128, 8, 3
    inp = Inputs(T, H, I, E, K, "swiglu", "normal")
    d = moe.Dims(E, H, I, "swiglu", _fmt(mode))
    blob = moe.prepare_weights(d, inp.w1, inp.w2)
    ws = torch.empty(moe.workspace_bytes(d, T, K, mode), dtype=torch.uint8, device="cuda")
    y = torch.empty(T, H, dtype=torch.bfloat16, device="cuda")
    yd = moe.forward(d, blob, inp.x, inp.logits, K, mode, False, True)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        moe.forward(d, blob, inp.x, inp.logits, K, mode, False, False, workspace=ws, out=y)
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=s):
            moe.forward(d, blob, inp.x, inp.logits, K, mode, False, False, workspace=ws, out=y,
                        stream=s)
    torch.cuda.synchronize()
    for rep in range(3):
        y.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, yd), f"fused graph replay {rep}"


def test_fused_matches_deterministic():
    """The fused finalize reduces each token's K routes in the deterministic
    finalize's order and arithmetic: the two outputs are the same bits."""
    T, H, I, E, K = 32, 256, 128, 8, 4
    inp = Inputs(T, H, I, E, K, "swiglu", "normal")
    for mode in MODES:
        print(f"case mode={mode}", flush=True)
        d = moe.Dims(E, H, I, "swiglu", _fmt(mode))
        blob = moe.prepare_weights(d, inp.w1, inp.w2)
        yd = moe.forward(d, blob, inp.x, inp.logits, K, mode, False, True)
        yf = moe.forward(d, blob, inp.x, inp.logits, K, mode, False, False)
        torch.cuda.synchronize()
        assert torch.equal(yf, yd), f"fused vs det {mode}"


@pytest.mark.parametrize("mode,on_input", [("mxfp8", False), ("w4a4_token", True), ("w4a16", False)])
def test_fused_on_reused_workspace(mode, on_input):
    """Fused forwards of different inputs, then a smaller one, on one
    workspace: the rows of O a completing block reads back are this call's
    (a stale row from the call before would change the sum), and the arrival
    counters start from zero on every call."""
    H, I, E = 512, 256, 16
    d = None
    ws = None
    for i, (T, K) in enumerate([(96, 4), (96, 4), (40, 3), (96, 4)]):
        print(f"case mode={mode} call={i} T={T} K={K}", flush=True)
        inp = Inputs(T, H, I, E, K, "swiglu", "normal", seed=100 + i)
        if d is None:
            d = moe.Dims(E, H, I, "swiglu", _fmt(mode))
            blob = moe.prepare_weights(d, inp.w1, inp.w2)
            ws = torch.empty(moe.workspace_bytes(d, 96, 4, mode), dtype=torch.uint8, device="cuda")
        yf = moe.forward(d, blob, inp.x, inp.logits, K, mode, on_input, False, workspace=ws)
        torch.cuda.synchronize()
        yd = moe.forward(d, blob, inp.x, inp.logits, K, mode, on_input, True)
        torch.cuda.synchronize()
        assert torch.equal(yf, yd), f"call {i}: fused vs det {mode}"


@pytest.mark.parametrize("T,K,H", [(37, 5, 384), (9, 3, 2052), (2100, 2, 260)])
def test_standalone_finalize(T, K, H):
    """moe_finalize against the oracle's sequential finalize, fp32 and bf16 O:
    one block per token (T >= 2048) and per token and 1024-column chunk with
    a partial last chunk (H = 2052)."""
    g = torch.Generator().manual_seed(7 + T)
    O = torch.randn(T * K, H, generator=g)
    perm = torch.randperm(T * K, generator=g).to(torch.int32)
    w = torch.rand(T, K, generator=g)

    def ref_of(O64, weights):
        ref = np.empty((T, H))
        R.lib().orc_finalize(T, K, H, R._p(O64), R._p(perm.numpy()),
                             None if weights is None else R._p(weights.double().numpy()),
                             R._p(ref))
        return ref

    for weights in (w, None):
        for o_bf16 in (False, True):
            Od = O.cuda().bfloat16() if o_bf16 else O.cuda()
            y = moe.finalize(Od, perm.cuda(), None if weights is None else weights.cuda(), T, K)
            torch.cuda.synchronize()
            O64 = (O.bfloat16() if o_bf16 else O).double().numpy()
            ref = ref_of(np.ascontiguousarray(O64), weights)
            yg = bf16_to_f64(y)
            assert yg.shape == (T, H)
            # one bf16 rounding of an fp32 sum of K terms
            bound = 2.0 ** -8 * np.abs(ref) + 1e-6 * np.abs(O64).max() * K
            assert np.all(np.abs(yg - ref) <= bound), (T, K, H, weights is None, o_bf16)
