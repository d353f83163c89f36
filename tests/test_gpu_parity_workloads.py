"""GPU parity at the five synthetic workloads' full sizes, in the launch
configuration the benchmark times. Routing, permutation and the quantized
FC1 input are compared bit-exactly in full; prepared weights on a sample of
experts; the layer output on every token where the oracle can afford it
(T <= 256) and on a seeded sample of tokens otherwise (their outputs do not
depend on other tokens except through the per-tensor FC2-input scale, for
which the oracle runs FC1 over every route)."""
import time

import numpy as np
import pytest
import torch

pytestmark = [pytest.mark.gpu, pytest.mark.slow]

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import block_scaled_fp4_top_amd as moe  # noqa: E402
from oracle import reference as R  # noqa: E402
from synth_inputs import WORKLOADS  # noqa: E402
from tests.helpers import (Inputs, assert_output_close_flips, bf16_to_f64,  # noqa: E402
                           check_fc2_input, unpack_expert)
from tests.test_gpu_parity_small import check_routing, check_x_quant  # noqa: E402

THREADS = 16


def _log(msg):
    print(f"[{time.strftime('%H:%M:%S')}] {msg}", flush=True)


@pytest.mark.parametrize("name", list(WORKLOADS))
def test_workload_full_size(name):
    wl = WORKLOADS[name]
    _log(f"workload {name}: generating inputs")
    inp = Inputs(wl.T, wl.H, wl.I, wl.E, wl.K, wl.act, wl.logits, seed=wl.seed,
                 gen_device="cpu" if wl.T * wl.H < 10000 else "cuda")
    d = moe.Dims(wl.E, wl.H, wl.I, wl.act, wl.wfmt)
    blob = moe.prepare_weights(d, inp.w1, inp.w2)
    ws = torch.empty(moe.workspace_bytes(d, wl.T, wl.K, wl.mode), dtype=torch.uint8, device="cuda")
    ys = {}
    for fin in wl.finalize:
        ys[fin] = moe.forward(d, blob, inp.x, inp.logits, wl.K, wl.mode, wl.on_input,
                              fin == "det", workspace=ws)
    torch.cuda.synchronize()
    _log("forward done; oracle routing/permutation/quantization")
    W = inp.oracle_weights(wl.wfmt)
    if wl.T <= 256:
        tokens = None
    else:
        rng = np.random.default_rng(1234)
        tokens = sorted(rng.choice(wl.T, size=8, replace=False).tolist())
    ref = R.forward(inp.x_bits(), inp.logits_np(), W, wl.K, wl.mode, wl.act, wl.on_input,
                    tokens=tokens, threads=THREADS)
    _log(f"oracle done ({len(W.q)} experts quantized)")
    check_routing(d, ws, wl.T, wl.K, wl.mode, ref)
    check_x_quant(d, ws, wl.T, wl.K, wl.mode, ref)
    # prepared weights: a few experts, including the most loaded one
    blob_np = blob.cpu().numpy()
    hot = int(np.argmax(ref["counts"]))
    for e in sorted({0, hot, wl.E - 1} & set(W.q)):
        w1c, w1s, g1, w2c, w2s, g2 = unpack_expert(blob_np, e)
        (oc1, os1, og1), (oc2, os2, og2) = W.q[e]
        assert np.array_equal(w1c, oc1) and np.array_equal(w1s, os1), e
        assert np.array_equal(w2c, oc2) and np.array_equal(w2s, os2), e
        if wl.wfmt == "nvfp4":
            assert g1 == og1 and g2 == og2
    check_fc2_input(moe, d, ws, wl.T, wl.K, wl.mode, ref, name)
    toks = ref["tokens"]
    for fin, y in ys.items():
        yg = bf16_to_f64(y)[toks]
        mx, fro = assert_output_close_flips(yg, ref, W, wl.mode, wl.K, wl.on_input,
                                            f"{name} {fin}")
        _log(f"{name} finalize={fin}: max|err|/rms={mx:.3e} rel_fro={fro:.3e}")
    if "fused" in ys:
        # every token, not a sample: the fused output equals the deterministic
        # one up to the order of its fp32 atomic sums (one bf16 rounding step
        # where the two fp32 sums fall on either side of a rounding boundary).
        # A tile the fused FC2 missed or added twice would be off by whole
        # route contributions. The deterministic FC2 runs the default block
        # order, so this also checks the fused path's own order.
        y_det = ys.get("det")
        if y_det is None:
            y_det = moe.forward(d, blob, inp.x, inp.logits, wl.K, wl.mode, wl.on_input, True,
                                workspace=ws)
        yd = y_det.float()
        yf = ys["fused"].float()
        rms = float(yd.pow(2).mean().sqrt())
        excess = ((yf - yd).abs() - 2.0 ** -7 * yd.abs()).max().item()
        assert excess <= 1e-3 * rms, f"{name}: fused vs deterministic differ by {excess:.3e} (rms {rms:.3e})"
        _log(f"{name}: fused == deterministic up to summation order on all {wl.T} tokens")
