"""The forward without allocation (moe_forward_noalloc), called through the C
ABI, against moe_forward on a caller workspace: bit-identical outputs with
either finalize (the fused one reduces in the deterministic order), on two
calls in a row where the second has fewer tokens (the built-in workspace
keeps the first call's contents)."""
import pytest
import torch

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import block_scaled_fp4_top_amd as moe  # noqa: E402
from tests.helpers import Inputs  # noqa: E402

CASES = [  # mode, act, on_input, (T_first, T_second), E, H, I, K
    ("w4a16", "swiglu", False, (256, 37), 64, 2048, 1024, 6),
    ("w4a4_tensor", "relu2", True, (64, 9), 256, 1024, 512, 8),
    ("w4a4_token", "swiglu", True, (300, 120), 16, 512, 256, 4),
    ("mxfp8", "swiglu", False, (200, 1), 32, 512, 256, 8),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: c[0])
def test_noalloc_matches_workspace_forward(case):
    mode, act, on_input, Ts, E, H, I, K = case
    print(f"noalloc case {mode} {act} on_input={on_input} T={Ts} E={E} H={H} I={I} K={K}", flush=True)
    big = Inputs(Ts[0], H, I, E, K, act, "normal", seed=31)
    small = Inputs(Ts[1], H, I, E, K, act, "zipf", seed=32, make_weights=False)
    d = moe.Dims(E, H, I, act, "mxfp8" if mode == "mxfp8" else "nvfp4")
    blob = moe.prepare_weights(d, big.w1, big.w2)
    for det in (True, False):
        outs = []
        for inp in (big, small):          # two calls in a row, the second smaller
            y_na = moe.forward_noalloc(d, blob, inp.x, inp.logits, K, mode, on_input, det)
            y_ws = moe.forward(d, blob, inp.x, inp.logits, K, mode, on_input, det)
            torch.cuda.synchronize()
            outs.append((y_na.clone(), y_ws.clone()))
        for (y_na, y_ws), inp in zip(outs, (big, small)):
            assert torch.equal(y_na.view(torch.int16), y_ws.view(torch.int16)), \
                f"{mode} det={det} T={inp.T}: no-alloc forward differs from the workspace forward"


def test_noalloc_rejects_oversized_forward():
    """A shape whose workspace exceeds the built-in 64 MiB is refused before any
    launch (MOE_ERR_WORKSPACE)."""
    E, H, I, K, T = 8, 2048, 1024, 8, 1024
    d = moe.Dims(E, H, I, "swiglu", "nvfp4")
    assert moe.workspace_bytes(d, T, K, "w4a16") > 64 << 20
    inp = Inputs(T, H, I, E, K, "swiglu", "normal", seed=3, make_weights=False)
    blob = torch.zeros(moe.prepared_bytes(d), dtype=torch.uint8, device="cuda")
    with pytest.raises(moe.MoeError) as ei:
        moe.forward_noalloc(d, blob, inp.x, inp.logits, K, "w4a16")
    assert ei.value.code == 3
