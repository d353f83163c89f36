"""Writes tiny_oracle_output.json: the oracle's output on the tiny NVFP4 W4A4
per-tensor workload (T=16, H=256, I=128, E=8, top-2, SwiGLU, output side,
seed 0). Calls only oracle/ and synth_inputs/; a regression fixture for the
oracle itself (run from the repository root: python tests/golden/make_golden.py).
"""
import hashlib
import json
import os
import sys

import numpy as np
import torch

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__)))))
from oracle import reference as R  # noqa: E402
from synth_inputs import make_expert_weights, make_logits, make_x  # noqa: E402


def compute():
    T, H, I, E, K = 16, 256, 128, 8, 2
    x = make_x(0, T, H).view(torch.int16).numpy().view(np.uint16)
    lg = make_logits(0, T, E, "normal").numpy()
    w1, w2 = make_expert_weights(0, E, 2 * I, H, I)
    w1, w2 = w1.numpy(), w2.numpy()
    W = R.QuantWeights("nvfp4", E, H, I, "swiglu", lambda e: (w1[e], w2[e]))
    return R.forward(x, lg, W, K, "w4a4_tensor", "swiglu", False)


def summary(out):
    y = out["y"]
    return {
        "ids": out["ids"].ravel().tolist(),
        "counts": out["counts"].tolist(),
        "x_global_scale_hex": float(out["xq"]["g"][0]).hex(),
        "y_sha256": hashlib.sha256(np.ascontiguousarray(y).tobytes()).hexdigest(),
        "y_samples_hex": [float(v).hex() for v in y.ravel()[::137]],
    }


if __name__ == "__main__":
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "tiny_oracle_output.json")
    with open(path, "w") as f:
        json.dump({"source": "written by tests/golden/make_golden.py (oracle only)",
                   **summary(compute())}, f, indent=1)
    print("wrote", path)
