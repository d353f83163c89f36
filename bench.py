"""Benchmark of one block-scaled MoE layer forward on one MI355X.

Default workload: NVFP4 W4A16 decode layer, T=256 tokens, H=2048, I=1024,
E=64 experts, top-6, SwiGLU, router weight on the output side, deterministic
(fixed-order) finalize; the fused-finalize variant is timed beside it.

A step is one moe_forward (routing, permutation, FC1 with fused SwiGLU,
FC2-input store, FC2, finalize) over resident inputs. Weights are prepared
once (off the timed path). Several prepared weight copies are rotated so the
working set exceeds the 256 MB Infinity Cache and weight reads come from HBM.

Prints one JSON line (see --help for options).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MFMA_PEAK_TFLOPS = {"bf16": 2500.0, "f16": 2500.0, "fp8": 5000.0}
METRIC = "MoE layer tokens/s on 1 MI355X; % MFMA peak (prefill), % HBM BW (decode)"
MALL_BYTES = 256 << 20


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="decode_w4a16_T256_H2048_I1024_E64_K6")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample-tokens", type=int, default=48)
    ap.add_argument("--copies", type=int, default=0, help="prepared weight copies (0 = auto)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain device copy of known size (PMC calibration)")
    return ap.parse_args()


def touched_bytes(d, counts, wfmt):
    """Algorithmic weight bytes of FC1 and FC2 for the experts with rows."""
    touched = int((counts > 0).sum())
    if wfmt == "nvfp4":
        b1 = d.N1 * d.H // 2 + d.N1 * d.H // 16 + 4
        b2 = d.H * d.I // 2 + d.H * d.I // 16 + 4
    else:
        b1 = d.N1 * d.H + d.N1 * d.H // 32
        b2 = d.H * d.I + d.H * d.I // 32
    return touched, touched * b1, touched * b2


def kernel_hash():
    """Hash of the GEMM device code (moe_gemm.hip up to its host launchers,
    and the layout/codec header)."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "block_scaled_fp4_top_amd", "csrc")
    with open(os.path.join(csrc, "moe_gemm.hip"), "rb") as fh:
        h.update(fh.read().split(b"// ---- host launchers")[0])
    with open(os.path.join(csrc, "moe_internal.h"), "rb") as fh:
        h.update(fh.read())
    return h.hexdigest()[:16]


def committed_traffic(workload, kernel):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it
    was taken on the current kernel sources."""
    path = os.path.join(ROOT, "profiles", f"pmc_{kernel}_{workload}.txt")
    if not os.path.exists(path):
        return None
    vals = {}
    with open(path) as f:
        for line in f:
            if ":" in line:
                k, v = line.split(":", 1)
                vals[k.strip()] = v.strip()
    if vals.get("kernel_sources_sha256_16") != kernel_hash():
        return None
    try:
        return float(vals["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def copy_calibration():
    import torch
    n = 1 << 30
    a = torch.empty(n, dtype=torch.uint8, device="cuda")
    b = torch.empty(n, dtype=torch.uint8, device="cuda")
    a.fill_(1)
    for _ in range(5):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "launches": 5}))


def routing_summary(counts):
    """The realized expert histogram in brief (rows per expert)."""
    import numpy as np
    c = np.sort(np.asarray(counts, dtype=np.int64))[::-1]
    return {"max_rows": int(c[0]), "mean_rows": round(float(c.mean()), 2),
            "empty_experts": int((c == 0).sum()), "top3_rows": [int(v) for v in c[:3]],
            "groups_under_16_rows": int(((c > 0) & (c < 16)).sum())}


def host_cpu():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(wl, x, logits, w1, w2, sample_tokens):
    """The oracle (as it stands) on a sample of the same workload: weights are
    quantized first (not timed, like the GPU's preparation); then S1..S7 of the
    oracle run single-threaded for the first `sample_tokens` tokens (routing,
    permutation and x quantization cover all tokens)."""
    import numpy as np
    import torch

    from oracle import reference as R
    T = wl.T
    toks = list(range(min(sample_tokens, T)))
    xb = x.cpu().view(torch.int16).numpy().view(np.uint16)
    lg = logits.cpu().numpy()
    W = R.QuantWeights(wl.wfmt, wl.E, wl.H, wl.I, wl.act,
                       lambda e: (w1[e].cpu().numpy(), w2[e].cpu().numpy()))
    ids, _ = R.route(lg, wl.K)
    need = set(int(e) for e in ids.ravel()) if wl.mode == "w4a4_tensor" else \
        set(int(e) for e in ids[toks].ravel())
    W.ensure(need, threads=min(16, os.cpu_count() or 1))
    t0 = time.perf_counter()
    R.forward(xb, lg, W, wl.K, wl.mode, wl.act, wl.on_input, tokens=toks, threads=1)
    dt = time.perf_counter() - t0
    return {"value": len(toks) / dt, "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "host_cpu": host_cpu(),
            "sample": f"{len(toks)} of {T} tokens (all {wl.K} routes each), single thread; "
                      f"weights quantized beforehand, not timed; {dt:.1f} s"}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the layer runs all experts on a single MI355X).", file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration()
        return
    import numpy as np
    import torch

    import block_scaled_fp4_top_amd as moe
    from synth_inputs import WORKLOADS, make_logits, make_x
    from synth_inputs.gen import STREAM_W1, STREAM_W2, make_weight

    wl = WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    d = moe.Dims(wl.E, wl.H, wl.I, wl.act, wl.wfmt)
    x = make_x(wl.seed, wl.T, wl.H, device=dev)
    logits = make_logits(wl.seed, wl.T, wl.E, wl.logits, device=dev)
    w1 = torch.empty((wl.E, wl.N1, wl.H), dtype=torch.float32, device=dev)
    w2 = torch.empty((wl.E, wl.H, wl.I), dtype=torch.float32, device=dev)
    for e in range(wl.E):
        w1[e] = make_weight(wl.seed, STREAM_W1, e, wl.N1, wl.H, device=dev)
        w2[e] = make_weight(wl.seed, STREAM_W2, e, wl.H, wl.I, device=dev)
    nbytes = moe.prepared_bytes(d)
    copies = args.copies or max(1, math.ceil(3 * MALL_BYTES / nbytes))
    copies = min(copies, 8)
    blobs = [moe.prepare_weights(d, w1, w2) for _ in range(copies)]
    torch.cuda.synchronize()
    moe.check_prepared(d, blobs[0])
    cpu_w = None
    if not args.no_cpu_baseline:
        cpu_w = (w1.cpu(), w2.cpu())
    del w1, w2
    torch.cuda.empty_cache()

    ws = torch.empty(moe.workspace_bytes(d, wl.T, wl.K, wl.mode), dtype=torch.uint8, device=dev)
    y = torch.empty((wl.T, wl.H), dtype=torch.bfloat16, device=dev)

    def step(i, det):
        moe.forward(d, blobs[i % copies], x, logits, wl.K, wl.mode, wl.on_input, det,
                    workspace=ws, out=y)

    results = {}
    for det in (True, False):
        if det is False and "fused" not in wl.finalize:
            continue
        # eager pass: per-stage HIP events on the launch stream
        for i in range(args.warmup):
            step(i, det)
        torch.cuda.synchronize()
        moe.stage_times()  # reset
        moe.stage_timing(True)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(args.steps):
            step(i, det)
        torch.cuda.synchronize()
        dt_eager = time.perf_counter() - t0
        moe.stage_timing(False)
        st, nfw = moe.stage_times()
        # graph pass: one captured forward per weight copy, replayed in turn
        graphs = []
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for i in range(copies):
                step(i, det)
            torch.cuda.synchronize()
            for i in range(copies):
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g, stream=side):
                    moe.forward(d, blobs[i], x, logits, wl.K, wl.mode, wl.on_input, det,
                                workspace=ws, out=y, stream=side)
                graphs.append(g)
        torch.cuda.synchronize()
        for i in range(args.warmup):
            graphs[i % copies].replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(args.steps):
            graphs[i % copies].replay()
        torch.cuda.synchronize()
        dt_graph = time.perf_counter() - t0
        # distribution: one event pair per replay (outside the timed loop above)
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
        evs[0].record()
        for i in range(args.steps):
            graphs[i % copies].replay()
            evs[i + 1].record()
        torch.cuda.synchronize()
        per = sorted(evs[i].elapsed_time(evs[i + 1]) for i in range(args.steps))
        pct = {f"p{q}": round(per[min(len(per) - 1, int(q / 100 * len(per)))], 5) for q in (10, 50, 90)}
        results[det] = (dt_graph / args.steps * 1e3, dt_eager / args.steps * 1e3,
                        {k: v / max(nfw, 1) for k, v in st.items()}, pct)
        del graphs

    counts = moe.workspace_view(d, ws, wl.T, wl.K, wl.mode, "counts").cpu().numpy()
    touched, wb1, wb2 = touched_bytes(d, counts, wl.wfmt)
    R_ = wl.T * wl.K
    # algorithmic bytes per launch (see the design notes): weights of the
    # touched experts, the kernel's activation input once, its output once
    x_in = wl.T * wl.H * (2 if wl.mode == "w4a16" else (1 if wl.mode == "mxfp8" else 0.5 + 1 / 16))
    fc1_out = R_ * wl.I * (2 if wl.mode == "w4a16" else 4)
    fc2_in = R_ * wl.I * (2 if wl.mode == "w4a16" else (1 + 1 / 32 if wl.mode == "mxfp8" else 0.5 + 1 / 16))
    fc2_out = R_ * wl.H * 4
    bytes_fc1 = wb1 + x_in + fc1_out
    bytes_fc2 = wb2 + fc2_in + fc2_out
    flops_fc1 = 2.0 * R_ * wl.N1 * wl.H
    flops_fc2 = 2.0 * R_ * wl.H * wl.I
    ms_det, ms_eager, st_det, pct_det = results[True] if True in results else results[False]
    kernel = "fc1" if st_det["fc1"] >= st_det["fc2"] else "fc2"
    kms = st_det[kernel]
    kbytes = bytes_fc1 if kernel == "fc1" else bytes_fc2
    kflops = flops_fc1 if kernel == "fc1" else flops_fc2
    decode = wl.T <= 1024
    dtype = {"w4a16": "bf16", "w4a4_tensor": "f16", "w4a4_token": "f16", "mxfp8": "fp8"}[wl.mode]
    if decode:
        ach = kbytes / (kms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(ach / HBM_PEAK_GBS, 4)}
    else:
        ach = kflops / (kms * 1e-3) / 1e12
        peak = MFMA_PEAK_TFLOPS[dtype]
        roof = {"bound": "mfma", "achieved": round(ach, 1), "peak": peak, "unit": "TFLOP/s",
                "frac": round(ach / peak, 4)}
    tr = committed_traffic(wl.name, kernel)
    roof["traffic"] = tr
    roof["kernel"] = f"gemm_kernel ({kernel.upper()})"
    roof["avg_launch_us"] = round(kms * 1e3, 2)
    roof["algorithmic_bytes"] = int(kbytes)
    roof["algorithmic_flops"] = kflops

    out = {
        "metric": METRIC,
        "value": round(wl.T / (ms_det * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_det, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dtype,
        "data": "synthetic",
        "config": {"workload": wl.name, "T": wl.T, "H": wl.H, "I": wl.I, "E": wl.E,
                   "K": wl.K, "mode": wl.mode, "act": wl.act,
                   "router_weight_on_input": wl.on_input,
                   "finalize": "deterministic" if True in results else "fused",
                   "timing": "hipGraph replay of one forward per step",
                   "weight_copies_rotated": copies, "touched_experts": touched,
                   "routing": routing_summary(counts)},
        "eager_ms_per_step": round(ms_eager, 5),
        "graph_step_ms_percentiles": pct_det,
        "stages_us": {k: round(v * 1e3, 2) for k, v in st_det.items()},
        "layer_tflops": round((flops_fc1 + flops_fc2) / (ms_det * 1e-3) / 1e12, 2),
        "layer_weight_gbs": round((wb1 + wb2) / (ms_det * 1e-3) / 1e9, 1),
        "roofline": roof,
    }
    if False in results and True in results:
        ms_f, ms_fe, st_f, pct_f = results[False]
        out["fused_finalize"] = {"value": round(wl.T / (ms_f * 1e-3), 1),
                                 "ms_per_step": round(ms_f, 5),
                                 "graph_step_ms_percentiles": pct_f,
                                 "eager_ms_per_step": round(ms_fe, 5),
                                 "stages_us": {k: round(v * 1e3, 2) for k, v in st_f.items()}}
    out["cpu_baseline"] = None
    if cpu_w is not None:
        out["cpu_baseline"] = cpu_baseline(wl, x, logits, cpu_w[0], cpu_w[1],
                                           args.cpu_sample_tokens)
    print(json.dumps(out))


if __name__ == "__main__":
    main()
