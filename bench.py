"""Benchmark of one block-scaled MoE layer forward on one MI355X.

Default (the headline line): the MXFP8 W8A8 prefill layer, T=16384 tokens,
H=7168, I=2048, E=256 experts, top-8, SwiGLU, Zipf(1.1)-skewed routing, router
weight on the output side, fused finalize (its configured variant); the
deterministic finalize is timed beside it. The other workloads (tiny NVFP4
W4A4, NVFP4 W4A16 decode, NVFP4 W4A4 per-token prefill, NVFP4 W4A4 ReLU2
decode, and the prefill under the 4-over-6 contract and on MXFP4 re-blocked
GEMMs) follow as sub-records of the same line.

A step is one moe_forward (routing, permutation, activation quantization, FC1
with fused activation, FC2-input quantization, FC2, finalize) over inputs
already resident in HBM, replayed from a captured hipGraph. Weights are
prepared once, off the timed path; when a prepared blob is smaller than three
times the 256 MB Infinity Cache, several copies are rotated so weight reads
come from HBM.

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
MFMA_PEAK_TFLOPS = {"bf16": 2500.0, "f16": 2500.0, "fp8": 5000.0, "fp4": 10100.0}
DTYPES = {"w4a16": "bf16", "w4a4_tensor": "f16", "w4a4_token": "f16", "w4a4_token_4o6": "f16",
          "mxfp8": "fp8", "w4a4_token_mxfp4": "fp4"}
METRIC = "MoE layer tokens/s on 1 MI355X; % MFMA peak (prefill), % HBM BW (decode)"
MALL_BYTES = 256 << 20
HEADLINE = "prefill_mxfp8_zipf_T16384_H7168_I2048_E256_K8"
SUBRECORDS = ["tiny_w4a4_tensor_T16_H256_I128_E8_K2", "decode_w4a16_T256_H2048_I1024_E64_K6",
              "prefill_w4a4_token_T4096_H4096_I2048_E128_K8",
              "decode_w4a4_tensor_relu2_T64_H7168_I2048_E256_K8",
              # the prefill layer under the 4-over-6 activation contract, and with
              # its GEMMs on MXFP4 re-blocked operands (FP4 matrix cores)
              "prefill_w4a4_token4o6_T4096_H4096_I2048_E128_K8",
              "prefill_w4a4_token_mxfp4_T4096_H4096_I2048_E128_K8"]
# oracle sample per workload: tokens of a sub-batch that take about 10-30 s
# of single-thread CPU time
CPU_SAMPLE_TOKENS = {"tiny_w4a4_tensor_T16_H256_I128_E8_K2": 16,
                     "decode_w4a16_T256_H2048_I1024_E64_K6": 48,
                     "prefill_w4a4_token_T4096_H4096_I2048_E128_K8": 8,
                     "decode_w4a4_tensor_relu2_T64_H7168_I2048_E256_K8": 8,
                     "prefill_w4a4_token4o6_T4096_H4096_I2048_E128_K8": 8,
                     "prefill_w4a4_token_mxfp4_T4096_H4096_I2048_E128_K8": 8,
                     "prefill_mxfp8_zipf_T16384_H7168_I2048_E256_K8": 3,
                     "ep8_share_mxfp8_zipf_T2048_H7168_I2048_E32_K8": 3}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=HEADLINE)
    ap.add_argument("--no-subrecords", action="store_true",
                    help="time the headline workload only")
    ap.add_argument("--only-configured", action="store_true",
                    help="time only the workload's configured finalize variant (for profiling)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample-tokens", type=int, default=0, help="0 = per-workload default")
    ap.add_argument("--copies", type=int, default=0, help="prepared weight copies (0 = auto)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain device copy of known size (PMC calibration)")
    return ap.parse_args()


def weight_bytes(d, wfmt):
    """Prepared bytes of one expert's W1 and W2 (codes + block scales + global
    scale)."""
    if wfmt == "nvfp4":
        return (d.N1 * d.H // 2 + d.N1 * d.H // 16 + 4, d.H * d.I // 2 + d.H * d.I // 16 + 4)
    if wfmt == "mxfp4":
        return (d.N1 * d.H // 2 + d.N1 * d.H // 32 + 4, d.H * d.I // 2 + d.H * d.I // 32 + 4)
    return (d.N1 * d.H + d.N1 * d.H // 32, d.H * d.I + d.H * d.I // 32)


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
    was taken on the current kernel sources (else None)."""
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


def cpu_baseline(wl, x, logits, w1, w2, ntok):
    """The oracle as it stands, single-threaded, on a sub-batch of the
    workload: its first `ntok` tokens run as a batch of their own (routing,
    permutation, quantization, both GEMMs, finalize). The experts those
    tokens reach are quantized beforehand (not timed, like the GPU's weight
    preparation)."""
    import numpy as np
    import torch

    from oracle import reference as R
    ntok = min(ntok, wl.T)
    xb = x[:ntok].cpu().view(torch.int16).numpy().view(np.uint16)
    lg = logits[:ntok].cpu().numpy()
    W = R.QuantWeights(wl.wfmt, wl.E, wl.H, wl.I, wl.act,
                       lambda e: (w1[e].cpu().numpy(), w2[e].cpu().numpy()))
    ids, _ = R.route(lg, wl.K)
    W.ensure(set(int(e) for e in ids.ravel()), threads=min(16, os.cpu_count() or 1))
    t0 = time.perf_counter()
    R.forward(xb, lg, W, wl.K, wl.mode, wl.act, wl.on_input, threads=1)
    dt = time.perf_counter() - t0
    return {"value": round(ntok / dt, 4), "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "host_cpu": host_cpu(),
            "sample": f"the first {ntok} of {wl.T} tokens as a batch of their own (all {wl.K} "
                      f"routes each, every stage), single thread; experts quantized beforehand, "
                      f"not timed; {dt:.1f} s"}


def roofline(wl, d, counts, st_us, decode):
    """Roofline object for the dominant GEMM of one timed variant.

    Algorithmic bytes per launch (the layer's own data, no intermediates):
    FC1 = weights of the experts with rows + the layer input x (bf16, T*H*2);
    FC2 = weights of the experts with rows + the layer output y (bf16, T*H*2).
    Algorithmic flops per launch: FC1 2*R*N1*H, FC2 2*R*H*I (routed rows only).
    The duration is the kernel's own average, from HIP events recorded at its
    start and end on the launch stream in the eager pass."""
    touched = int((counts > 0).sum())
    b1, b2 = weight_bytes(d, wl.wfmt)
    io = wl.T * wl.H * 2
    R_ = wl.T * wl.K
    kern = "fc1" if st_us["fc1"] >= st_us["fc2"] else "fc2"
    kbytes = touched * (b1 if kern == "fc1" else b2) + io
    kflops = 2.0 * R_ * (wl.N1 * wl.H if kern == "fc1" else wl.H * wl.I)
    us = st_us[kern]
    dtype = DTYPES[wl.mode]
    if decode:
        ach = kbytes / (us * 1e-6) / 1e9
        r = {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
             "frac": round(ach / HBM_PEAK_GBS, 4)}
    else:
        ach = kflops / (us * 1e-6) / 1e12
        peak = MFMA_PEAK_TFLOPS[dtype]
        r = {"bound": "mfma", "achieved": round(ach, 1), "peak": peak, "unit": "TFLOP/s",
             "frac": round(ach / peak, 4)}
    r["traffic"] = committed_traffic(wl.name, kern)
    r["kernel"] = f"gemm_kernel ({kern.upper()})"
    r["avg_launch_us"] = round(us, 2)
    r["algorithmic_bytes"] = int(kbytes)
    r["algorithmic_flops"] = kflops
    return r


def run_workload(name, args, with_cpu, min_timed_s=0.0):
    """Times one workload (both finalize variants it runs); returns its record.
    min_timed_s > 0 (sub-records): the graph replays are repeated until they
    span at least that long, so that host jitter does not dominate the mean of
    a layer that takes tens of microseconds."""
    import numpy as np
    import torch

    import block_scaled_fp4_top_amd as moe
    from synth_inputs import WORKLOADS, make_logits, make_x
    from synth_inputs.gen import STREAM_W1, STREAM_W2, make_weight

    wl = WORKLOADS[name]
    dev = torch.device("cuda:0")
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
    cpu_w = (w1.cpu(), w2.cpu()) if with_cpu else None
    del w1, w2
    torch.cuda.empty_cache()

    ws = torch.empty(moe.workspace_bytes(d, wl.T, wl.K, wl.mode), dtype=torch.uint8, device=dev)
    y = torch.empty((wl.T, wl.H), dtype=torch.bfloat16, device=dev)

    def step(i, det):
        moe.forward(d, blobs[i % copies], x, logits, wl.K, wl.mode, wl.on_input, det,
                    workspace=ws, out=y)

    conf = "fused" if wl.finalize == ("fused",) else "det"   # the configured variant
    other = "det" if conf == "fused" else "fused"
    variants = {}
    for fin in ((conf,) if args.only_configured else (conf, other)):
        det = fin == "det"
        # eager pass: per-stage HIP events on the launch stream (the GEMMs'
        # events are recorded at their own start and end)
        for i in range(args.warmup):
            step(i, det)
        torch.cuda.synchronize()
        moe.stage_times()  # reset
        moe.stage_timing(True)
        for i in range(args.steps):
            step(i, det)
        torch.cuda.synchronize()
        moe.stage_timing(False)
        st, nfw = moe.stage_times()
        assert moe.forward_status(ws) == 0
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
        nrep = args.steps
        if min_timed_s > 0:  # a first estimate of the step time sets the count
            t0 = time.perf_counter()
            for i in range(args.steps):
                graphs[i % copies].replay()
            torch.cuda.synchronize()
            est = (time.perf_counter() - t0) / args.steps
            nrep = max(args.steps, min(5000, int(min_timed_s / max(est, 1e-6)) + 1))
        t0 = time.perf_counter()
        for i in range(nrep):
            graphs[i % copies].replay()
        torch.cuda.synchronize()
        dt = time.perf_counter() - t0
        # per-replay distribution (outside the timed loop above)
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
        evs[0].record()
        for i in range(args.steps):
            graphs[i % copies].replay()
            evs[i + 1].record()
        torch.cuda.synchronize()
        per = sorted(evs[i].elapsed_time(evs[i + 1]) for i in range(args.steps))
        pct = {f"p{q}": round(per[min(len(per) - 1, int(q / 100 * len(per)))], 5)
               for q in (10, 50, 90)}
        variants[fin] = {"ms": dt / nrep * 1e3, "pct": pct, "replays": nrep,
                         "st_us": {k: v / max(nfw, 1) * 1e3 for k, v in st.items()}}
        del graphs

    counts = moe.workspace_view(d, ws, wl.T, wl.K, wl.mode, "counts").cpu().numpy()
    touched = int((counts > 0).sum())
    b1, b2 = weight_bytes(d, wl.wfmt)
    decode = wl.T <= 1024
    R_ = wl.T * wl.K
    flops = 2.0 * R_ * (wl.N1 * wl.H + wl.H * wl.I)
    v = variants[conf]
    rec = {
        "value": round(wl.T / (v["ms"] * 1e-3), 1),
        "ms_per_step": round(v["ms"], 5),
        "dtype": DTYPES[wl.mode],
        "config": {"workload": wl.name, "T": wl.T, "H": wl.H, "I": wl.I, "E": wl.E, "K": wl.K,
                   "mode": wl.mode, "act": wl.act, "router_weight_on_input": wl.on_input,
                   "finalize": "fused" if conf == "fused" else "deterministic",
                   "timing": "hipGraph replay of one forward per step",
                   "weight_copies_rotated": copies, "touched_experts": touched,
                   "routing": routing_summary(counts)},
        "graph_replays_timed": v["replays"],
        "graph_step_ms_percentiles": v["pct"],
        "stages_us": {k: round(u, 2) for k, u in v["st_us"].items()},
        "layer_tflops": round(flops / (v["ms"] * 1e-3) / 1e12, 2),
        "layer_weight_gbs": round(touched * (b1 + b2) / (v["ms"] * 1e-3) / 1e9, 1),
        "roofline": roofline(wl, d, counts, v["st_us"], decode),
    }
    if other in variants:
        o = variants[other]
        rec["deterministic_finalize" if other == "det" else "fused_finalize"] = {
            "value": round(wl.T / (o["ms"] * 1e-3), 1), "ms_per_step": round(o["ms"], 5),
            "graph_replays_timed": o["replays"],
            "graph_step_ms_percentiles": o["pct"],
            "stages_us": {k: round(u, 2) for k, u in o["st_us"].items()},
            "roofline": roofline(wl, d, counts, o["st_us"], decode)}
    rec["cpu_baseline"] = None
    if cpu_w is not None:
        n = args.cpu_sample_tokens or CPU_SAMPLE_TOKENS.get(wl.name, 8)
        rec["cpu_baseline"] = cpu_baseline(wl, x, logits, cpu_w[0], cpu_w[1], n)
    del blobs, ws, y, x, logits
    torch.cuda.empty_cache()
    return rec


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the layer runs all experts on a single MI355X).", file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration()
        return
    import torch
    torch.cuda.set_device(0)
    head = run_workload(args.workload, args, not args.no_cpu_baseline)
    out = {"metric": METRIC, "value": head["value"], "unit": "tokens/s", "n_gpus": 1,
           "steps": args.steps, "warmup": args.warmup, "ms_per_step": head["ms_per_step"],
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
           "dtype": head["dtype"], "data": "synthetic"}
    for k, v in head.items():
        if k not in out:
            out[k] = v
    if not args.no_subrecords:
        out["workloads"] = {}
        for name in SUBRECORDS:
            if name == args.workload:
                continue
            print(f"# sub-record {name}", file=sys.stderr, flush=True)
            out["workloads"][name] = run_workload(name, args, False, min_timed_s=0.1)
    print(json.dumps(out))


if __name__ == "__main__":
    main()
