"""Benchmark of the fused SwiGLU MLP training step on one MI355X.

A step is one forward + full backward (all six kernels) over one batch of
synthetic input at D=4096, H=11008, B=8, S=8192 (T=65536), bf16 storage with
fp32 accumulation. Inputs are generated once and are resident in HBM before
the timed region. The metric is the pages' own: TFLOPS = 18*T*D*H / time
("[RFC] Full-pipeline SwiGLU MLP with forward/backward co-optimization",
table "Training results"), reported beside the dense bf16 MFMA peak.

Prints one JSON line. Besides the contract fields it carries:
  roofline      the dominant kernel (largest summed time): algorithmic FLOPs
                per launch / its mean launch duration, timed with HIP events
                that the library records around each launch on the launch
                stream during the timed loop; HBM traffic per launch from
                rocprofv3 counters when the committed measurement matches the
                current kernel sources, else null.
  cpu_baseline  the fp64 oracle timed on the host cores on the first rows of
                the same workload (a bounded sample), in the same unit.
  stages        mean duration and TFLOP/s of every kernel.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W]
"""

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6  # MI355X dense bf16 MFMA: 256 CU * 2.4 GHz * 4096 FLOP/clk
PEAK_FP32_TFLOPS = 157.3
PEAK_HBM_GBS = 8000.0

# Algorithmic FLOPs of each kernel per launch, in units of T*D*H.
STAGE_FLOPS = {"gateup_swiglu": 4, "down_proj": 2, "dgu_inplace": 2, "dwd": 2, "dwgu": 4, "dx": 4,
               "infer_gateup": 4, "infer_down": 2, "dwd+dgu": 4, "dwgu+dx": 8}


def stage_bytes(name, T, D, H, e):
    """Algorithmic HBM bytes of one launch: each operand read once, each
    result written once (dG/dU read-modify-write in the in-place kernel)."""
    TD, TH, DH = T * D, T * H, D * H
    return e * {
        "gateup_swiglu": TD + 2 * DH + 3 * TH,
        "down_proj": TH + DH + TD,
        "dgu_inplace": TD + DH + 2 * TH + 2 * TH,
        "dwd": TH + TD + DH,
        "dwgu": TD + 2 * TH + 2 * DH,
        "dx": 2 * TH + 2 * DH + TD,
        "infer_gateup": TD + 2 * DH + TH,
        "infer_down": TH + DH + TD,
        "dwd+dgu": (TH + TD + DH) + (TD + DH + 4 * TH),
        "dwgu+dx": (TD + 2 * TH + 2 * DH) + (2 * TH + 2 * DH + TD),
    }[name]


def kernel_source_hash():
    h = hashlib.sha256()
    for f in ("gemm_tile.hpp", "swiglu_mlp.hip"):
        with open(os.path.join(ROOT, "backward_gate_up_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def load_traffic(kernel):
    """HBM bytes per launch measured with rocprofv3 (profiles/traffic.json),
    only if it was measured on the current kernel sources."""
    p = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(p):
        return None
    with open(p) as f:
        d = json.load(f)
    rec = d.get("kernels", {}).get(kernel)
    if not rec or d.get("source_sha256") != kernel_source_hash():
        return None
    return rec.get("hbm_bytes_per_launch")


def cpu_baseline(inp, D, H, target_s):
    """Time the fp64 oracle (fwd + bwd) on the first rows of the workload."""
    import numpy as np

    import oracle

    try:
        from threadpoolctl import threadpool_info

        threads = max([i.get("num_threads", 1) for i in threadpool_info()
                       if i.get("user_api") == "blas"] or [1])
    except Exception:  # pragma: no cover
        threads = len(os.sched_getaffinity(0))

    def run(rows):
        f = {k: inp[k][:rows].float().numpy() if k in ("X", "dY") else inp[k].float().numpy()
             for k in ("X", "Wg", "Wu", "Wd", "dY")}
        t0 = time.perf_counter()
        oracle.fwd(f["X"], f["Wg"], f["Wu"], f["Wd"])
        oracle.bwd(f["dY"], f["X"], f["Wg"], f["Wu"], f["Wd"])
        return time.perf_counter() - t0

    probe = 256
    t = run(probe)
    rows = int(min(16384, max(probe, (target_s / max(t, 1e-3)) * probe)) // 256 * 256)
    rows = max(rows, probe)
    t = run(rows) if rows != probe else t
    # fwd + bwd of the oracle: the forward is recomputed inside bwd, so the
    # oracle does 24*rows*D*H FLOPs; the metric counts the method's 18*T*D*H.
    tflops = 18.0 * rows * D * H / t / 1e12
    return {"value": round(tflops, 5), "unit": "TFLOPS", "cores": int(threads), "kind": "oracle",
            "sample": f"fwd+bwd on the first {rows} of the workload's rows (same weights), "
                      f"{t:.1f} s, numpy float64 BLAS"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="before timing, copy a buffer of this many MiB once (a plain copy kernel "
                         "of known traffic, used to calibrate rocprofv3 FETCH_SIZE/WRITE_SIZE)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: the fused SwiGLU MLP path runs on one GPU; multi-GPU runs are not "
              "supported. Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch

    import backward_gate_up_amd as mlp
    from synth import WORKLOADS, workload_inputs

    name = "mlp_4096x11008_T65536"
    D, H, B, S, _ = WORKLOADS[name]
    T = B * S
    dev = torch.device("cuda:0")
    inp = workload_inputs(name, dtype="bf16")
    g = {k: v.to(dev) for k, v in inp.items()}
    X, Wg, Wu, Wd, dY = (g[k] for k in ("X", "Wg", "Wu", "Wd", "dY"))
    bf = torch.bfloat16
    y = torch.empty((T, D), dtype=bf, device=dev)
    saved = torch.empty((3, T, H), dtype=bf, device=dev)
    dx = torch.empty((T, D), dtype=bf, device=dev)
    dwg = torch.empty((D, H), dtype=bf, device=dev)
    dwu = torch.empty((D, H), dtype=bf, device=dev)
    dwd = torch.empty((H, D), dtype=bf, device=dev)

    if args.copy_calibration_mib > 0:
        n = args.copy_calibration_mib << 20
        src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    def step():
        mlp.fwd(X, Wg, Wu, Wd, y=y, saved=saved)
        mlp.bwd(dY, X, Wg, Wu, Wd, saved, dx=dx, dwg=dwg, dwu=dwu, dwd=dwd)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    with mlp.StageTimer(capacity=max(args.steps, 1)) as st:
        torch.cuda.synchronize()
        e0.record()
        for _ in range(args.steps):
            step()
        e1.record()
        torch.cuda.synchronize()
    ms_step = e0.elapsed_time(e1) / args.steps
    flops = 18.0 * T * D * H
    tflops = flops / (ms_step * 1e-3) / 1e12

    stages = {}
    for s in STAGE_FLOPS:
        n = st.count[s]
        if n:
            ms = st.ms[s] / n
            stages[s] = {"ms": round(ms, 4),
                         "tflops": round(STAGE_FLOPS[s] * T * D * H / (ms * 1e-3) / 1e12, 1),
                         "frac_bf16_peak": round(STAGE_FLOPS[s] * T * D * H / (ms * 1e-3) / 1e12
                                                 / PEAK_BF16_TFLOPS, 4)}
    dom = max(stages, key=lambda s: stages[s]["ms"])
    dom_ms = stages[dom]["ms"]
    achieved = STAGE_FLOPS[dom] * T * D * H / (dom_ms * 1e-3) / 1e12
    roofline = {"bound": "mfma", "achieved": round(achieved, 1), "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                "traffic": load_traffic(dom), "kernel": dom,
                "flops_per_launch": STAGE_FLOPS[dom] * T * D * H,
                "algorithmic_bytes_per_launch": stage_bytes(dom, T, D, H, 2),
                "launch_ms": dom_ms}

    out = {
        "metric": "fwd+bwd TFLOPS (18*T*D*H), D=4096 H=11008 B=8 S=8192",
        "value": round(tflops, 2),
        "unit": "TFLOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "swiglu_mlp_fwd_bwd", "D": D, "H": H, "B": B, "S": S, "T": T,
                   "parallelism": "single-gpu"},
        "frac_bf16_peak": round(tflops / PEAK_BF16_TFLOPS, 4),
        "roofline": roofline,
        "stages": stages,
    }
    del g, X, Wg, Wu, Wd, dY, y, saved, dx, dwg, dwu, dwd
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(inp, D, H, args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
