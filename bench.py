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
  parity        (same leg) one more step in the timed launch configuration,
                sampled (one row per 32-row block, one hidden unit per
                32-unit block) and checked against the oracle: normalized L2
                per output, worst local error, epilogue ulp.
  sclk          the graphics clock (amdsmi) while the step repeats for 3 s
                after the timed steps.
  stages        mean duration and TFLOP/s of every kernel.
  infer         the no-grad sweep (B=1, S=1..256) against 8 TB/s and a
                same-run stream copy; fp32_ieee, tp_shards, linear_layout:
                the other legs.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--infer-only]
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
    """SHA-256 over every kernel source file (csrc/*.hip, *.hpp) and the header."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "backward_gate_up_amd", "csrc")
    files = sorted(os.path.join(csrc, f) for f in os.listdir(csrc) if f.endswith((".hip", ".hpp")))
    for path in files + [os.path.join(ROOT, "include", "swiglu_mlp.h")]:
        with open(path, "rb") as fh:
            h.update(os.path.basename(path).encode() + b"\0" + fh.read())
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

    # size the sample from a probe, then once more from the first sample
    # (a small probe overstates the per-row time: fixed costs dominate it)
    rows, t = 256, run(256)
    for _ in range(2):
        if t >= 0.6 * target_s or rows >= 65536:
            break
        rows = int(min(65536, max(rows, (target_s / max(t, 1e-3)) * rows)) // 256 * 256)
        t = run(rows)
    # fwd + bwd of the oracle: the forward is recomputed inside bwd, so the
    # oracle does 24*rows*D*H FLOPs; the metric counts the method's 18*T*D*H.
    tflops = 18.0 * rows * D * H / t / 1e12
    return {"value": round(tflops, 5), "unit": "TFLOPS", "cores": int(threads), "kind": "oracle",
            "sample": f"fwd+bwd on the first {rows} of the workload's rows (same weights), "
                      f"{t:.1f} s, numpy float64 BLAS"}


def measure_clock(torch, step, seconds=3.0, settle=1.5, period=0.05):
    """The graphics clock while the step runs: amdsmi's gpu_metrics
    (current_gfxclks, one value per XCD, in MHz) sampled every `period` s
    while the step repeats for `seconds`, outside the timed region. The
    metrics are refreshed about once a second, so samples from the first
    `settle` seconds (which can still show the idle clock) are dropped.
    Reported beside the fraction of peak, which is quoted at 2.4 GHz."""
    import threading

    try:
        import amdsmi

        amdsmi.amdsmi_init()
        hs = amdsmi.amdsmi_get_processor_handles()
        h = hs[0]
        if len(hs) > 1:
            bus = getattr(torch.cuda.get_device_properties(0), "pci_bus_id", None)
            for c in hs:
                if bus is not None and int(amdsmi.amdsmi_get_gpu_device_bdf(c).split(":")[1], 16) == bus:
                    h = c
    except Exception as e:  # pragma: no cover - reported as unavailable
        return {"error": repr(e)}
    samples, stop = [], threading.Event()
    t0 = time.perf_counter()

    def sample():
        while not stop.is_set():
            try:
                v = amdsmi.amdsmi_get_gpu_metrics_info(h).get("current_gfxclks")
                xs = [float(x) for x in (v if isinstance(v, (list, tuple)) else [v]) if isinstance(x, (int, float))]
                xs = [x for x in xs if 0 < x < 10000]
                if xs and time.perf_counter() - t0 >= settle:
                    samples.append(sum(xs) / len(xs))
            except Exception:
                pass
            stop.wait(period)

    th = threading.Thread(target=sample, daemon=True)
    th.start()
    while time.perf_counter() - t0 < seconds:
        step()
        torch.cuda.synchronize()
    stop.set()
    th.join()
    if not samples:
        return None
    xs = sorted(samples)
    return {"sclk_mhz_mean": round(sum(xs) / len(xs), 1), "sclk_mhz_min": round(xs[0], 1),
            "sclk_mhz_max": round(xs[-1], 1), "samples": len(xs),
            "source": f"amdsmi gpu_metrics current_gfxclks (mean over XCDs; refreshed about once a second), "
                      f"sampled every {period} s while the step repeated for {seconds} s after the timed "
                      f"steps; the first {settle} s dropped"}


def headline_sample(T, H, seed=65536):
    """The rows and hidden units the parity check samples: one row in every
    32-row block of the tokens and one hidden unit in every 32-unit block,
    which touches every 32 x 32 block row and every 256 x 256 tile of each
    output (including every weight-gradient tile split over K)."""
    import numpy as np

    rng = np.random.default_rng(seed)
    pick = lambda n: np.arange(0, n, 32) + rng.integers(0, np.minimum(32, n - np.arange(0, n, 32)))
    return pick(T), pick(H)


def gather_parity_sample(mlp, torch, g, T, H):
    """One more forward + backward in the timed launch configuration; keeps
    the sampled rows of Y, dI, A, G, U (after fwd), dG, dU (after bwd) and
    the sampled hidden units of dWg, dWu (columns) and dWd (rows), on the
    host."""
    rows, hs = headline_sample(T, H)
    r = torch.as_tensor(rows, device=g["X"].device)
    h = torch.as_tensor(hs, device=g["X"].device)
    y, saved = mlp.fwd(g["X"], g["Wg"], g["Wu"], g["Wd"])
    agu = [saved[i].index_select(0, r) for i in range(3)]
    dx, dwg, dwu, dwd = mlp.bwd(g["dY"], g["X"], g["Wg"], g["Wu"], g["Wd"], saved)
    out = {"Y": y.index_select(0, r), "dI": dx.index_select(0, r), "A": agu[0], "G": agu[1], "U": agu[2],
           "dG": saved[1].index_select(0, r), "dU": saved[2].index_select(0, r),
           "dWg": dwg.index_select(1, h).t(), "dWu": dwu.index_select(1, h).t(), "dWd": dwd.index_select(0, h)}
    torch.cuda.synchronize()
    out = {k: v.float().cpu().numpy().astype("float64") for k, v in out.items()}
    return rows, hs, out


def parity_vs_oracle(inp, rows, hs, got):
    """The sampled outputs against the fp64 oracle (part of the leg that runs
    the oracle on the host): normalized L2 per output over the sample, the
    worst per-line and per-segment (32 and 256 elements: the footprints of a
    matrix-core block and of a tile) local error, and the largest ulp
    distance of A from rnd(SiLU(g) u) of the stored g, u."""
    import numpy as np

    import oracle

    f = {k: inp[k].float().numpy() for k in ("X", "Wg", "Wu", "Wd", "dY")}
    r = oracle.rows(rows, f["X"], f["Wg"], f["Wu"], f["Wd"], f["dY"])
    c = oracle.cols(hs, f["X"], f["Wg"], f["Wu"], f["Wd"], f["dY"])
    ref = {"Y": r["Y"], "dI": r["dI"], "G": r["G"], "U": r["U"], "dG": r["dG"], "dU": r["dU"],
           "dWg": c["dWg"].T, "dWu": c["dWu"].T, "dWd": c["dWd"]}

    def local(a, b, seg):
        d, n = a - b, b.shape[1]
        floor = np.sqrt(np.mean(b * b))
        w = -n % seg
        dd = np.pad(d, ((0, 0), (0, w))).reshape(b.shape[0], -1, seg)
        bb = np.pad(b, ((0, 0), (0, w))).reshape(b.shape[0], -1, seg)
        cnt = np.pad(np.ones_like(b), ((0, 0), (0, w))).reshape(b.shape[0], -1, seg).sum(-1)
        e = np.sqrt((dd * dd).sum(-1) / cnt) / np.maximum(np.sqrt((bb * bb).sum(-1) / cnt), floor)
        return float(e.max())

    nl2, worst = {}, {}
    for k, b in ref.items():
        a = got[k]
        nl2[k] = float(np.linalg.norm(a - b) / np.linalg.norm(b))
        worst[k] = max(local(a, b, b.shape[1]), local(a, b, 32), local(a, b, 256))
    a_ref = oracle.round_to(oracle.epilogue_fwd(got["G"], got["U"]), "bf16")
    ulp = int(oracle.ulp_distance(got["A"], a_ref, "bf16").max())
    ok = all(v <= 1e-2 for v in nl2.values()) and all(v <= 1e-2 for v in worst.values()) and ulp <= 1
    return {"sample": f"{len(rows)} rows (one per 32-row block) of Y, dI, G, U, dG, dU and {len(hs)} hidden "
                      "units (one per 32-unit block) of dWg, dWu, dWd, from one more step in the timed "
                      "launch configuration",
            "normalized_l2": {k: float(f"{v:.3e}") for k, v in nl2.items()},
            "worst_local": {k: float(f"{v:.3e}") for k, v in worst.items()},
            "epilogue_max_ulp": ulp, "tolerance": 1e-2, "pass": bool(ok)}


def stream_copy_gbps(torch, dev, mib=1024, reps=10):
    """A plain device-to-device copy of `mib` MiB (read + write), timed with
    HIP events in the same run: the achievable-bandwidth reference for the
    no-grad rows (GB/s counts both directions)."""
    src = torch.ones(mib << 18, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(2):
        dst.copy_(src)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        dst.copy_(src)
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / reps
    del src, dst
    return round(2 * (mib << 20) / (ms * 1e-3) / 1e9, 1)


def infer_sweep(mlp, torch, dev, reps=20, copy_gbps=None):
    """No-grad path at B=1, S in {1..256}, D/H in {1024/2816, 4096/11008}: device
    time per call (HIP events around the call only) with the 256 MB Infinity
    Cache flushed before every timed call by reading a 1 GiB buffer outside the
    events, and HBM GB/s from the call's algorithmic bytes
    2*(3*D*H + 2*T*D + 2*T*H), against 8 TB/s and against the same run's
    stream copy. A flush that writes leaves the caches full of dirty lines
    whose write-back then competes with the call's reads; that time is
    reported beside it (us_write_flush).
    Also the host-inclusive wall time of one call (Python binding, argument
    checks, the launches, completion), eagerly and as a replay of a HIP graph
    that captured the same call (checked bitwise against the eager output),
    measured alternately after warm-up replays; the same per call for eight
    calls back to back (eagerly, and as one graph of all eight: a decode
    step through eight layers); and the intermediate memory of the call
    (workspace + Y) beside A + Y."""
    from synth import INFER_DH, INFER_S, make_inputs

    flush = torch.ones(1 << 28, dtype=torch.float32, device=dev)  # 1 GiB
    out = {}
    for D, H in INFER_DH:
        w = make_inputs(1, D, H, seed=77, dtype="bf16", with_dy=False)
        Wg, Wu, Wd = (w[k].to(dev) for k in ("Wg", "Wu", "Wd"))
        rows = {}
        for S in INFER_S:
            X = make_inputs(S, D, H, seed=S, dtype="bf16", with_dy=False)["X"].to(dev)
            y = torch.empty((S, D), dtype=torch.bfloat16, device=dev)
            ws = torch.empty(mlp.infer_workspace_bytes(S, D, H), dtype=torch.uint8, device=dev)
            for _ in range(3):
                mlp.infer(X, Wg, Wu, Wd, y=y, workspace=ws)

            def device_us(write):
                ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                      for _ in range(reps)]
                for a, b in ev:
                    if write:
                        flush.fill_(1.0)
                    else:
                        flush.sum()
                    a.record()
                    mlp.infer(X, Wg, Wu, Wd, y=y, workspace=ws)
                    b.record()
                torch.cuda.synchronize()
                us = sorted(a.elapsed_time(b) * 1e3 for a, b in ev)
                return us[len(us) // 2]

            med = device_us(False)
            med_w = device_us(True)
            nbytes = 2 * (3 * D * H + 2 * S * D + 2 * S * H)

            y_eager = y.clone()
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph):
                mlp.infer(X, Wg, Wu, Wd, y=y, workspace=ws)
            y.zero_()
            graph.replay()
            torch.cuda.synchronize()
            same = bool(torch.equal(y, y_eager))
            for _ in range(5):
                graph.replay()
            torch.cuda.synchronize()
            eager_call = lambda: mlp.infer(X, Wg, Wu, Wd, y=y, workspace=ws)
            t_e, t_g = [], []
            for _ in range(reps):
                for call, ts in ((eager_call, t_e), (graph.replay, t_g)):
                    flush.sum()
                    torch.cuda.synchronize()
                    t0 = time.perf_counter()
                    call()
                    torch.cuda.synchronize()
                    ts.append((time.perf_counter() - t0) * 1e6)
            del graph
            # eight calls back to back (a decode step through eight layers):
            # eager, and replayed from one graph that captured all eight
            g8 = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g8):
                for _ in range(8):
                    mlp.infer(X, Wg, Wu, Wd, y=y, workspace=ws)
            for _ in range(3):
                g8.replay()
            eager8 = lambda: [mlp.infer(X, Wg, Wu, Wd, y=y, workspace=ws) for _ in range(8)]
            t_e8, t_g8 = [], []
            for _ in range(reps // 2):
                for call, ts in ((eager8, t_e8), (g8.replay, t_g8)):
                    flush.sum()
                    torch.cuda.synchronize()
                    t0 = time.perf_counter()
                    call()
                    torch.cuda.synchronize()
                    ts.append((time.perf_counter() - t0) * 1e6 / 8)
            del g8
            gbps = nbytes / (med * 1e-6) / 1e9
            a_y = 2 * S * (H + D)
            inter = ws.numel() + 2 * S * D
            rows[str(S)] = {"us": round(med, 2), "us_write_flush": round(med_w, 2),
                            "GBps": round(gbps, 1), "frac_hbm": round(gbps / PEAK_HBM_GBS, 3),
                            "frac_copy": round(gbps / copy_gbps, 3) if copy_gbps else None,
                            "wall_us_eager": round(sorted(t_e)[reps // 2], 1),
                            "wall_us_graph": round(sorted(t_g)[reps // 2], 1),
                            "graph_bitwise_equal": same,
                            "wall_us_per_call_8_eager": round(sorted(t_e8)[len(t_e8) // 2], 1),
                            "wall_us_per_call_8_graph": round(sorted(t_g8)[len(t_g8) // 2], 1),
                            "intermediate_MiB": round(inter / 2**20, 3),
                            "intermediate_over_A_plus_Y": round(inter / a_y, 3)}
        out[f"{D}x{H}"] = rows
    del flush
    return out


def vendor_gemm(torch, dev, reps=10):
    """Context, not part of the step: hipBLASLt (torch.mm) on two of the
    step's GEMM shapes at D=4096, H=11008, T=65536, without the fused
    epilogues. dI's shape with both operands K-major ([T, 2H] times a
    transposed [D, 2H]), and gate/up's with X K-major and [Wg | Wu] N-major.
    Timed with events on torch's stream after two warm-up calls."""
    T, D, H = 65536, 4096, 11008
    bf = torch.bfloat16
    gen = torch.Generator(device=dev)
    gen.manual_seed(0)
    out = {}

    def run(name, a, b):
        for _ in range(2):
            c = torch.mm(a, b)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            c = torch.mm(a, b)
        e1.record()
        torch.cuda.synchronize()
        del c
        ms = e0.elapsed_time(e1) / reps
        tf = 2.0 * a.shape[0] * a.shape[1] * b.shape[1] / ms / 1e9
        out[name] = {"ms": round(ms, 4), "tflops": round(tf, 1), "frac_bf16_peak": round(tf / PEAK_BF16_TFLOPS, 4)}

    dg = torch.randn(T, 2 * H, device=dev, dtype=bf, generator=gen)
    w = torch.randn(D, 2 * H, device=dev, dtype=bf, generator=gen)
    run("dI_shape_KxK", dg, w.t())
    del dg, w
    x = torch.randn(T, D, device=dev, dtype=bf, generator=gen)
    wgu = torch.randn(D, 2 * H, device=dev, dtype=bf, generator=gen)
    run("gateup_shape_KxN", x, wgu)
    return out


def ingest_vendor(pass_a_csv, out_md, command):
    """Clock and matrix-core occupancy of the hipBLASLt kernels of
    `bench.py --vendor-gemm` from one counter pass (the same counters and
    formulas as ingest_counters). The GEMM kernels (names containing "Cijk")
    are told apart by order of first appearance: dI's shape, then
    gate/up's. Means over the last 4 dispatches of each."""
    import csv
    from collections import OrderedDict, defaultdict

    per = OrderedDict()
    with open(pass_a_csv) as f:
        for r in csv.DictReader(f):
            n = r["Kernel_Name"]
            if "Cijk" not in n:
                continue
            d = per.setdefault(n, defaultdict(dict))[r["Dispatch_Id"]]
            d[r["Counter_Name"]] = d.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
            d["dur_ns"] = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
    labels = ["dI shape, both K-major", "gate/up shape, X K-major, W N-major"]
    lines = ["| GEMM | kernel | ms | sclk GHz | MFMA busy % | effective % of peak | wait % |",
             "|---|---|---|---|---|---|---|"]
    for label, (name, disp) in zip(labels, per.items()):
        rows = [disp[k] for k in sorted(disp, key=int)][-4:]
        ms = sum(r["dur_ns"] for r in rows) / len(rows) / 1e6
        cyc = sum(r["GRBM_GUI_ACTIVE"] for r in rows) / len(rows) / 8
        sclk = cyc / (ms * 1e-3) / 1e9
        busy = sum(r["SQ_VALU_MFMA_BUSY_CYCLES"] for r in rows) / len(rows) / (cyc * 1024)
        wait = sum(r["SQ_WAIT_ANY"] for r in rows) / max(sum(r["SQ_WAVE_CYCLES"] for r in rows), 1)
        short = name if len(name) <= 60 else name[:57] + "..."
        lines.append(f"| {label} | `{short}` | {ms:.3f} | {sclk:.2f} | {100 * busy:.1f} | "
                     f"{100 * sclk * busy / 2.4:.1f} | {100 * wait:.1f} |")
    head = ("# hipBLASLt at two of the step's GEMM shapes (context): clock and matrix-core occupancy, bf16\n\n"
            "D=4096, H=11008, T=65536, plain GEMMs through torch.mm, no fused epilogue. Commands (repository "
            f"root, one MI355X):\n\n```\n{command}\n```\n\n"
            "ms: duration of each dispatch in the counter run (kernels run one at a time there). sclk: "
            "GRBM_GUI_ACTIVE / 8 over the duration. MFMA busy: SQ_VALU_MFMA_BUSY_CYCLES / (per-XCD cycles x "
            "1024 SIMDs). Effective % of peak: sclk x busy / 2.4 GHz. Wait %: SQ_WAIT_ANY / SQ_WAVE_CYCLES. "
            "The same counters for this repository's kernels are in counters_swiglu_fwd_bwd_T65536_bf16.md.\n\n")
    with open(out_md, "w") as f:
        f.write(head + "\n".join(lines) + "\n")
    print(head + "\n".join(lines))


def fp32_leg(mlp, torch, dev, steps=10, warmup=3):
    """True-IEEE fp32 mode at D=2048, H=5632, B=8, S=512 (T=4096): mean step time
    of fwd + bwd and TFLOP/s (18*T*D*H) against the fp32 matrix peak."""
    from synth import WORKLOADS, workload_inputs

    name = "mlp_2048x5632_T4096_fp32"
    D, H, B, S, _ = WORKLOADS[name]
    T = B * S
    g = {k: v.to(dev) for k, v in workload_inputs(name, dtype="fp32").items()}
    f32 = torch.float32
    y = torch.empty((T, D), dtype=f32, device=dev)
    saved = torch.empty((3, T, H), dtype=f32, device=dev)
    dx = torch.empty((T, D), dtype=f32, device=dev)
    dwg, dwu = (torch.empty((D, H), dtype=f32, device=dev) for _ in range(2))
    dwd = torch.empty((H, D), dtype=f32, device=dev)

    def step():
        mlp.fwd(g["X"], g["Wg"], g["Wu"], g["Wd"], y=y, saved=saved)
        mlp.bwd(g["dY"], g["X"], g["Wg"], g["Wu"], g["Wd"], saved, dx=dx, dwg=dwg, dwu=dwu, dwd=dwd)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(steps):
        step()
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / steps
    tf = 18.0 * T * D * H / (ms * 1e-3) / 1e12
    return {"config": {"D": D, "H": H, "B": B, "S": S, "T": T}, "dtype": "f32", "ms_per_step": round(ms, 3),
            "tflops": round(tf, 2), "peak_tflops": PEAK_FP32_TFLOPS, "frac_fp32_peak": round(tf / PEAK_FP32_TFLOPS, 4)}


def linear_layout_leg(mlp, torch, g, T, D, H, steps=10, warmup=3):
    """The headline step with the weights in the nn.Linear layout (gate_proj,
    up_proj [H, D], down_proj [D, H]; the forward GEMMs read K-major weights,
    dA and dI N-major ones), same inputs: mean step time and TFLOP/s."""
    wl = {k: g[k].t().contiguous() for k in ("Wg", "Wu", "Wd")}
    bf = torch.bfloat16
    dev = g["X"].device
    y, saved = torch.empty((T, D), dtype=bf, device=dev), torch.empty((3, T, H), dtype=bf, device=dev)
    dx = torch.empty((T, D), dtype=bf, device=dev)
    dwg, dwu, dwd = (torch.empty_like(wl[k]) for k in ("Wg", "Wu", "Wd"))

    def step():
        mlp.fwd(g["X"], wl["Wg"], wl["Wu"], wl["Wd"], y=y, saved=saved, linear=True)
        mlp.bwd(g["dY"], g["X"], wl["Wg"], wl["Wu"], wl["Wd"], saved, dx=dx, dwg=dwg, dwu=dwu, dwd=dwd,
                linear=True)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    with mlp.StageTimer(capacity=steps) as st:
        a.record()
        for _ in range(steps):
            step()
        b.record()
        torch.cuda.synchronize()
    ms = a.elapsed_time(b) / steps
    tf = 18.0 * T * D * H / (ms * 1e-3) / 1e12
    stages = {k: round(v / st.count[k], 4) for k, v in st.ms.items() if st.count[k]}
    return {"ms_per_step": round(ms, 3), "tflops": round(tf, 1), "frac_bf16_peak": round(tf / PEAK_BF16_TFLOPS, 4),
            "stage_ms": stages}


def tp_shard_sweep(mlp, torch, dev, T, D, H, steps=5, warmup=2):
    """Tensor-parallel shard shapes on one GPU: the same step at H/P for
    P in {2, 4, 8} (Wg, Wu split by columns and Wd by rows; each GPU of a
    TP group runs exactly this). Synthetic bf16 inputs of the headline's
    scales; TFLOP/s = 18*T*D*(H/P) / mean step time."""
    out = {}
    g = torch.Generator(device=dev).manual_seed(5)
    bf = torch.bfloat16
    X = torch.randn(T, D, device=dev, generator=g).to(bf)
    dY = torch.randn(T, D, device=dev, generator=g).to(bf)
    for P in (2, 4, 8):
        h = H // P
        Wg = (torch.randn(D, h, device=dev, generator=g) / D ** 0.5).to(bf)
        Wu = (torch.randn(D, h, device=dev, generator=g) / D ** 0.5).to(bf)
        Wd = (torch.randn(h, D, device=dev, generator=g) / H ** 0.5).to(bf)
        y, saved = torch.empty((T, D), dtype=bf, device=dev), torch.empty((3, T, h), dtype=bf, device=dev)
        dx = torch.empty((T, D), dtype=bf, device=dev)
        dwg, dwu = (torch.empty((D, h), dtype=bf, device=dev) for _ in range(2))
        dwd = torch.empty((h, D), dtype=bf, device=dev)

        def step():
            mlp.fwd(X, Wg, Wu, Wd, y=y, saved=saved)
            mlp.bwd(dY, X, Wg, Wu, Wd, saved, dx=dx, dwg=dwg, dwu=dwu, dwd=dwd)

        for _ in range(warmup):
            step()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(steps):
            step()
        b.record()
        torch.cuda.synchronize()
        ms = a.elapsed_time(b) / steps
        tf = 18.0 * T * D * h / (ms * 1e-3) / 1e12
        out[f"P={P}"] = {"H_shard": h, "ms_per_step": round(ms, 3), "tflops": round(tf, 1),
                         "frac_bf16_peak": round(tf / PEAK_BF16_TFLOPS, 4)}
        del Wg, Wu, Wd, y, saved, dx, dwg, dwu, dwd
    return out


def ingest_traffic(fetch_csv, write_csv, copy_mib, command):
    """Turn two rocprofv3 --pmc runs of `bench.py --copy-calibration-mib N`
    (FETCH_SIZE, then WRITE_SIZE; KiB per dispatch) into profiles/traffic.json.
    Each counter is scaled by what it reads for the plain copy kernel of known
    size in the same run (copy: N MiB read + N MiB written), then averaged per
    launch of each stage (stage = last template argument of the kernel)."""
    import csv
    import re
    from collections import defaultdict

    from backward_gate_up_amd._lib import STAGE_NAMES

    def per_dispatch(path, counter):
        vals, names = defaultdict(float), {}
        with open(path) as f:
            for r in csv.DictReader(f):
                if r["Counter_Name"] == counter:
                    k = int(r["Dispatch_Id"])
                    vals[k] += float(r["Counter_Value"]) * 1024.0
                    names[k] = r["Kernel_Name"]
        return vals, names

    known = copy_mib << 20
    out = {"source_sha256": kernel_source_hash(), "command": command, "kernels": {}}
    res = {}
    for key, path, counter in (("fetch", fetch_csv, "FETCH_SIZE"), ("write", write_csv, "WRITE_SIZE")):
        vals, names = per_dispatch(path, counter)
        copies = [v for k, v in vals.items() if "copyBuffer" in names[k] or "copy" in names[k].lower()]
        if not copies:
            raise SystemExit(f"no copy kernel found in {path}")
        factor = known / copies[0]
        out[f"{key}_factor"] = round(factor, 4)
        per_stage = defaultdict(list)
        for k, v in vals.items():
            m = re.search(r"(mlp_gemm|mlp_gemm_pair|ring_gemm|ring_wgrad)<.*,\s*(\d+)>\(", names[k])
            if m:
                per_stage[STAGE_NAMES[int(m.group(2))]].append(v * factor)
        res[key] = {st: sum(v) / len(v) for st, v in per_stage.items()}
    for st in res["fetch"]:
        f, w = res["fetch"][st], res["write"].get(st, 0.0)
        out["kernels"][st] = {"fetch_bytes_per_launch": int(f), "write_bytes_per_launch": int(w),
                              "hbm_bytes_per_launch": int(f + w)}
    path = os.path.join(ROOT, "profiles", "traffic.json")
    with open(path, "w") as fh:
        json.dump(out, fh, indent=1)
    print(json.dumps(out, indent=1))


def ingest_counters(trace_csv, pass_a_csv, pass_b_csv, out_md, command):
    """Per-kernel clock, matrix-core occupancy, stalls and traffic of the
    training step from a kernel trace and two counter passes of
    `bench.py --steps 2 --warmup 1 --no-infer --no-fp32 --no-tp --no-linear
    --no-cpu-baseline`, with profiles/traffic.json (FETCH/WRITE) when it
    matches the sources. Means over every launch of each kernel.
      sclk: GRBM_GUI_ACTIVE / 8 (rocprofv3 sums the 8 XCDs) / duration;
      MFMA busy: SQ_VALU_MFMA_BUSY_CYCLES / (per-XCD cycles x 1024 SIMDs);
      effective % of peak: sclk x busy / 2.4 GHz;
      wait: SQ_WAIT_ANY / SQ_WAVE_CYCLES (waves in s_waitcnt), LDS wait:
      SQ_WAIT_INST_LDS / SQ_WAVE_CYCLES, LDS conflict: SQ_LDS_BANK_CONFLICT
      / SQ_LDS_IDX_ACTIVE, TA FIFO full: SQ_VMEM_TA_ADDR_FIFO_FULL per
      CU-cycle."""
    import csv
    import re
    from collections import defaultdict

    from backward_gate_up_amd._lib import STAGE_NAMES

    def key(n):
        m = re.search(r"(ring_gemm|ring_wgrad)<[^>]*?(\d+)>\(", n)
        return STAGE_NAMES[int(m.group(2))] if m else None

    dur = defaultdict(list)
    with open(trace_csv) as f:
        for r in csv.DictReader(f):
            k = key(r["Kernel_Name"])
            if k:
                dur[k].append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e6)
    cnt = defaultdict(lambda: defaultdict(float))
    disp = defaultdict(set)
    for path in (pass_a_csv, pass_b_csv):
        with open(path) as f:
            for r in csv.DictReader(f):
                k = key(r["Kernel_Name"])
                if k:
                    cnt[k][r["Counter_Name"]] += float(r["Counter_Value"])
                    disp[(k, path)].add(r["Dispatch_Id"])
    traffic = {}
    tp = os.path.join(ROOT, "profiles", "traffic.json")
    if os.path.exists(tp):
        with open(tp) as f:
            t = json.load(f)
        if t.get("source_sha256") == kernel_source_hash():
            traffic = t["kernels"]
    order = ["gateup_swiglu", "down_proj", "dgu_inplace", "dwd", "dwgu", "dx"]
    lines = ["| kernel | ms | sclk GHz | MFMA busy % | effective % of peak | wait % | LDS wait % | "
             "LDS conflict % | TA FIFO full % | fetch GB | write GB |",
             "|---|---|---|---|---|---|---|---|---|---|---|"]
    for k in order:
        if k not in cnt or not dur.get(k):
            continue
        c = cnt[k]
        na = len(disp[(k, pass_a_csv)]) or 1
        nb = len(disp[(k, pass_b_csv)]) or 1
        sel = dur[k][2:7] or dur[k]  # the timed launches of the trace run (2 warm-up, 5 timed steps)
        ms = sum(sel) / len(sel)
        # GRBM_GUI_ACTIVE is in both passes: per-dispatch means of each
        cyc = c["GRBM_GUI_ACTIVE"] / (na + nb) / 8
        sclk = cyc / (ms * 1e-3) / 1e9
        busy = c["SQ_VALU_MFMA_BUSY_CYCLES"] / na / (cyc * 1024)
        wave = c["SQ_WAVE_CYCLES"] / na
        tr = traffic.get(k, {})
        lines.append(f"| {k} | {ms:.3f} | {sclk:.2f} | {100 * busy:.1f} | {100 * sclk * busy / 2.4:.1f} | "
                     f"{100 * c['SQ_WAIT_ANY'] / na / wave:.1f} | {100 * c['SQ_WAIT_INST_LDS'] / na / wave:.1f} | "
                     f"{100 * c['SQ_LDS_BANK_CONFLICT'] / max(c['SQ_LDS_IDX_ACTIVE'], 1):.1f} | "
                     f"{100 * c['SQ_VMEM_TA_ADDR_FIFO_FULL'] / nb / (cyc * 256):.1f} | "
                     f"{tr.get('fetch_bytes_per_launch', float('nan')) / 1e9:.2f} | "
                     f"{tr.get('write_bytes_per_launch', float('nan')) / 1e9:.2f} |")
    head = ("# Clock, matrix-core occupancy, stalls and traffic: fused SwiGLU MLP fwd+bwd, D=4096 H=11008 "
            "T=65536, bf16\n\nCommands (repository root, one MI355X; each pass a run of its own):\n\n```\n"
            f"{command}\n```\n\n"
            "Means over every launch of each kernel (the warm-up and timed steps of each run). ms: the kernel "
            "trace (timed steps). sclk: GRBM_GUI_ACTIVE / 8 (rocprofv3 sums the 8 XCDs) over the kernel's duration. MFMA "
            "busy: SQ_VALU_MFMA_BUSY_CYCLES / (per-XCD cycles x 1024 SIMDs). Effective % of peak: sclk x busy "
            "/ 2.4 GHz, the clock the 2516.6 TFLOP/s peak is quoted at. Wait %: SQ_WAIT_ANY / SQ_WAVE_CYCLES "
            "(wave-cycles in s_waitcnt, for loads or LDS). LDS wait %: SQ_WAIT_INST_LDS / SQ_WAVE_CYCLES. LDS "
            "conflict %: SQ_LDS_BANK_CONFLICT / SQ_LDS_IDX_ACTIVE. TA FIFO full %: SQ_VMEM_TA_ADDR_FIFO_FULL "
            "per CU-cycle (the texture unit's address queue refusing further loads). Fetch and write: "
            "profiles/traffic.json (FETCH_SIZE, WRITE_SIZE scaled by a 1 GiB copy in the same run), per "
            "launch.\n\n")
    with open(out_md, "w") as f:
        f.write(head + "\n".join(lines) + "\n")
    print(head + "\n".join(lines))


def ingest_trace(trace_csv, out_md, command, warmup=2, timed=5):
    """Per-kernel durations of the training step from a rocprofv3 kernel
    trace (csv) of `bench.py --steps 5 --warmup 2 --no-infer
    --no-cpu-baseline --no-fp32 --no-tp --no-linear`: the mean over the last
    `timed` launches of each ring kernel after `warmup`, plus the split-K
    reduction that
    follows each weight-gradient launch, with TFLOP/s, algorithmic bytes and
    the traffic of profiles/traffic.json when it matches the sources."""
    import csv
    import re
    from collections import defaultdict

    from backward_gate_up_amd._lib import STAGE_NAMES

    with open(trace_csv) as f:
        rows = sorted(csv.DictReader(f), key=lambda r: int(r["Start_Timestamp"]))
    dur, red, names = defaultdict(list), defaultdict(list), {}
    last = None
    for r in rows:
        n = r["Kernel_Name"]
        d = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e6
        m = re.search(r"(ring_gemm|ring_wgrad)<[^>]*?(\d+)>\(", n)
        if m:
            last = STAGE_NAMES[int(m.group(2))]
            dur[last].append(d)
            names[last] = re.sub(r"\(.*", "", n).replace("void ", "")
        elif "splitk_reduce_tiles" in n and last:
            red[last].append(d)
    T, D, H = 65536, 4096, 11008
    traffic = {}
    tp = os.path.join(ROOT, "profiles", "traffic.json")
    if os.path.exists(tp):
        with open(tp) as f:
            t = json.load(f)
        if t.get("source_sha256") == kernel_source_hash():
            traffic = t["kernels"]
    lines = ["| kernel | stage | trace ms | reduction ms | stage ms | TFLOP/s | % of peak | algorithmic GB | "
             "fetch GB | write GB |", "|---|---|---|---|---|---|---|---|---|---|"]
    total = 0.0
    for st in ("gateup_swiglu", "down_proj", "dgu_inplace", "dwd", "dwgu", "dx"):
        if not dur.get(st):
            continue
        sel = dur[st][warmup:warmup + timed]
        ms = sum(sel) / len(sel)
        rsel = red[st][warmup:warmup + timed] if red.get(st) else []
        rd = sum(rsel) / len(rsel) if rsel else 0.0
        tf = STAGE_FLOPS[st] * T * D * H / ((ms + rd) * 1e-3) / 1e12
        total += ms + rd
        tr = traffic.get(st, {})
        lines.append(f"| `{names[st]}` | {st} | {ms:.3f} | {rd:.3f} | {ms + rd:.3f} | {tf:.0f} | "
                     f"{100 * tf / PEAK_BF16_TFLOPS:.1f} | {stage_bytes(st, T, D, H, 2) / 1e9:.2f} | "
                     f"{tr.get('fetch_bytes_per_launch', float('nan')) / 1e9:.2f} | "
                     f"{tr.get('write_bytes_per_launch', float('nan')) / 1e9:.2f} |")
    head = ("# Kernel trace: fused SwiGLU MLP fwd+bwd, D=4096 H=11008 T=65536 (B=8, S=8192), bf16\n\n"
            f"Command (repository root, one MI355X):\n\n```\n{command}\n```\n\n"
            f"Means over launches {warmup + 1} to {warmup + timed} of each kernel (the timed steps). The "
            "weight-gradient "
            "stages are two launches: the ring kernel, then `splitk_reduce_tiles` adding the fp32 partial "
            "tiles of the tiles split over K. TFLOP/s from each stage's algorithmic FLOPs (4, 2, 2, 2, 4, 4 "
            "x T D H). Algorithmic bytes: each operand read once, each result written once. Fetch / write: "
            "profiles/traffic.json.\n\n")
    tail = (f"\nStage times sum to {total:.2f} ms per step = {18.0 * T * D * H / (total * 1e-3) / 1e12:.0f} "
            f"TFLOP/s ({100 * 18.0 * T * D * H / (total * 1e-3) / 1e12 / PEAK_BF16_TFLOPS:.1f} % of dense "
            "bf16 peak).\n")
    with open(out_md, "w") as f:
        f.write(head + "\n".join(lines) + "\n" + tail)
    print(head + "\n".join(lines) + "\n" + tail)


INFER_TRACE_CALLS = 3


def infer_trace(mlp, torch, dev):
    """A fixed, short sequence of no-grad calls for rocprofv3: a 1 GiB copy
    (the counters' calibration kernel: 1 GiB read + 1 GiB written), then for
    each shape of the sweep, in order, INFER_TRACE_CALLS calls, each after a
    read of a 1 GiB buffer that flushes the 256 MB cache. ingest_infer maps
    the dispatches back to the shapes by this order."""
    from synth import INFER_DH, INFER_S, make_inputs

    src = torch.ones(1 << 28, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    dst.copy_(src)
    del dst
    order = []
    for D, H in INFER_DH:
        w = make_inputs(1, D, H, seed=77, dtype="bf16", with_dy=False)
        Wg, Wu, Wd = (w[k].to(dev) for k in ("Wg", "Wu", "Wd"))
        for S in INFER_S:
            X = make_inputs(S, D, H, seed=S, dtype="bf16", with_dy=False)["X"].to(dev)
            ws = torch.empty(mlp.infer_workspace_bytes(S, D, H), dtype=torch.uint8, device=dev)
            y = torch.empty((S, D), dtype=torch.bfloat16, device=dev)
            for _ in range(INFER_TRACE_CALLS):
                src.sum()
                mlp.infer(X, Wg, Wu, Wd, y=y, workspace=ws)
            order.append([D, H, S])
    torch.cuda.synchronize()
    return order


def ingest_infer(trace_csv, fetch_csv, write_csv, out_md, command):
    """Summarise a kernel trace and FETCH_SIZE / WRITE_SIZE counter passes of
    `bench.py --infer-trace` (three runs of the same command) as a table per
    shape: kernels, device time of the call (first kernel start to last
    kernel end, mean over the calls), algorithmic GB/s, and the counters'
    bytes scaled by what they read for the 1 GiB copy."""
    import csv
    import re
    from collections import defaultdict

    from synth import INFER_DH, INFER_S

    ours = lambda n: "swiglu::" in n
    with open(trace_csv) as f:
        rows = sorted(csv.DictReader(f), key=lambda r: int(r["Start_Timestamp"]))
    calls = []  # one list of (name, start, end) per call
    for r in rows:
        n = r["Kernel_Name"]
        if not ours(n):
            if calls and calls[-1]:
                calls.append([])
            continue
        if not calls:
            calls.append([])
        calls[-1].append((n, int(r["Start_Timestamp"]), int(r["End_Timestamp"])))
    calls = [c for c in calls if c]
    shapes = [(D, H, S) for D, H in INFER_DH for S in INFER_S]
    assert len(calls) == len(shapes) * INFER_TRACE_CALLS, (len(calls), len(shapes))

    def counters(path, counter):
        per, names = defaultdict(float), {}
        with open(path) as f:
            for r in csv.DictReader(f):
                if r["Counter_Name"] == counter:
                    k = int(r["Dispatch_Id"])
                    per[k] += float(r["Counter_Value"]) * 1024.0
                    names[k] = r["Kernel_Name"]
        ids = sorted(per)
        copy = [per[k] for k in ids if "copy" in names[k].lower()][0]
        seq = [per[k] for k in ids if ours(names[k])]
        return seq, copy

    fetch, fcopy = counters(fetch_csv, "FETCH_SIZE")
    write, wcopy = counters(write_csv, "WRITE_SIZE")
    ff, wf = (1 << 30) / fcopy, (1 << 30) / wcopy
    short = lambda n: re.sub(r"\(.*", "", n).replace("void ", "").replace("swiglu::", "")
    lines = ["| D -> H | S | kernels | device us | algorithmic GB/s | % of 8 TB/s | fetch MB | write MB |",
             "|---|---|---|---|---|---|---|---|"]
    i = k = 0
    for D, H, S in shapes:
        cs = calls[i:i + INFER_TRACE_CALLS]
        i += INFER_TRACE_CALLS
        nk = len(cs[0])
        us = sum((c[-1][2] - c[0][1]) / 1e3 for c in cs) / len(cs)
        fb = sum(fetch[k:k + nk * INFER_TRACE_CALLS]) * ff / INFER_TRACE_CALLS
        wb = sum(write[k:k + nk * INFER_TRACE_CALLS]) * wf / INFER_TRACE_CALLS
        k += nk * INFER_TRACE_CALLS
        nbytes = 2 * (3 * D * H + 2 * S * D + 2 * S * H)
        gbps = nbytes / (us * 1e-6) / 1e9
        names = " + ".join(f"`{short(n)}` {(e - b) / 1e3:.1f}" for n, b, e in cs[-1])
        lines.append(f"| {D} -> {H} | {S} | {names} | {us:.1f} | {gbps:.0f} | {100 * gbps / PEAK_HBM_GBS:.0f} | "
                     f"{fb / 1e6:.1f} | {wb / 1e6:.1f} |")
    head = (f"# No-grad SwiGLU MLP, B=1, S=1..256, bf16: kernel trace and HBM traffic\n\n"
            f"Commands (repository root, one MI355X; three runs of the same program):\n\n```\n{command}\n```\n\n"
            f"Each call follows a read of a 1 GiB buffer (the 256 MB cache holds no weights). Device us: from the "
            f"first kernel's start to the last kernel's end, mean over {INFER_TRACE_CALLS} calls; the kernels "
            f"column gives the last call's kernels and their us. Algorithmic bytes: 2 (3 D H + 2 S D + 2 S H). "
            f"Fetch and write: FETCH_SIZE and WRITE_SIZE summed over the call's kernels, scaled by what they "
            f"read for the 1 GiB copy in the same run (fetch x{ff:.3f}, write x{wf:.3f}). FETCH_SIZE counts "
            f"what L2 requests from the fabric, so it includes bytes the Infinity Cache serves.\n\n")
    with open(out_md, "w") as f:
        f.write(head + "\n".join(lines) + "\n")
    print(head + "\n".join(lines))


def main():
    if len(sys.argv) > 1 and sys.argv[1] == "--ingest-traffic":
        ingest_traffic(sys.argv[2], sys.argv[3], int(sys.argv[4]), " ".join(sys.argv[5:]))
        return
    if len(sys.argv) > 1 and sys.argv[1] == "--ingest-trace":
        ingest_trace(sys.argv[2], sys.argv[3], " ".join(sys.argv[4:]))
        return
    if len(sys.argv) > 1 and sys.argv[1] == "--ingest-counters":
        ingest_counters(sys.argv[2], sys.argv[3], sys.argv[4], sys.argv[5], " ".join(sys.argv[6:]))
        return
    if len(sys.argv) > 1 and sys.argv[1] == "--ingest-infer":
        ingest_infer(sys.argv[2], sys.argv[3], sys.argv[4], sys.argv[5], " ".join(sys.argv[6:]))
        return
    if len(sys.argv) > 1 and sys.argv[1] == "--ingest-vendor":
        ingest_vendor(sys.argv[2], sys.argv[3], " ".join(sys.argv[4:]))
        return
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-infer", action="store_true", help="skip the no-grad (inference) sweep")
    ap.add_argument("--infer-only", action="store_true",
                    help="only the no-grad sweep (and the stream-copy reference): one JSON line")
    ap.add_argument("--infer-trace", action="store_true",
                    help="only a short fixed sequence of no-grad calls, for rocprofv3 (see ingest_infer)")
    ap.add_argument("--no-fp32", action="store_true", help="skip the true-IEEE fp32 run")
    ap.add_argument("--no-tp", action="store_true", help="skip the tensor-parallel shard-shape sweep")
    ap.add_argument("--no-linear", action="store_true", help="skip the nn.Linear weight-layout leg")
    ap.add_argument("--no-clock", action="store_true", help="skip the 3 s graphics-clock window (profiled runs)")
    ap.add_argument("--vendor-gemm", action="store_true",
                    help="only hipBLASLt (torch.mm) at two of the step's GEMM shapes, for context: one JSON line")
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

    if args.infer_trace:
        order = infer_trace(mlp, torch, torch.device("cuda:0"))
        print(json.dumps({"infer_trace": order, "calls_per_shape": INFER_TRACE_CALLS}), flush=True)
        return
    if args.vendor_gemm:
        print(json.dumps({"vendor_gemm": vendor_gemm(torch, torch.device("cuda:0"))}), flush=True)
        return
    if args.infer_only:
        dev = torch.device("cuda:0")
        copy = stream_copy_gbps(torch, dev)
        print(json.dumps({"metric": "no-grad HBM GB/s (B=1, 256 MB cache flushed per call by a 1 GiB read)",
                          "unit": "GB/s", "peak_GBps": PEAK_HBM_GBS, "stream_copy_GBps": copy,
                          "by_shape": infer_sweep(mlp, torch, dev, copy_gbps=copy)}), flush=True)
        return

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

    # events between steps: the whole loop gives the mean, each step its own time
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    with mlp.StageTimer(capacity=max(args.steps, 1)) as st:
        torch.cuda.synchronize()
        ev[0].record()
        for i in range(args.steps):
            step()
            ev[i + 1].record()
        torch.cuda.synchronize()
    ms_step = ev[0].elapsed_time(ev[-1]) / args.steps
    per_step = sorted(ev[i].elapsed_time(ev[i + 1]) for i in range(args.steps))
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
        "sclk": None if args.no_clock else measure_clock(torch, step),
        "step_ms": {"mean": round(ms_step, 3), "median": round(per_step[len(per_step) // 2], 3),
                    "min": round(per_step[0], 3), "max": round(per_step[-1], 3)},
        "roofline": roofline,
        "stages": stages,
    }
    psample = None
    if not args.no_cpu_baseline:
        psample = gather_parity_sample(mlp, torch, g, T, H)
    del y, saved, dx, dwg, dwu, dwd
    if not args.no_linear:
        out["linear_layout"] = linear_layout_leg(mlp, torch, g, T, D, H)
    del g, X, Wg, Wu, Wd, dY
    if not args.no_fp32:
        out["fp32_ieee"] = fp32_leg(mlp, torch, dev)
    if not args.no_tp:
        out["tp_shards"] = tp_shard_sweep(mlp, torch, dev, T, D, H)
    if not args.no_infer:
        copy = stream_copy_gbps(torch, dev)
        out["infer"] = {"metric": "no-grad HBM GB/s (B=1, 256 MB cache flushed per call by a 1 GiB read)",
                        "peak_GBps": PEAK_HBM_GBS, "stream_copy_GBps": copy,
                        "by_shape": infer_sweep(mlp, torch, dev, copy_gbps=copy)}
    if not args.no_cpu_baseline:
        # the leg that runs the oracle on the host: its time on a bounded
        # sample, and the parity of the sampled GPU outputs
        out["cpu_baseline"] = cpu_baseline(inp, D, H, args.cpu_seconds)
        out["parity"] = parity_vs_oracle(inp, *psample)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
