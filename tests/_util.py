"""Shared helpers for the GPU tests (no arithmetic of the method here)."""

import numpy as np
import torch

TOL = {"bf16": 1e-2, "fp16": 1e-2, "fp32": 1e-5}
FMT = {torch.bfloat16: "bf16", torch.float16: "fp16", torch.float32: "fp32"}


def f64(t):
    """Exact float64 copy of a (CPU or GPU) tensor."""
    return t.detach().float().cpu().numpy().astype(np.float64)


def nl2(got, ref):
    """Normalized L2 error ||got - ref|| / ||ref|| in float64."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    den = np.linalg.norm(ref)
    return float(np.linalg.norm(got - ref) / (den if den > 0 else 1.0))


def banner(msg):
    print(f"[gpu-test] {msg}", flush=True)


def to_dev(inp, dev="cuda:0"):
    return {k: v.to(dev) for k, v in inp.items()}


def run_train(mlp, g):
    """fwd + bwd through the C ABI; returns every output plus the saved planes
    as they were after fwd (A, G, U) and after bwd (A, dG, dU)."""
    y, saved = mlp.fwd(g["X"], g["Wg"], g["Wu"], g["Wd"])
    after_fwd = saved.clone()
    dx, dwg, dwu, dwd = mlp.bwd(g["dY"], g["X"], g["Wg"], g["Wu"], g["Wd"], saved)
    torch.cuda.synchronize()
    return {"Y": y, "dI": dx, "dWg": dwg, "dWu": dwu, "dWd": dwd,
            "A": after_fwd[0], "G": after_fwd[1], "U": after_fwd[2],
            "A_after": saved[0], "dG": saved[1], "dU": saved[2]}
