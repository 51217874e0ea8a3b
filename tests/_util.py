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


# ---------------------------------------------------------------------------
# Element-local parity. A whole-tensor normalized L2 can hide a localized
# fault: one zeroed row or one wrong 32 x 32 block of a [16384, 1024] output
# adds less than the 1e-2 bound. So every output is also checked region by
# region: each row, each 32 x 32 block (the matrix-core block of the
# kernels), and each 256 x 256 output tile.
#
# Local error of a region R: rms(got_R - ref_R) / max(rms(ref_R), rms(ref)).
# Where the region's own scale is at least the tensor's, this is the region's
# normalized L2; a region of small values is measured against the tensor's
# scale instead, so a handful of near-cancelling elements cannot blow it up.
# ---------------------------------------------------------------------------

def _block_ss(a, bm, bn):
    """Sums of squares over bm x bn blocks of a 2-D array (zero padded) and
    the number of real elements in each block."""
    M, N = a.shape
    pm, pn = -M % bm, -N % bn
    sq = np.pad(a * a, ((0, pm), (0, pn)))
    ss = sq.reshape((M + pm) // bm, bm, (N + pn) // bn, bn).sum(axis=(1, 3))
    cnt = np.pad(np.ones((M, N)), ((0, pm), (0, pn))).reshape(ss.shape[0], bm, ss.shape[1], bn).sum(axis=(1, 3))
    return ss, cnt


def local_errors(got, ref, block=(32, 32), tile=(256, 256)):
    """Worst local errors of a 2-D result: per row, per block and per tile
    region (shapes in rows x columns), plus the whole-tensor normalized L2.
    Returns a dict with the maxima and where each occurs (row index, block
    and tile coordinates). For a sample of rows of a larger result, pass
    block=(1, 32), tile=(1, 256): the footprints of a 32 x 32 matrix-core
    block and of a 256 x 256 tile on each sampled row."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    if ref.ndim == 1:
        got, ref = got[None, :], ref[None, :]
    assert got.shape == ref.shape, (got.shape, ref.shape)
    out = {"whole": nl2(got, ref)}
    if ref.size == 0:
        out.update(row=0.0, block=0.0, tile=0.0, row_at=None, block_at=None, tile_at=None)
        return out
    diff = got - ref
    rms_all = float(np.sqrt(np.mean(ref * ref)))
    floor = rms_all if rms_all > 0 else 1.0
    for key, (bm, bn) in (("row", (1, ref.shape[1])), ("block", block), ("tile", tile)):
        ss_d, cnt = _block_ss(diff, bm, bn)
        ss_r, _ = _block_ss(ref, bm, bn)
        with np.errstate(invalid="ignore", divide="ignore"):
            e = np.sqrt(ss_d / cnt) / np.maximum(np.sqrt(ss_r / cnt), floor)
        e = np.where(np.isfinite(e), e, np.inf)  # NaN / Inf in got: never passes
        at = np.unravel_index(int(np.argmax(e)), e.shape)
        out[key] = float(e[at])
        out[key + "_at"] = int(at[0]) if key == "row" else (int(at[0]), int(at[1]))
    return out


SAMPLED = {"block": (1, 32), "tile": (1, 256)}


def local_ok(errs, tol):
    return all(errs[k] <= tol for k in ("whole", "row", "block", "tile"))


def assert_local(got, ref, tol, label, **kw):
    """Whole-tensor, per-row, per-32x32-block and per-256x256-tile errors all
    within tol; the message names the worst region."""
    e = local_errors(got, ref, **kw)
    assert local_ok(e, tol), (label, {k: v for k, v in e.items()})
    return e


def fmt_local(e):
    return f"whole={e['whole']:.2e} row={e['row']:.2e} blk={e['block']:.2e} tile={e['tile']:.2e}"
