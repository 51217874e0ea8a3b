"""Parity of the nn.Linear weight layout (GPU).

With SWIGLU_FLAG_LINEAR_WEIGHTS the kernels read gate_proj and up_proj
weights [H, D] and down_proj [D, H] as given (the forward GEMMs then take
K-major weights, dA and dI N-major ones) and write the weight gradients in
the same layout. The oracle computes in its own notation (Wg, Wu [D, H],
Wd [H, D]); the test hands it the transposes and transposes its weight
gradients back, which is bookkeeping, not arithmetic. Same bounds as the
kernel layout: whole-tensor, per-row, per-32x32-block and per-256x256-tile
normalized L2 <= 1e-2 (bf16, fp16), <= 1e-5 (fp32). Shapes cover every
dispatch regime: the 64-row tile engine (T <= 512, also the few-token
shapes, which the weight-streaming kernels do not take in this layout),
the ring engine (T > 512) with ragged edges, and weight-gradient tiles
split over K.
"""

import numpy as np
import pytest
import torch

import oracle as O
from synth import make_inputs, workload_inputs
from tests._util import TOL, assert_local, banner, f64, fmt_local, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def mlp():
    import backward_gate_up_amd as m

    return m


def _lin(g):
    """The same weights in the nn.Linear layout (contiguous copies made by
    the test, outside the library)."""
    return {"X": g["X"], "dY": g.get("dY"), "Wg": g["Wg"].t().contiguous(), "Wu": g["Wu"].t().contiguous(),
            "Wd": g["Wd"].t().contiguous()}


def _check(mlp, inp, fmt, label, planes=True):
    g = _lin(to_dev(inp))
    y, saved = mlp.fwd(g["X"], g["Wg"], g["Wu"], g["Wd"], linear=True)
    after_fwd = saved.clone() if planes else None
    dx, dwg, dwu, dwd = mlp.bwd(g["dY"], g["X"], g["Wg"], g["Wu"], g["Wd"], saved, linear=True)
    torch.cuda.synchronize()
    assert dwg.shape == g["Wg"].shape and dwd.shape == g["Wd"].shape
    f = {k: v.float().numpy() for k, v in inp.items()}
    ref = O.bwd(f["dY"], f["X"], f["Wg"], f["Wu"], f["Wd"], keep=planes)
    if not planes:
        ref["Y"] = O.fwd(f["X"], f["Wg"], f["Wu"], f["Wd"])["Y"]
    got = {"Y": y, "dI": dx, "dWg": dwg.t(), "dWu": dwu.t(), "dWd": dwd.t()}
    if planes:
        got.update(G=after_fwd[1], U=after_fwd[2], dG=saved[1], dU=saved[2])
    for k, v in got.items():
        banner(f"{label} {k}: {fmt_local(assert_local(f64(v), ref[k], TOL[fmt], (label, k)))}")
    if planes and fmt != "fp32":
        a_ref = O.round_to(O.epilogue_fwd(f64(after_fwd[1]), f64(after_fwd[2])), fmt)
        assert int(O.ulp_distance(f64(after_fwd[0]), a_ref, fmt).max()) <= 1
    return g, y


@pytest.mark.parametrize("T,D,H", [(1, 64, 64), (40, 264, 520), (64, 200, 136), (129, 512, 264),
                                   (300, 1024, 2816), (513, 256, 512), (1000, 384, 648), (777, 136, 200)])
def test_linear_layout_ragged_bf16(mlp, T, D, H):
    _check(mlp, make_inputs(T, D, H, seed=11 * T + D, dtype="bf16"), "bf16", f"linear T={T} D={D} H={H}")


@pytest.mark.parametrize("fmt", ["fp16", "fp32"])
def test_linear_layout_fp16_fp32(mlp, fmt):
    for T, D, H in ((37, 136, 264), (700, 264, 392)):
        _check(mlp, make_inputs(T, D, H, seed=T + 5, dtype=fmt), fmt, f"linear {fmt} T={T} D={D} H={H}")


def test_linear_layout_T16384(mlp):
    _check(mlp, workload_inputs("mlp_1024x2816_T16384"), "bf16", "linear 1024x2816 T=16384")


def test_linear_layout_split_remainder_ragged(mlp):
    """T=8192, D=1032, H=6664: dWd [D, H] has 5 x 27 = 135 tiles (all split
    over K), [dWg | dWu] [H, D] x 2 has 270 (one round of 256, 14 split)."""
    _check(mlp, make_inputs(8192, 1032, 6664, seed=8193, dtype="bf16"), "bf16",
           "linear split remainder T=8192 D=1032 H=6664", planes=False)


@pytest.mark.parametrize("S", [1, 16, 128, 256, 600])
def test_linear_layout_no_grad(mlp, S):
    D, H = 1024, 2816
    inp = make_inputs(S, D, H, seed=300 + S, dtype="bf16", with_dy=False)
    g = _lin(to_dev(inp))
    y = mlp.infer(g["X"], g["Wg"], g["Wu"], g["Wd"], linear=True)
    y_train, _ = mlp.fwd(g["X"], g["Wg"], g["Wu"], g["Wd"], linear=True)
    y_na = mlp.infer_noalloc(g["X"], g["Wg"], g["Wu"], g["Wd"], linear=True)
    torch.cuda.synchronize()
    f = {k: v.float().numpy() for k, v in inp.items()}
    e = assert_local(f64(y), O.infer(f["X"], f["Wg"], f["Wu"], f["Wd"]), 1e-2, ("linear infer", S))
    banner(f"linear infer S={S}: {fmt_local(e)}")
    # the same kernels as the training forward in this layout, and the
    # allocation-free entry point runs the same plan
    assert torch.equal(y, y_train) and torch.equal(y_na, y)
