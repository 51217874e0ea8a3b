"""Structural properties of the GPU results (GPU).

Euler-homogeneity identities (Y is linear in Wu and in Wd, G and U linear in
X): <dWd,Wd> = <dWu,Wu> = <dY,Y> and <dI,X> = <dWg,Wg> + <dWu,Wu>; finite,
nonzero gradients for every parameter and the input (the trainability gate
of "Scope one-round FP32 SwiGLU to the exact Qwen3.5 contract", xorl PR #51);
bitwise run-to-run determinism; inputs left unchanged; the autograd wrapper's
single-use rule ("[RFC] Full-pipeline SwiGLU MLP ...", section "Known
limitations and validation gaps").
"""

import numpy as np
import pytest
import torch

from synth import make_inputs
from tests._util import banner, f64, run_train, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def mlp():
    import backward_gate_up_amd as m

    return m


def test_homogeneity_identities_and_trainability(mlp):
    inp = make_inputs(2048, 512, 1024, seed=11, dtype="bf16")
    out = run_train(mlp, to_dev(inp))
    ip = lambda a, b: float(np.sum(f64(a) * f64(b)))
    yy = ip(inp["dY"], out["Y"])
    wd = ip(out["dWd"], inp["Wd"])
    wu = ip(out["dWu"], inp["Wu"])
    wg = ip(out["dWg"], inp["Wg"])
    xi = ip(out["dI"], inp["X"])
    banner(f"<dY,Y>={yy:.6g} <dWd,Wd>={wd:.6g} <dWu,Wu>={wu:.6g} <dI,X>={xi:.6g} sum={wg + wu:.6g}")
    assert wd == pytest.approx(yy, rel=1e-2)
    assert wu == pytest.approx(yy, rel=1e-2)
    assert xi == pytest.approx(wg + wu, rel=1e-2)
    for k in ("dI", "dWg", "dWu", "dWd"):
        t = out[k]
        assert torch.isfinite(t).all(), k
        assert (t != 0).float().mean().item() > 0.99, k


def test_determinism_and_inputs_unchanged(mlp):
    inp = make_inputs(1000, 256, 640, seed=3, dtype="bf16")
    g = to_dev(inp)
    before = {k: v.clone() for k, v in g.items()}
    o1 = run_train(mlp, g)
    o2 = run_train(mlp, g)
    for k in o1:
        assert torch.equal(o1[k], o2[k]), k
    for k in g:
        assert torch.equal(g[k], before[k]), k


def test_autograd_function_and_single_use(mlp):
    inp = make_inputs(96, 128, 256, seed=4, dtype="bf16")
    g = to_dev(inp)
    leaves = {k: g[k].clone().requires_grad_(True) for k in ("X", "Wg", "Wu", "Wd")}
    x3 = leaves["X"].view(4, 24, 128)
    y = mlp.swiglu_mlp(x3, leaves["Wg"], leaves["Wu"], leaves["Wd"])
    assert y.shape == (4, 24, 128)
    y.backward(g["dY"].view(4, 24, 128), retain_graph=True)
    ref = run_train(mlp, g)
    assert torch.equal(y.detach().view(96, 128), ref["Y"])
    assert torch.equal(leaves["X"].grad, ref["dI"])
    assert torch.equal(leaves["Wg"].grad, ref["dWg"])
    assert torch.equal(leaves["Wu"].grad, ref["dWu"])
    assert torch.equal(leaves["Wd"].grad, ref["dWd"])
    with pytest.raises(RuntimeError, match="backward called twice"):
        y.backward(g["dY"].view(4, 24, 128))
    y2 = mlp.swiglu_mlp(leaves["X"], leaves["Wg"], leaves["Wu"], leaves["Wd"])
    with pytest.raises(RuntimeError, match="create_graph"):
        torch.autograd.grad(y2.sum(), leaves["X"], create_graph=True)
    with torch.no_grad():
        y3 = mlp.swiglu_mlp(x3, leaves["Wg"], leaves["Wu"], leaves["Wd"])
    assert torch.equal(y3.view(96, 128), ref["Y"])


def test_device_errors_raise(mlp):
    from backward_gate_up_amd import SwiGLUError

    inp = to_dev(make_inputs(16, 64, 128, seed=1, dtype="bf16"))
    y = torch.empty((16, 64), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(SwiGLUError, match="ALIAS"):
        mlp.fwd(inp["X"], inp["Wg"], inp["Wu"], inp["Wd"], y=inp["X"])
    with pytest.raises(SwiGLUError, match="SHAPE"):
        mlp.fwd(inp["X"][:, :60].contiguous(), inp["Wg"][:60].contiguous(),
                inp["Wu"][:60].contiguous(), inp["Wd"][:, :60].contiguous())
    with pytest.raises(SwiGLUError, match="ALIGN"):
        buf = torch.empty(16 * 64 + 1, dtype=torch.bfloat16, device="cuda")
        mlp.fwd(inp["X"], inp["Wg"], inp["Wu"], inp["Wd"], y=buf[1:].view(16, 64))


@pytest.mark.parametrize("T", [8, 100, 300, 600])
def test_nan_and_inf_propagate(mlp, T):
    """A non-finite input value reaches exactly the outputs that depend on it,
    with no trap, on every kernel family (few-token, split-K no-grad, 64-row
    tiles, ring). NaN in one row of X poisons that row of Y and dI and every
    weight gradient; the other rows stay finite. +Inf in one gate value
    (through Wg) takes the fast and the IEEE logistic paths."""
    D, H, bad = 256, 384, 3
    inp = make_inputs(T, D, H, seed=T + 5, dtype="bf16")
    g = to_dev(inp)
    g["X"][bad, 7] = float("nan")
    out = run_train(mlp, g)
    rows = torch.arange(T, device="cuda") != bad
    for k in ("Y", "dI"):
        assert torch.isnan(out[k][bad]).all(), k
        assert torch.isfinite(out[k][rows]).all(), k
    for k in ("dWg", "dWu", "dWd"):
        assert torch.isnan(out[k]).any(), k
    y_ng = mlp.infer(g["X"], g["Wg"], g["Wu"], g["Wd"])
    torch.cuda.synchronize()
    assert torch.isnan(y_ng[bad]).all() and torch.isfinite(y_ng[rows]).all()
    # +-Inf gate pre-activations: one column of Wg set to +Inf reaches every
    # row's g in that hidden unit; SiLU(+Inf) = +Inf, SiLU(-Inf) = -Inf * 0
    g = to_dev(inp)
    g["Wg"][:, 5] = float("inf")
    y, saved = mlp.fwd(g["X"], g["Wg"], g["Wu"], g["Wd"])
    torch.cuda.synchronize()
    G, A = saved[1][:, 5].float(), saved[0][:, 5].float()
    assert torch.isinf(G).all() or torch.isnan(G).any()
    assert not torch.isfinite(A).all()
    other = torch.ones(H, dtype=torch.bool, device="cuda")
    other[5] = False
    assert torch.isfinite(saved[0][:, other]).all()
