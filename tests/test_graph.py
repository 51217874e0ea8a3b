"""The C ABI under HIP-graph capture (GPU).

The no-grad call and a full training step (forward + backward) are captured
once through torch.cuda.graph on the current stream. Each graph is then
replayed several times, with unrelated eager work and synchronizations in
between. Every replay must reproduce the eager outputs bit for bit (the
path is deterministic: a fixed tile and split order, and the one atomic
counter per unit only elects which workgroup adds the partials, in a fixed
order; it records no memset nodes), and the replayed outputs are checked
against the fp64 oracle as well, at the parity bounds (whole tensor, per
row, per 32 x 32 block, per 256 x 256 tile). The pages name small-shape host overhead as the no-grad path's only
loss ("[RFC] Full-pipeline SwiGLU MLP with forward/backward co-optimization",
"Inference results"), and replaying a graph is how a caller removes it.
"""

import pytest
import torch

import oracle as O
from synth import make_inputs
from tests._util import assert_local, banner, f64, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def mlp():
    import backward_gate_up_amd as m

    return m


def _noise():
    # unrelated eager work between replays (allocations, kernels, a reduction)
    a = torch.randn(1 << 20, device="cuda")
    return float(a.square().sum())


@pytest.mark.parametrize("D,H", [(1024, 2816), (256, 384)])
@pytest.mark.parametrize("S", [1, 16, 64, 200])
def test_infer_graph_replay(mlp, S, D, H):
    banner(f"graph infer S={S} D={D} H={H}")
    g = to_dev(make_inputs(S, D, H, seed=31 + S, dtype="bf16", with_dy=False))
    y = torch.empty((S, D), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(mlp.infer_workspace_bytes(S, D, H), dtype=torch.uint8, device="cuda")
    mlp.infer(g["X"], g["Wg"], g["Wu"], g["Wd"], y=y, workspace=ws)
    torch.cuda.synchronize()
    ref = y.clone()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        mlp.infer(g["X"], g["Wg"], g["Wu"], g["Wd"], y=y, workspace=ws)
    for r in range(4):
        y.fill_(float("nan"))
        _noise()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, ref), f"replay {r}"
    f = {k: v.float().cpu().numpy() for k, v in g.items()}
    assert_local(f64(y), O.infer(f["X"], f["Wg"], f["Wu"], f["Wd"]), 1e-2, ("graph infer", S, D, H))
    # new inputs written into the captured buffers flow through the graph
    x2 = make_inputs(S, D, H, seed=99, dtype="bf16", with_dy=False)["X"]
    g["X"].copy_(x2.cuda())
    graph.replay()
    mlp_eager = mlp.infer(g["X"], g["Wg"], g["Wu"], g["Wd"])
    torch.cuda.synchronize()
    assert torch.equal(y, mlp_eager)
    assert_local(f64(y), O.infer(x2.float().numpy(), f["Wg"], f["Wu"], f["Wd"]), 1e-2, ("graph infer new X", S))


@pytest.mark.parametrize("T,D,H", [(300, 256, 384), (1024, 512, 1024)])
def test_train_step_graph_replay(mlp, T, D, H):
    banner(f"graph train T={T} D={D} H={H}")
    g = to_dev(make_inputs(T, D, H, seed=7 + T, dtype="bf16"))
    bf = torch.bfloat16
    y = torch.empty((T, D), dtype=bf, device="cuda")
    saved = torch.empty((3, T, H), dtype=bf, device="cuda")
    dx = torch.empty((T, D), dtype=bf, device="cuda")
    dwg = torch.empty((D, H), dtype=bf, device="cuda")
    dwu = torch.empty((D, H), dtype=bf, device="cuda")
    dwd = torch.empty((H, D), dtype=bf, device="cuda")
    outs = (y, dx, dwg, dwu, dwd)

    def step():
        mlp.fwd(g["X"], g["Wg"], g["Wu"], g["Wd"], y=y, saved=saved)
        mlp.bwd(g["dY"], g["X"], g["Wg"], g["Wu"], g["Wd"], saved, dx=dx, dwg=dwg, dwu=dwu, dwd=dwd)

    step()
    torch.cuda.synchronize()
    ref = [t.clone() for t in outs]
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    for r in range(3):
        for t in outs:
            t.fill_(float("nan"))
        _noise()
        graph.replay()
        torch.cuda.synchronize()
        for name, got, want in zip(("Y", "dI", "dWg", "dWu", "dWd"), outs, ref):
            assert torch.equal(got, want), f"replay {r}: {name}"
    f = {k: v.float().cpu().numpy() for k, v in g.items()}
    oref = O.bwd(f["dY"], f["X"], f["Wg"], f["Wu"], f["Wd"])
    oref["Y"] = O.fwd(f["X"], f["Wg"], f["Wu"], f["Wd"])["Y"]
    for name, got in zip(("Y", "dI", "dWg", "dWu", "dWd"), outs):
        assert_local(f64(got), oref[name], 1e-2, ("graph train", name))
