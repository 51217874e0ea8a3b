"""The fused epilogues to within 1 ulp (GPU).

With X = I (T = D) every gate/up GEMM output is a single product, so
G = Wg and U = Wu exactly; with Wd = I (H = D) the down projection is exact
(Y = A) and dA = dY exactly. Then the forward epilogue (A) and the in-place
backward epilogue (dG, dU) can be compared element by element with the
correctly rounded fp64 values of the oracle's epilogue definitions.
"""

import numpy as np
import pytest
import torch

import oracle as O
from synth import make_inputs
from tests._util import banner, f64, run_train, to_dev

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("fmt,dt", [("bf16", torch.bfloat16), ("fp16", torch.float16)])
@pytest.mark.parametrize("n", [64, 264])
def test_one_hot_input_and_identity_down(fmt, dt, n):
    import backward_gate_up_amd as mlp

    inp = make_inputs(n, n, n, seed=n, dtype=fmt)
    inp["X"] = torch.eye(n, dtype=dt)
    inp["Wd"] = torch.eye(n, dtype=dt)
    # unit-scale gate/up values exercise the whole SiLU curve
    inp["Wg"] = (inp["Wg"].float() * n ** 0.5).to(dt)
    inp["Wu"] = (inp["Wu"].float() * n ** 0.5).to(dt)
    out = run_train(mlp, to_dev(inp))
    assert torch.equal(out["G"].cpu(), inp["Wg"])
    assert torch.equal(out["U"].cpu(), inp["Wu"])
    assert torch.equal(out["Y"], out["A"])
    g, u, dy = f64(inp["Wg"]), f64(inp["Wu"]), f64(inp["dY"])
    a_ref = O.round_to(O.epilogue_fwd(g, u), fmt)
    dg_ref, du_ref = O.epilogue_bwd(dy, g, u)
    ua = O.ulp_distance(f64(out["A"]), a_ref, fmt)
    ug = O.ulp_distance(f64(out["dG"]), O.round_to(dg_ref, fmt), fmt)
    uu = O.ulp_distance(f64(out["dU"]), O.round_to(du_ref, fmt), fmt)
    banner(f"epilogue {fmt} n={n}: max ulp A={ua.max()} dG={ug.max()} dU={uu.max()}; "
           f"exact A {np.mean(ua == 0):.4f} dG {np.mean(ug == 0):.4f} dU {np.mean(uu == 0):.4f}")
    assert ua.max() <= 1 and ug.max() <= 1 and uu.max() <= 1
    # nearly all are correctly rounded; 1-ulp cases are near-ties
    assert np.mean(ua == 0) > 0.99 and np.mean(ug == 0) > 0.98 and np.mean(uu == 0) > 0.99


@pytest.mark.parametrize("fmt,dt", [("bf16", torch.bfloat16), ("fp16", torch.float16)])
def test_epilogues_at_very_negative_gates(fmt, dt):
    """Gate values down to -130, where sigma(g) = e^g falls through the fp32
    denormal range: for bf16 the products SiLU(g) u, dA SiLU(g) and
    dA u SiLU'(g) are still normal bf16 numbers near g = -90, and they must be
    correctly rounded (within 1 ulp) there too, as for ordinary gates. Same
    exact-GEMM set-up as above (X = I, Wd = I)."""
    import backward_gate_up_amd as mlp

    n = 264
    inp = make_inputs(n, n, n, seed=11 + n, dtype=fmt)
    inp["X"] = torch.eye(n, dtype=dt)
    inp["Wd"] = torch.eye(n, dtype=dt)
    gen = torch.Generator().manual_seed(3)
    vals = torch.linspace(-130.0, 12.0, n * n)[torch.randperm(n * n, generator=gen)]
    inp["Wg"] = vals.view(n, n).to(dt)
    inp["Wu"] = (inp["Wu"].float() * n ** 0.5).to(dt)
    out = run_train(mlp, to_dev(inp))
    assert torch.equal(out["G"].cpu(), inp["Wg"])
    g, u, dy = f64(inp["Wg"]), f64(inp["Wu"]), f64(inp["dY"])
    a_ref = O.round_to(O.epilogue_fwd(g, u), fmt)
    dg_ref, du_ref = O.epilogue_bwd(dy, g, u)
    ua = O.ulp_distance(f64(out["A"]), a_ref, fmt)
    ug = O.ulp_distance(f64(out["dG"]), O.round_to(dg_ref, fmt), fmt)
    uu = O.ulp_distance(f64(out["dU"]), O.round_to(du_ref, fmt), fmt)
    deep = g < -88.0
    banner(f"very negative gates {fmt}: max ulp A={ua.max()} dG={ug.max()} dU={uu.max()}; "
           f"nonzero A among g < -88: {int((a_ref[deep] != 0).sum())}")
    assert ua.max() <= 1 and ug.max() <= 1 and uu.max() <= 1
    if fmt == "bf16":
        # the range is really exercised: tiny but nonzero bf16 results
        assert (a_ref[deep] != 0).sum() > 100
