"""The autograd Function and nn.Module levels against the fp64 oracle (GPU).

A [B, S, D] input goes through ``SwiGLUMLPPacked`` with autograd; the upstream
gradient dY enters through loss = <Y, dY>, so the gradients autograd returns
are the oracle's bwd(dY, ...) at the normalized-L2 bound of 1e-2 (bf16). The
same module under torch.no_grad() takes the no-grad path and returns the
training Y bit for bit. The autograd Function is single use ("[RFC]
Full-pipeline SwiGLU MLP with forward/backward co-optimization", "Known
limitations and validation gaps"): a second backward and double backward are
refused.
"""

import pytest
import torch

import oracle as O
from synth import make_inputs
from tests._util import TOL, assert_local, banner, f64, fmt_local

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def mlp():
    import backward_gate_up_amd as m

    return m


@pytest.mark.parametrize("B,S,D,H,dt", [(2, 150, 256, 384, torch.bfloat16), (4, 700, 512, 1376, torch.bfloat16),
                                        (1, 333, 136, 264, torch.float16)])
def test_module_grads_vs_oracle(mlp, B, S, D, H, dt):
    fmt = {torch.bfloat16: "bf16", torch.float16: "fp16"}[dt]
    banner(f"module B={B} S={S} D={D} H={H} {fmt}")
    inp = make_inputs(B * S, D, H, seed=B * 1000 + S, dtype=fmt)
    mod = mlp.SwiGLUMLPPacked(D, H, dtype=dt, device="cuda")
    with torch.no_grad():
        mod.w_gate.copy_(inp["Wg"])
        mod.w_up.copy_(inp["Wu"])
        mod.w_down.copy_(inp["Wd"])
    x = inp["X"].view(B, S, D).cuda().requires_grad_(True)
    dy = inp["dY"].view(B, S, D).cuda()
    y = mod(x)
    assert y.shape == (B, S, D) and y.dtype == dt
    (y.float() * dy.float()).sum().backward()
    f = {k: v.float().numpy() for k, v in inp.items()}
    ref = O.bwd(f["dY"], f["X"], f["Wg"], f["Wu"], f["Wd"])
    ref["Y"] = O.fwd(f["X"], f["Wg"], f["Wu"], f["Wd"])["Y"]
    got = {"Y": y.reshape(B * S, D), "dI": x.grad.reshape(B * S, D), "dWg": mod.w_gate.grad,
           "dWu": mod.w_up.grad, "dWd": mod.w_down.grad}
    for k, v in got.items():
        banner(f"{k} {fmt_local(assert_local(f64(v), ref[k], TOL[fmt], ('module', k)))}")
    with torch.no_grad():
        y_ng = mod(x)
    torch.cuda.synchronize()
    assert torch.equal(y_ng, y.detach())


def test_function_single_use(mlp):
    inp = make_inputs(64, 128, 256, seed=3, dtype="bf16")
    x = inp["X"].cuda().requires_grad_(True)
    w = [inp[k].cuda().requires_grad_(True) for k in ("Wg", "Wu", "Wd")]
    y = mlp.swiglu_mlp(x, *w)
    y.sum().backward(retain_graph=True)
    with pytest.raises(RuntimeError, match="twice"):
        y.sum().backward()
    y2 = mlp.swiglu_mlp(x, *w)
    with pytest.raises(RuntimeError, match="create_graph"):
        torch.autograd.grad(y2.sum(), x, create_graph=True)


@pytest.mark.parametrize("B,S,D,H", [(2, 300, 256, 688), (1, 48, 128, 344)])
def test_hf_llama_mlp_state_dict_drop_in(mlp, B, S, D, H):
    """transformers' LlamaMLP built from a small local LlamaConfig (no
    download): its state dict loads unchanged into SwiGLUMLP(config), and Y
    and every gradient (x, gate_proj, up_proj, down_proj weights, in
    nn.Linear layout) match the oracle; LlamaMLP's own eager forward in fp32
    on the CPU agrees too. The upstream gradient enters as loss = <Y, dY>."""
    from transformers import LlamaConfig
    from transformers.models.llama.modeling_llama import LlamaMLP

    banner(f"LlamaMLP drop-in B={B} S={S} D={D} H={H}")
    cfg = LlamaConfig(hidden_size=D, intermediate_size=H)
    inp = make_inputs(B * S, D, H, seed=D + H + S, dtype="bf16")
    ref_mod = LlamaMLP(cfg)
    with torch.no_grad():
        ref_mod.gate_proj.weight.copy_(inp["Wg"].t().float())
        ref_mod.up_proj.weight.copy_(inp["Wu"].t().float())
        ref_mod.down_proj.weight.copy_(inp["Wd"].t().float())
    sd = {k: v.to(torch.bfloat16) for k, v in ref_mod.state_dict().items()}
    mod = mlp.SwiGLUMLP(cfg).to(device="cuda", dtype=torch.bfloat16)
    mod.load_state_dict(sd, strict=True)
    x = inp["X"].view(B, S, D).cuda().requires_grad_(True)
    dy = inp["dY"].view(B, S, D).cuda()
    y = mod(x)
    assert y.shape == (B, S, D) and y.dtype == torch.bfloat16
    (y.float() * dy.float()).sum().backward()
    f = {k: v.float().numpy() for k, v in inp.items()}
    ref = O.bwd(f["dY"], f["X"], f["Wg"], f["Wu"], f["Wd"])
    ref["Y"] = O.fwd(f["X"], f["Wg"], f["Wu"], f["Wd"])["Y"]
    got = {"Y": y.reshape(B * S, D), "dI": x.grad.reshape(B * S, D), "dWg": mod.gate_proj.weight.grad.t(),
           "dWu": mod.up_proj.weight.grad.t(), "dWd": mod.down_proj.weight.grad.t()}
    for k, v in got.items():
        banner(f"  {k} {fmt_local(assert_local(f64(v), ref[k], TOL['bf16'], ('llama drop-in', k)))}")
    with torch.no_grad():
        y_hf = ref_mod(inp["X"].float().view(B, S, D)).reshape(B * S, D).double().numpy()
    assert_local(y_hf, ref["Y"], 1e-5, "LlamaMLP fp32 forward vs oracle")
    with torch.no_grad():
        y_ng = mod(x)
    torch.cuda.synchronize()
    assert torch.equal(y_ng, y.detach())
