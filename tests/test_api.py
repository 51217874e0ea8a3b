"""Host-side checks of the Python API levels (CPU; no kernel runs here).

The op wrappers, the autograd Function and the nn.Module must refuse host
tensors and mismatched caller buffers before anything reaches the C ABI: a
host pointer handed to the kernels would be read as a device address.
"""

import pytest
import torch

import backward_gate_up_amd as m


def _w(D=64, H=128, dtype=torch.bfloat16):
    g = torch.Generator().manual_seed(0)
    return (torch.randn(D, H, generator=g).to(dtype), torch.randn(D, H, generator=g).to(dtype),
            torch.randn(H, D, generator=g).to(dtype))


def test_host_tensors_rejected_by_every_entry():
    wg, wu, wd = _w()
    x = torch.randn(5, 64).to(torch.bfloat16)
    for call in (lambda: m.fwd(x, wg, wu, wd), lambda: m.infer(x, wg, wu, wd),
                 lambda: m.bwd(x, x, wg, wu, wd, torch.empty(3, 5, 128, dtype=torch.bfloat16)),
                 lambda: m.swiglu_mlp(x.view(1, 5, 64), wg, wu, wd)):
        with pytest.raises(ValueError, match="GPU"):
            call()


def test_shape_and_dtype_mismatch_rejected():
    wg, wu, wd = _w()
    x = torch.randn(5, 64).to(torch.bfloat16)
    with pytest.raises(ValueError, match="shape mismatch"):
        m.fwd(x, wg, wu[:, :64], wd)
    with pytest.raises(ValueError, match="share dtype"):
        m.fwd(x, wg.float(), wu, wd)
    with pytest.raises(TypeError):
        m._dt(torch.zeros(1, dtype=torch.float64))


def test_caller_buffers_checked():
    like = torch.empty(4, 8, dtype=torch.bfloat16)
    assert m._buf(None, (4, 8), like, "y").shape == (4, 8)
    with pytest.raises(ValueError, match="bfloat16"):
        m._buf(torch.empty(4, 8), (4, 8), like, "y")
    with pytest.raises(ValueError, match="shape"):
        m._buf(torch.empty(8, 4, dtype=torch.bfloat16), (4, 8), like, "y")
    with pytest.raises(ValueError, match="contiguous"):
        m._buf(torch.empty(8, 4, dtype=torch.bfloat16).t(), (4, 8), like, "y")


def test_module_layout_and_from_linears():
    mod = m.SwiGLUMLPPacked(64, 128, dtype=torch.bfloat16, generator=torch.Generator().manual_seed(1))
    assert (mod.hidden_size, mod.intermediate_size) == (64, 128)
    assert mod.w_gate.shape == (64, 128) and mod.w_up.shape == (64, 128) and mod.w_down.shape == (128, 64)
    assert len(list(mod.parameters())) == 3
    lin = [torch.nn.Linear(64, 128, bias=False), torch.nn.Linear(64, 128, bias=False),
           torch.nn.Linear(128, 64, bias=False)]
    m2 = m.SwiGLUMLPPacked.from_linears(*lin)
    # x @ W.T for nn.Linear equals x @ w in the kernels' layout
    assert torch.equal(m2.w_gate, lin[0].weight.t())
    assert torch.equal(m2.w_up, lin[1].weight.t())
    assert torch.equal(m2.w_down, lin[2].weight.t())
    assert m2.w_gate.is_contiguous() and m2.w_down.is_contiguous()
    with pytest.raises(ValueError, match="bias"):
        m.SwiGLUMLPPacked.from_linears(torch.nn.Linear(64, 128), *lin[1:])
    with pytest.raises(ValueError, match="GPU"):
        mod(torch.randn(2, 3, 64).to(torch.bfloat16))


def test_hf_interchangeable_module_matches_llama_mlp_surface():
    """SwiGLUMLP(config) has LlamaMLP's constructor, attributes, submodules
    and state-dict keys and shapes (nn.Linear layout), so a LlamaMLP state
    dict loads unchanged, strictly; bias and non-SiLU activations are
    refused."""
    from transformers import LlamaConfig
    from transformers.models.llama.modeling_llama import LlamaMLP

    cfg = LlamaConfig(hidden_size=64, intermediate_size=160)
    ref = LlamaMLP(cfg)
    mod = m.SwiGLUMLP(cfg)
    assert (mod.hidden_size, mod.intermediate_size) == (64, 160) and mod.config is cfg
    sd = ref.state_dict()
    assert {k: tuple(v.shape) for k, v in mod.state_dict().items()} == {k: tuple(v.shape) for k, v in sd.items()}
    mod.load_state_dict(sd, strict=True)
    for name in ("gate_proj", "up_proj", "down_proj"):
        assert torch.equal(getattr(mod, name).weight, getattr(ref, name).weight)
        assert getattr(mod, name).bias is None
    import inspect
    assert list(inspect.signature(mod.forward).parameters) == list(inspect.signature(ref.forward).parameters)
    with pytest.raises(ValueError, match="bias"):
        m.SwiGLUMLP(LlamaConfig(hidden_size=64, intermediate_size=160, mlp_bias=True))
    with pytest.raises(ValueError, match="hidden_act"):
        m.SwiGLUMLP(LlamaConfig(hidden_size=64, intermediate_size=160, hidden_act="gelu"))
    with pytest.raises(ValueError, match="GPU"):
        mod.to(torch.bfloat16)(torch.randn(2, 3, 64).to(torch.bfloat16))


def test_linear_layout_shape_checks():
    x = torch.empty(4, 64, dtype=torch.bfloat16)
    wk = (torch.empty(64, 96, dtype=torch.bfloat16), torch.empty(64, 96, dtype=torch.bfloat16),
          torch.empty(96, 64, dtype=torch.bfloat16))
    wl = tuple(w.t().contiguous() for w in wk)
    with pytest.raises(ValueError, match="GPU"):
        m._shapes(x, *wk)
    with pytest.raises(ValueError, match="GPU"):
        m._shapes(x, *wl, linear=True)
    with pytest.raises(ValueError, match="shape mismatch"):
        m._shapes(x, *wk, linear=True)
    with pytest.raises(ValueError, match="shape mismatch"):
        m._shapes(x, *wl)
