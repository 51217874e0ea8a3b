"""Fused SwiGLU MLP for MI355X (gfx950): Python binding of libswiglu_mlp.so.

This module only marshals arguments: every arithmetic step runs in the HIP
kernels behind the C ABI declared in include/swiglu_mlp.h. PyTorch supplies
device memory and the current stream. There is no fallback: if the library
is missing or the device is not gfx950, calls raise.

Three levels, following the maintainers' layering on "[RFC] Full-pipeline
SwiGLU MLP with forward/backward co-optimization" (Liger-Kernel issue #1347,
discussion thread, "Three levels of APIs"): op-level wrappers (fwd / bwd /
infer, and the ``swiglu_mlp`` entry that flattens [..., D] inputs and picks
the no-grad path when autograd is off), an autograd Function composing them,
and nn.Modules: ``SwiGLUMLP(config)`` has the constructor and forward of the
transformers MLP modules (gate_proj, up_proj, down_proj nn.Linear layers, so
their state dicts load unchanged; the kernels read the nn.Linear weight
layout directly), and ``SwiGLUMLPPacked`` keeps [D, H] / [H, D] weights.

Weight layouts (``linear``): False (kernel layout): Wg, Wu [D, H], Wd [H, D];
True (nn.Linear layout): Wg, Wu [H, D], Wd [D, H]. Weight gradients come back
in the layout of their weights.
"""

import ctypes

import torch

from . import _lib as _L
from ._lib import SwiGLUError, STAGE_NAMES, NUM_STAGES  # noqa: F401

__all__ = ["fwd", "bwd", "infer", "infer_noalloc", "SwiGLUMLPFunction", "swiglu_mlp", "SwiGLUMLP",
           "SwiGLUMLPPacked", "saved_bytes",
           "infer_workspace_bytes", "bwd_workspace_bytes", "SwiGLUError", "StageTimer"]

_DT = {torch.bfloat16: _L.BF16, torch.float16: _L.FP16, torch.float32: _L.FP32}


def _dt(t):
    try:
        return _DT[t.dtype]
    except KeyError:
        raise TypeError(f"unsupported dtype {t.dtype}; use bfloat16, float16 or float32") from None


def _p(t):
    return None if t is None or t.numel() == 0 else t.data_ptr()


def _stream(device):
    return torch.cuda.current_stream(device).cuda_stream


def _check(rc, where):
    if rc != 0:
        raise SwiGLUError(rc, where)


def _shapes(x, wg, wu, wd, linear=False):
    if x.dim() != 2 or wg.dim() != 2 or wu.dim() != 2 or wd.dim() != 2:
        raise ValueError("expected X[T,D] and 2-D weights")
    T, D = x.shape
    H = wg.shape[0] if linear else wg.shape[1]
    want = ((H, D), (H, D), (D, H)) if linear else ((D, H), (D, H), (H, D))
    if tuple(wg.shape) != want[0] or tuple(wu.shape) != want[1] or tuple(wd.shape) != want[2]:
        lay = "Wg[H,D], Wu[H,D], Wd[D,H]" if linear else "Wg[D,H], Wu[D,H], Wd[H,D]"
        raise ValueError(f"shape mismatch (expected {lay}): X{tuple(x.shape)} Wg{tuple(wg.shape)} "
                         f"Wu{tuple(wu.shape)} Wd{tuple(wd.shape)}")
    for t in (wg, wu, wd):
        if t.dtype != x.dtype or t.device != x.device:
            raise ValueError("all tensors must share dtype and device")
    if x.device.type != "cuda":
        raise ValueError("tensors must be on a GPU (cuda/HIP device)")
    return T, D, H


def _buf(t, shape, like, name):
    """A caller-provided output or workspace: allocate it if None, else check
    that it is a contiguous tensor of the given shape on the inputs' device
    and dtype (a host tensor here would hand a host pointer to the kernels)."""
    if t is None:
        return torch.empty(shape, dtype=like.dtype, device=like.device)
    if t.device != like.device or t.dtype != like.dtype:
        raise ValueError(f"{name} must be a {like.dtype} tensor on {like.device}")
    if not t.is_contiguous() or tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must be a contiguous tensor of shape {tuple(shape)}")
    return t


def saved_bytes(T, H, dtype=torch.bfloat16):
    return _L.lib().swiglu_mlp_saved_bytes(T, H, _DT[dtype])


def infer_workspace_bytes(T, D, H, dtype=torch.bfloat16):
    return _L.lib().swiglu_mlp_infer_workspace_bytes(T, D, H, _DT[dtype])


def _flags(two_round=False, linear=False):
    return (_L.FLAG_TWO_ROUND if two_round else 0) | (_L.FLAG_LINEAR_WEIGHTS if linear else 0)


def fwd(x, wg, wu, wd, y=None, saved=None, two_round=False, linear=False):
    """Training forward. Returns (Y[T,D], saved) where ``saved`` is the
    [3, T, H] A|G|U buffer that ``bwd`` consumes. ``two_round`` selects the
    historical two-round SwiGLU program A = rnd(rnd(SiLU(g)) u) instead of
    the one-round A = rnd(SiLU(g) u); ``linear``: nn.Linear weight layout."""
    x, wg, wu, wd = (t.contiguous() for t in (x, wg, wu, wd))
    T, D, H = _shapes(x, wg, wu, wd, linear)
    y = _buf(y, (T, D), x, "y")
    saved = _buf(saved, (3, T, H), x, "saved")
    rc = _L.lib().swiglu_mlp_fwd_ex(_p(x), _p(wg), _p(wu), _p(wd), _p(y), _p(saved),
                                    T, D, H, _dt(x), _flags(two_round, linear), _stream(x.device))
    _check(rc, "swiglu_mlp_fwd_ex")
    return y, saved


def bwd_workspace_bytes(T, D, H, dtype=torch.bfloat16):
    return _L.lib().swiglu_mlp_bwd_workspace_bytes(T, D, H, _DT[dtype])


def bwd(dy, x, wg, wu, wd, saved, dx=None, dwg=None, dwu=None, dwd=None, workspace=None, linear=False):
    """Full backward. Overwrites the G/U planes of ``saved`` with dG/dU.
    Returns (dX, dWg, dWu, dWd), the weight gradients in their weights'
    layout. ``workspace``: at least ``bwd_workspace_bytes`` bytes (allocated
    here when None and needed)."""
    dy, x, wg, wu, wd = (t.contiguous() for t in (dy, x, wg, wu, wd))
    T, D, H = _shapes(x, wg, wu, wd, linear)
    if tuple(dy.shape) != (T, D) or dy.dtype != x.dtype or dy.device != x.device:
        raise ValueError("dY must match X in shape, dtype and device")
    if (not saved.is_contiguous() or saved.numel() != 3 * T * H or saved.dtype != x.dtype
            or saved.device != x.device):
        raise ValueError("saved must be the contiguous [3, T, H] buffer returned by fwd")
    dx, dwg, dwu, dwd = (_buf(dx, (T, D), x, "dx"), _buf(dwg, tuple(wg.shape), x, "dwg"),
                         _buf(dwu, tuple(wu.shape), x, "dwu"), _buf(dwd, tuple(wd.shape), x, "dwd"))
    need = bwd_workspace_bytes(T, D, H, x.dtype)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=x.device) if need else None
    elif workspace.device != x.device or not workspace.is_contiguous():
        raise ValueError(f"workspace must be a contiguous tensor on {x.device}")
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    rc = _L.lib().swiglu_mlp_bwd_ex(_p(dy), _p(x), _p(wg), _p(wu), _p(wd), _p(saved),
                                    _p(dx), _p(dwg), _p(dwu), _p(dwd), _p(workspace), ws_bytes,
                                    T, D, H, _dt(x), _flags(linear=linear), _stream(x.device))
    _check(rc, "swiglu_mlp_bwd_ex")
    return dx, dwg, dwu, dwd


def infer(x, wg, wu, wd, y=None, workspace=None, two_round=False, linear=False):
    """No-grad forward: only the workspace (A[T,H], plus arrival counters and
    fp32 partial sums for T <= 128; ``infer_workspace_bytes`` bytes) and
    Y[T,D] are written."""
    x, wg, wu, wd = (t.contiguous() for t in (x, wg, wu, wd))
    T, D, H = _shapes(x, wg, wu, wd, linear)
    y = _buf(y, (T, D), x, "y")
    if workspace is None:
        workspace = torch.empty(infer_workspace_bytes(T, D, H, x.dtype), dtype=torch.uint8, device=x.device)
    elif workspace.device != x.device or not workspace.is_contiguous():
        raise ValueError(f"workspace must be a contiguous tensor on {x.device}")
    nbytes = workspace.numel() * workspace.element_size()
    rc = _L.lib().swiglu_mlp_infer_ex(_p(x), _p(wg), _p(wu), _p(wd), _p(y), _p(workspace), nbytes,
                                      T, D, H, _dt(x), _flags(two_round, linear), _stream(x.device))
    _check(rc, "swiglu_mlp_infer_ex")
    return y


def infer_noalloc(x, wg, wu, wd, y=None, two_round=False, linear=False):
    """No-grad forward through the allocation-free entry point: the library's
    fixed per-device scratch holds the workspace (calls on one device must
    not overlap). Raises SwiGLUError (SWIGLU_ERR_SCRATCH) when the shape
    needs more than that scratch."""
    x, wg, wu, wd = (t.contiguous() for t in (x, wg, wu, wd))
    T, D, H = _shapes(x, wg, wu, wd, linear)
    y = _buf(y, (T, D), x, "y")
    rc = _L.lib().swiglu_mlp_infer_noalloc(_p(x), _p(wg), _p(wu), _p(wd), _p(y), T, D, H, _dt(x),
                                           _flags(two_round, linear), _stream(x.device))
    _check(rc, "swiglu_mlp_infer_noalloc")
    return y


class SwiGLUMLPFunction(torch.autograd.Function):
    """autograd.Function over fwd/bwd. The saved buffer is single-use: its
    G/U planes are overwritten by dG/dU during backward, so a second backward
    (retain_graph=True) or double backward (create_graph=True) is refused
    (issue #1347, section "Known limitations and validation gaps")."""

    @staticmethod
    def forward(ctx, x, wg, wu, wd, two_round=False, linear=False):
        y, saved = fwd(x, wg, wu, wd, two_round=two_round, linear=linear)
        ctx.save_for_backward(x, wg, wu, wd)
        ctx.saved_buf = saved
        ctx.linear = linear
        return y

    @staticmethod
    def backward(ctx, dy):
        if torch.is_grad_enabled():
            raise RuntimeError("swiglu_mlp: create_graph=True (double backward) is not supported")
        if ctx.saved_buf is None:
            raise RuntimeError("swiglu_mlp: backward called twice; the saved A|G|U buffer was "
                               "consumed by the first backward (retain_graph is not supported)")
        x, wg, wu, wd = ctx.saved_tensors
        saved, ctx.saved_buf = ctx.saved_buf, None
        dx, dwg, dwu, dwd = bwd(dy, x, wg, wu, wd, saved, linear=ctx.linear)
        return dx, dwg, dwu, dwd, None, None


def swiglu_mlp(x, wg, wu, wd, two_round=False, linear=False):
    """Y = (SiLU(x Wg) * (x Wu)) Wd for x[..., D] (with ``linear``, the
    nn.Linear weights: Y = down(SiLU(gate(x)) * up(x))). Uses the no-grad
    path when autograd does not need gradients."""
    lead = x.shape[:-1]
    x2 = x.reshape(-1, x.shape[-1])
    needs = torch.is_grad_enabled() and any(t.requires_grad for t in (x, wg, wu, wd))
    if needs:
        y = SwiGLUMLPFunction.apply(x2, wg, wu, wd, two_round, linear)
    else:
        y = infer(x2, wg, wu, wd, two_round=two_round, linear=linear)
    return y.reshape(*lead, x.shape[-1])


class SwiGLUMLP(torch.nn.Module):
    """Drop-in for the transformers ``xxxMLP`` modules of SwiGLU models (for
    example ``LlamaMLP``): the same ``__init__(config)`` and ``forward(x)``
    signatures, the same submodules ``gate_proj``, ``up_proj`` (hidden_size
    -> intermediate_size) and ``down_proj`` (intermediate_size ->
    hidden_size) as bias-free nn.Linear layers, so a state dict of such a
    module loads unchanged, and y = down_proj(SiLU(gate_proj(x)) *
    up_proj(x)) computed by the fused kernels, which read the nn.Linear
    weights in place. Standard SwiGLU only: ``config.mlp_bias`` must be false
    and ``config.hidden_act`` "silu" (or "swish"). Parameters must be bf16,
    fp16 or fp32 on a gfx950 GPU. ``two_round`` (keyword) selects the
    historical two-round SwiGLU epilogue."""

    def __init__(self, config, two_round=False):
        super().__init__()
        if getattr(config, "mlp_bias", False):
            raise ValueError("SwiGLUMLP has no bias terms (config.mlp_bias must be False)")
        act = getattr(config, "hidden_act", "silu")
        if act not in ("silu", "swish"):
            raise ValueError(f"SwiGLUMLP computes SiLU gating; config.hidden_act is {act!r}")
        self.config = config
        self.hidden_size = int(config.hidden_size)
        self.intermediate_size = int(config.intermediate_size)
        self.two_round = bool(two_round)
        self.gate_proj = torch.nn.Linear(self.hidden_size, self.intermediate_size, bias=False)
        self.up_proj = torch.nn.Linear(self.hidden_size, self.intermediate_size, bias=False)
        self.down_proj = torch.nn.Linear(self.intermediate_size, self.hidden_size, bias=False)

    def forward(self, x):
        return swiglu_mlp(x, self.gate_proj.weight, self.up_proj.weight, self.down_proj.weight,
                          two_round=self.two_round, linear=True)

    def extra_repr(self):
        return "two_round=True" if self.two_round else ""


class SwiGLUMLPPacked(torch.nn.Module):
    """SwiGLU MLP block with the weights in the kernels' own layout:
    ``w_gate``, ``w_up`` [D, H] and ``w_down`` [H, D] (row-major), y =
    (SiLU(x Wg) * (x Wu)) Wd on x[..., D]. ``from_linears`` converts an
    nn.Linear triple (weights [H, D] and [D, H]) once; ``SwiGLUMLP`` uses
    the nn.Linear layout directly instead."""

    def __init__(self, hidden_size, intermediate_size, dtype=torch.bfloat16, device=None, generator=None,
                 two_round=False):
        super().__init__()
        self.two_round = bool(two_round)
        D, H = int(hidden_size), int(intermediate_size)
        kw = {"dtype": torch.float32, "device": "cpu"}
        # normal init with variance 1/fan_in keeps G, U and Y at the scale of x
        wg = torch.randn(D, H, generator=generator, **kw) / D ** 0.5
        wu = torch.randn(D, H, generator=generator, **kw) / D ** 0.5
        wd = torch.randn(H, D, generator=generator, **kw) / H ** 0.5
        mk = lambda t: torch.nn.Parameter(t.to(dtype=dtype, device=device))
        self.w_gate, self.w_up, self.w_down = mk(wg), mk(wu), mk(wd)

    @classmethod
    def from_linears(cls, gate_proj, up_proj, down_proj, two_round=False):
        """Build from nn.Linear layers (gate_proj, up_proj: D -> H; down_proj:
        H -> D; no bias), copying their weights into the kernels' layout."""
        for lin in (gate_proj, up_proj, down_proj):
            if lin.bias is not None:
                raise ValueError("SwiGLUMLPPacked has no bias terms")
        H, D = gate_proj.weight.shape
        w = gate_proj.weight
        m = cls.__new__(cls)
        torch.nn.Module.__init__(m)
        m.two_round = bool(two_round)
        mk = lambda t: torch.nn.Parameter(t.detach().t().contiguous())
        m.w_gate, m.w_up, m.w_down = mk(gate_proj.weight), mk(up_proj.weight), mk(down_proj.weight)
        if tuple(m.w_down.shape) != (H, D) or m.w_up.shape != m.w_gate.shape or m.w_gate.dtype != w.dtype:
            raise ValueError("gate_proj, up_proj must map D -> H and down_proj H -> D")
        return m

    @property
    def hidden_size(self):
        return self.w_gate.shape[0]

    @property
    def intermediate_size(self):
        return self.w_gate.shape[1]

    def forward(self, x):
        return swiglu_mlp(x, self.w_gate, self.w_up, self.w_down, two_round=self.two_round)

    def extra_repr(self):
        r = f"hidden_size={self.hidden_size}, intermediate_size={self.intermediate_size}"
        return r + (", two_round=True" if self.two_round else "")


class StageTimer:
    """HIP-event timing of each kernel launch, recorded by the library on the
    launch stream (profiling aid). Use as a context manager around a timed
    loop; ``ms[name]`` holds the summed milliseconds and ``count[name]`` the
    launches."""

    def __init__(self, capacity=4096):
        self.capacity = capacity
        self.ms, self.count = {}, {}

    def __enter__(self):
        _check(_L.lib().swiglu_mlp_timer_start(self.capacity), "swiglu_mlp_timer_start")
        return self

    def __exit__(self, *exc):
        ms = (ctypes.c_double * NUM_STAGES)()
        cnt = (ctypes.c_int * NUM_STAGES)()
        _check(_L.lib().swiglu_mlp_timer_stop(ms, cnt, NUM_STAGES), "swiglu_mlp_timer_stop")
        self.ms = {STAGE_NAMES[i]: ms[i] for i in range(NUM_STAGES)}
        self.count = {STAGE_NAMES[i]: cnt[i] for i in range(NUM_STAGES)}
        return False
