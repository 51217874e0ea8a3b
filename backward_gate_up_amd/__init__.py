"""Fused SwiGLU MLP for MI355X (gfx950): Python binding of libswiglu_mlp.so.

This module only marshals arguments: every arithmetic step runs in the HIP
kernels behind the C ABI declared in include/swiglu_mlp.h. PyTorch supplies
device memory and the current stream. There is no fallback: if the library
is missing or the device is not gfx950, calls raise.

Three levels, following the maintainers' layering on "[RFC] Full-pipeline
SwiGLU MLP with forward/backward co-optimization" (Liger-Kernel issue #1347,
discussion thread): op-level wrappers (fwd / bwd / infer), an autograd
Function composing them, and the ``swiglu_mlp`` convenience entry that
flattens [..., D] inputs and picks the no-grad path when autograd is off.
"""

import ctypes

import torch

from . import _lib as _L
from ._lib import SwiGLUError, STAGE_NAMES, NUM_STAGES  # noqa: F401

__all__ = ["fwd", "bwd", "infer", "SwiGLUMLPFunction", "swiglu_mlp", "saved_bytes",
           "infer_workspace_bytes", "SwiGLUError", "StageTimer"]

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


def _shapes(x, wg, wu, wd):
    if x.dim() != 2 or wg.dim() != 2 or wu.dim() != 2 or wd.dim() != 2:
        raise ValueError("expected X[T,D], Wg[D,H], Wu[D,H], Wd[H,D]")
    T, D = x.shape
    if wg.shape[0] != D or wu.shape != wg.shape or tuple(wd.shape) != (wg.shape[1], D):
        raise ValueError(f"shape mismatch: X{tuple(x.shape)} Wg{tuple(wg.shape)} "
                         f"Wu{tuple(wu.shape)} Wd{tuple(wd.shape)}")
    for t in (wg, wu, wd):
        if t.dtype != x.dtype or t.device != x.device:
            raise ValueError("all tensors must share dtype and device")
    if x.device.type != "cuda":
        raise ValueError("tensors must be on a GPU (cuda/HIP device)")
    return T, D, wg.shape[1]


def saved_bytes(T, H, dtype=torch.bfloat16):
    return _L.lib().swiglu_mlp_saved_bytes(T, H, _DT[dtype])


def infer_workspace_bytes(T, D, H, dtype=torch.bfloat16):
    return _L.lib().swiglu_mlp_infer_workspace_bytes(T, D, H, _DT[dtype])


def fwd(x, wg, wu, wd, y=None, saved=None):
    """Training forward. Returns (Y[T,D], saved) where ``saved`` is the
    [3, T, H] A|G|U buffer that ``bwd`` consumes."""
    x, wg, wu, wd = (t.contiguous() for t in (x, wg, wu, wd))
    T, D, H = _shapes(x, wg, wu, wd)
    if y is None:
        y = torch.empty((T, D), dtype=x.dtype, device=x.device)
    if saved is None:
        saved = torch.empty((3, T, H), dtype=x.dtype, device=x.device)
    rc = _L.lib().swiglu_mlp_fwd(_p(x), _p(wg), _p(wu), _p(wd), _p(y), _p(saved),
                                 T, D, H, _dt(x), _stream(x.device))
    _check(rc, "swiglu_mlp_fwd")
    return y, saved


def bwd(dy, x, wg, wu, wd, saved, dx=None, dwg=None, dwu=None, dwd=None):
    """Full backward. Overwrites the G/U planes of ``saved`` with dG/dU.
    Returns (dX, dWg, dWu, dWd)."""
    dy, x, wg, wu, wd = (t.contiguous() for t in (dy, x, wg, wu, wd))
    T, D, H = _shapes(x, wg, wu, wd)
    if tuple(dy.shape) != (T, D) or dy.dtype != x.dtype:
        raise ValueError("dY must match X in shape and dtype")
    if not saved.is_contiguous() or saved.numel() != 3 * T * H or saved.dtype != x.dtype:
        raise ValueError("saved must be the contiguous [3, T, H] buffer returned by fwd")
    mk = lambda t, shape: torch.empty(shape, dtype=x.dtype, device=x.device) if t is None else t
    dx, dwg, dwu, dwd = mk(dx, (T, D)), mk(dwg, (D, H)), mk(dwu, (D, H)), mk(dwd, (H, D))
    rc = _L.lib().swiglu_mlp_bwd(_p(dy), _p(x), _p(wg), _p(wu), _p(wd), _p(saved),
                                 _p(dx), _p(dwg), _p(dwu), _p(dwd), None, 0,
                                 T, D, H, _dt(x), _stream(x.device))
    _check(rc, "swiglu_mlp_bwd")
    return dx, dwg, dwu, dwd


def infer(x, wg, wu, wd, y=None, workspace=None):
    """No-grad forward: only A[T,H] (the workspace) and Y[T,D] are written."""
    x, wg, wu, wd = (t.contiguous() for t in (x, wg, wu, wd))
    T, D, H = _shapes(x, wg, wu, wd)
    if y is None:
        y = torch.empty((T, D), dtype=x.dtype, device=x.device)
    if workspace is None:
        workspace = torch.empty((T, H), dtype=x.dtype, device=x.device)
    nbytes = workspace.numel() * workspace.element_size()
    rc = _L.lib().swiglu_mlp_infer(_p(x), _p(wg), _p(wu), _p(wd), _p(y), _p(workspace), nbytes,
                                   T, D, H, _dt(x), _stream(x.device))
    _check(rc, "swiglu_mlp_infer")
    return y


class SwiGLUMLPFunction(torch.autograd.Function):
    """autograd.Function over fwd/bwd. The saved buffer is single-use: its
    G/U planes are overwritten by dG/dU during backward, so a second backward
    (retain_graph=True) or double backward (create_graph=True) is refused
    (issue #1347, section "Known limitations and validation gaps")."""

    @staticmethod
    def forward(ctx, x, wg, wu, wd):
        y, saved = fwd(x, wg, wu, wd)
        ctx.save_for_backward(x, wg, wu, wd)
        ctx.saved_buf = saved
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
        dx, dwg, dwu, dwd = bwd(dy, x, wg, wu, wd, saved)
        return dx, dwg, dwu, dwd


def swiglu_mlp(x, wg, wu, wd):
    """Y = (SiLU(x Wg) * (x Wu)) Wd for x[..., D]. Uses the no-grad path when
    autograd does not need gradients."""
    lead = x.shape[:-1]
    x2 = x.reshape(-1, x.shape[-1])
    needs = torch.is_grad_enabled() and any(t.requires_grad for t in (x, wg, wu, wd))
    y = SwiGLUMLPFunction.apply(x2, wg, wu, wd) if needs else infer(x2, wg, wu, wd)
    return y.reshape(*lead, wd.shape[1])


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
