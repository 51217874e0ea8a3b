"""The allocation-free no-grad entry point (GPU), through the C ABI.

swiglu_mlp_infer_noalloc keeps its workspace in a fixed per-device scratch
array of the library. Its output must equal, bit for bit, that of
swiglu_mlp_infer (same kernels, same launch plan, deterministic reduction)
on two calls in a row, the second with a smaller input (the scratch keeps
the first call's contents, including the arrival counters the call must
clear), and be within the oracle's bound. A shape beyond the scratch is
refused on the host.
"""

import ctypes

import pytest
import torch

import oracle as O
from synth import make_inputs
from tests._util import assert_local, banner, f64, fmt_local, to_dev

pytestmark = pytest.mark.gpu


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr())


def _infer(L, g, noalloc):
    T, D = g["X"].shape
    H = g["Wg"].shape[1]
    y = torch.full((T, D), float("nan"), dtype=g["X"].dtype, device="cuda")
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    args = [_ptr(g[k]) for k in ("X", "Wg", "Wu", "Wd")] + [_ptr(y)]
    if noalloc:
        rc = L.swiglu_mlp_infer_noalloc(*args, T, D, H, 0, 0, stream)
    else:
        nbytes = L.swiglu_mlp_infer_workspace_bytes(T, D, H, 0)
        ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
        rc = L.swiglu_mlp_infer(*args, _ptr(ws), nbytes, T, D, H, 0, stream)
    assert rc == 0, rc
    torch.cuda.synchronize()
    return y


@pytest.mark.parametrize("first,second", [((120, 4096, 11008), (5, 1024, 2816)),
                                          ((300, 1024, 2816), (77, 4096, 11008))])
def test_noalloc_matches_infer(first, second):
    from backward_gate_up_amd import _lib

    L = _lib.lib()
    for T, D, H in (first, second):
        banner(f"noalloc T={T} D={D} H={H}")
        inp = make_inputs(T, D, H, seed=T + D, dtype="bf16", with_dy=False)
        g = to_dev(inp)
        y_na = _infer(L, g, noalloc=True)
        y_ref = _infer(L, g, noalloc=False)
        assert torch.equal(y_na, y_ref), (T, D, H)
        f = {k: v.float().numpy() for k, v in inp.items()}
        e = assert_local(f64(y_na), O.infer(f["X"], f["Wg"], f["Wu"], f["Wd"]), 1e-2, ("noalloc", T, D, H))
        banner(f"  bitwise equal to swiglu_mlp_infer; vs oracle {fmt_local(e)}")


def test_noalloc_refuses_shape_beyond_scratch():
    from backward_gate_up_amd import _lib
    from backward_gate_up_amd import infer_noalloc, SwiGLUError

    g = to_dev(make_inputs(1600, 4096, 11008, seed=9, dtype="bf16", with_dy=False))
    with pytest.raises(SwiGLUError, match="SCRATCH"):
        infer_noalloc(g["X"], g["Wg"], g["Wu"], g["Wd"])
    assert _lib.lib().swiglu_mlp_infer_workspace_bytes(1600, 4096, 11008, 0) > _lib.NOALLOC_SCRATCH_BYTES
