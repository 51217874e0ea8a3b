"""The C ABI: the library loads, exports every declared symbol, answers size
queries, and rejects bad arguments from the host before touching a device.

The CPU tests never launch work: every call either is a pure size query or
fails validation before any HIP call (null, shape, dtype, alignment,
aliasing). GPU-marked tests cover the device check and the binding's guards.
"""

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "swiglu_mlp.h")


def _lib():
    from backward_gate_up_amd import _lib

    return _lib.lib()


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(swiglu_mlp_\w+)\s*\(", src)))


def test_library_exports_every_declared_symbol():
    names = _declared()
    assert {"swiglu_mlp_fwd", "swiglu_mlp_bwd", "swiglu_mlp_infer"} <= set(names)
    L = _lib()
    for n in names:
        assert hasattr(L, n), n
        assert ctypes.cast(getattr(L, n), ctypes.c_void_p).value


def test_size_queries():
    L = _lib()
    assert L.swiglu_mlp_saved_bytes(65536, 11008, 0) == 3 * 65536 * 11008 * 2
    assert L.swiglu_mlp_saved_bytes(4096, 5632, 2) == 3 * 4096 * 5632 * 4
    assert L.swiglu_mlp_saved_bytes(10, 16, 9) == 0
    assert L.swiglu_mlp_infer_workspace_bytes(256, 4096, 11008, 0) == 256 * 11008 * 2
    # weight gradients: whole rounds of 256 tiles run unsplit; the tiles of a
    # partly filled last round are split over K into fp32 partial tiles
    # (256 KiB each). D=4096, H=11008: dWd has 43 x 16 = 688 tiles = 2 rounds
    # + 176, split 4 ways; [dWg | dWu] has 1376 = 5 rounds + 96, split 5 ways.
    assert L.swiglu_mlp_bwd_workspace_bytes(65536, 4096, 11008, 0) == 176 * 4 * 256 * 256 * 4
    assert L.swiglu_mlp_bwd_workspace_bytes(65536, 4096, 8192, 0) == 0    # 512 and 1024 tiles: whole rounds
    assert L.swiglu_mlp_bwd_workspace_bytes(16384, 1024, 2816, 0) > 0     # split-K weight gradients
    assert L.swiglu_mlp_bwd_workspace_bytes(16384, 1024, 2816, 2) == 0    # fp32 engine: no split
    assert L.swiglu_mlp_bwd_workspace_bytes(512, 1024, 2816, 0) == 0      # small-T engine


def test_infer_memory_matches_pages_table():
    # Inference intermediate memory on the pages = A + Y (tests/golden/infer_memory.txt)
    L = _lib()
    MiB = float(1 << 20)
    with open(os.path.join(ROOT, "tests", "golden", "infer_memory.txt")) as f:
        rows = [[float(v) for v in ln.split()] for ln in f if ln.strip() and not ln.startswith("#")]
    for D, H, S, mb in rows:
        T, D, H = int(S), int(D), int(H)
        a = L.swiglu_mlp_infer_workspace_bytes(T, D, H, 0)
        y = T * D * 2
        assert round((a + y) / MiB, 1) == mb


def test_status_strings():
    L = _lib()
    for s in range(11):
        assert len(L.swiglu_mlp_status_string(s)) > 0
    assert L.swiglu_mlp_status_string(99) == b"unknown status"


# Fake, never-dereferenced device addresses: validation fails before any use.
BASE = 1 << 40


def _fwd(L, X=BASE, Wg=BASE + (1 << 30), Wu=BASE + (2 << 30), Wd=BASE + (3 << 30),
         Y=BASE + (4 << 30), S=BASE + (5 << 30), T=16, D=64, H=128, dt=0):
    return L.swiglu_mlp_fwd(X, Wg, Wu, Wd, Y, S, T, D, H, dt, None)


def test_host_validation_codes():
    L = _lib()
    assert _fwd(L, dt=7) == 3                      # dtype
    assert _fwd(L, T=-1) == 2                      # shape
    assert _fwd(L, D=60) == 2 and _fwd(L, H=0) == 2
    assert _fwd(L, X=None) == 1                    # null
    assert _fwd(L, Wd=BASE + (3 << 30) + 8) == 4   # alignment
    assert _fwd(L, Y=BASE + 64) == 5               # Y overlaps X
    assert _fwd(L, S=BASE + (1 << 30)) == 5        # saved overlaps Wg
    assert _fwd(L, S=BASE + (4 << 30) + 16) == 5   # saved overlaps Y
    # bwd: output overlapping the saved buffer, and two overlapping outputs
    b = [BASE + (i << 30) for i in range(11)]
    args = lambda **kw: [kw.get(n, b[i]) for i, n in enumerate(
        ["dY", "X", "Wg", "Wu", "Wd", "S", "dX", "dWg", "dWu", "dWd", "ws"])]
    call = lambda a, T=16: L.swiglu_mlp_bwd(*a[:10], None, 0, T, 64, 128, 0, None)
    assert call(args(dX=b[5] + 32)) == 5
    assert call(args(dWu=b[7] + 16)) == 5
    assert call(args(dWd=None)) == 1
    # a split-K shape needs a workspace: missing, too small, overlapping
    T, D, H = 16384, 1024, 2816
    need = L.swiglu_mlp_bwd_workspace_bytes(T, D, H, 0)
    callw = lambda a, ws, n: L.swiglu_mlp_bwd(*a[:10], ws, n, T, D, H, 0, None)
    big = [BASE + (i << 34) for i in range(11)]
    bargs = [big[i] for i in range(10)]
    assert callw(bargs, None, 0) == 6
    assert callw(bargs, big[10], need - 16) == 6
    assert callw(bargs, big[10] + 8, need) == 4
    assert callw(bargs, big[9] + 64, need) == 5
    # infer: workspace too small, then missing
    assert L.swiglu_mlp_infer(b[0], b[1], b[2], b[3], b[4], b[5], 16 * 128 * 2 - 2, 16, 64, 128, 0, None) == 6
    assert L.swiglu_mlp_infer(b[0], b[1], b[2], b[3], b[4], None, 0, 16, 64, 128, 0, None) == 6


def test_empty_token_count_allows_null_token_buffers():
    L = _lib()
    # T = 0: X, Y, saved may be NULL; validation then reaches the device check
    rc = _fwd(L, X=None, Y=None, S=None, T=0)
    assert rc in (0, 7)  # 7 without a gfx950 device (this host), 0 with one


def test_no_device_is_reported_not_crashed():
    import torch

    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    assert _fwd(_lib()) == 7


def test_unknown_flags_rejected_before_anything_else():
    L = _lib()
    b = [BASE + (i << 30) for i in range(7)]
    for bad in (4, 8, 0x80000000):
        assert L.swiglu_mlp_fwd_ex(*b[:6], 16, 64, 128, 0, bad, None) == 9
        assert L.swiglu_mlp_infer_ex(*b[:6], 16 * 128 * 2, 16, 64, 128, 0, bad, None) == 9
        assert L.swiglu_mlp_bwd_ex(*[b[i % 7] + (i << 34) for i in range(10)], None, 0, 16, 64, 128, 0, bad,
                                   None) == 9
    # a bad dtype is reported first; known flags pass to the remaining checks
    assert L.swiglu_mlp_fwd_ex(*b[:6], 16, 64, 128, 7, 4, None) == 3
    assert L.swiglu_mlp_fwd_ex(b[0], b[1], b[2], b[3], b[0] + 64, b[5], 16, 64, 128, 0, 3, None) == 5
    assert L.swiglu_mlp_fwd_ex(b[0], b[1], b[2], b[3], b[0] + 64, b[5], 16, 64, 128, 0, 1, None) == 5
    assert L.swiglu_mlp_infer_ex(*b[:5], None, 0, 16, 64, 128, 0, 1, None) == 6


def test_shape_limits_of_32_bit_lane_offsets():
    """D and H are the leading dimensions of every operand. A tile spans 256
    rows, so its lane offsets reach 256 * ld * elt_bytes, which must stay
    below 2^31: D, H <= 4194296 for bf16/fp16 and <= 2097144 for fp32
    (multiples of 8). Just inside the limit the call gets past the shape
    check and fails on the misaligned Wd; just outside it returns
    SWIGLU_ERR_SHAPE. Nothing is launched either way."""
    L = _lib()
    far = [1 << 44, 2 << 44, 3 << 44, 4 << 44, 5 << 44, 6 << 44]
    for dt, lim in ((0, 4194296), (1, 4194296), (2, 2097144)):
        for which in ("D", "H"):
            def call(v, misalign=True):
                D, H = (v, 64) if which == "D" else (64, v)
                b = list(far)
                if misalign:
                    b[3] += 8
                return L.swiglu_mlp_fwd(*b, 16, D, H, dt, None)
            assert call(lim) == 4, (dt, which)            # past the shape check
            assert call(lim + 8) == 2, (dt, which)        # SWIGLU_ERR_SHAPE
            assert L.swiglu_mlp_infer(*far[:5], far[5], 1 << 40, 16, *((lim + 8, 64) if which == "D" else (64, lim + 8)),
                                      dt, None) == 2
    # the tile count of a launch must fit in int32
    assert L.swiglu_mlp_fwd(*far[:3], far[3] + 8, *far[4:], (1 << 31) - 1, 8, 8, 0, None) == 4
    assert L.swiglu_mlp_fwd(*far, (1 << 31) - 1, 4194296, 64, 0, None) == 2


def test_no_grad_intermediate_memory_bound():
    """No-grad intermediate memory (workspace + Y) at B=1, S = 1 ... 256 for
    both inference shapes of the pages: within 3 (A + Y) at every S (the
    split-K partials of the down projection are capped), and exactly A + Y
    where no K is split (S = 256, and fp32). The pages' table ("[RFC]
    Full-pipeline SwiGLU MLP ...", "Intermediate-memory results") gives A + Y
    at S = 256."""
    L = _lib()
    for D, H in ((1024, 2816), (4096, 11008)):
        for S in (1, 2, 4, 8, 16, 32, 64, 128, 256):
            a_y = 2 * S * (H + D)
            ws = L.swiglu_mlp_infer_workspace_bytes(S, D, H, 0)
            assert ws >= 2 * S * H
            assert ws + 2 * S * D <= 3 * a_y, (D, S, ws)
            assert L.swiglu_mlp_infer_workspace_bytes(S, D, H, 2) == 4 * S * H
        assert L.swiglu_mlp_infer_workspace_bytes(256, D, H, 0) + 2 * 256 * D == 2 * 256 * (H + D)


def test_noalloc_rejects_shapes_beyond_its_scratch():
    """The allocation-free no-grad entry point checks its fixed scratch on
    the host: a shape whose workspace exceeds it returns SWIGLU_ERR_SCRATCH
    before anything else that touches a device."""
    from backward_gate_up_amd._lib import NOALLOC_SCRATCH_BYTES

    L = _lib()
    b = [BASE + (i << 36) for i in range(5)]
    D, H = 4096, 11008
    assert L.swiglu_mlp_infer_workspace_bytes(1524, D, H, 0) <= NOALLOC_SCRATCH_BYTES
    assert L.swiglu_mlp_infer_workspace_bytes(1525, D, H, 0) > NOALLOC_SCRATCH_BYTES
    assert L.swiglu_mlp_infer_noalloc(*b, 1525, D, H, 0, 0, None) == 10
    assert L.swiglu_mlp_infer_noalloc(*b, 1 << 20, D, H, 2, 0, None) == 10
    assert L.swiglu_mlp_infer_noalloc(*b, 16, D, H, 0, 4, None) == 9        # flags
    assert L.swiglu_mlp_infer_noalloc(*b[:4], b[0] + 64, 16, D, H, 0, 0, None) == 5  # Y overlaps X
