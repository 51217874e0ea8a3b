"""Parity of the HIP path with the fp64 oracle (GPU).

Bounds: normalized L2 <= 1e-2 for bf16/fp16 outputs and gradients, <= 1e-5
in fp32 mode, over the whole tensor and also over every row, every 32 x 32
block and every 256 x 256 tile (tests/_util.py, local_errors), so that one
wrong row, matrix-core block or split-K tile cannot hide in the global
figure; the forward SwiGLU epilogue within 1 ulp of the correctly rounded
SiLU(g)*u of the GPU's own stored g, u. Small shapes exercise ragged tails in
every dimension; the pages' training shapes run in full; the largest one
(T = 65536, D = 4096, H = 11008) is checked in the same launch configuration
the benchmark times, on one row in every 32-row block and one hidden unit in
every 32-unit block, which touches every 32 x 32 block row and every tile of
each output, including every weight-gradient tile that the library splits
over K.
"""

import numpy as np
import pytest
import torch

import oracle as O
from synth import WORKLOADS, make_inputs, workload_inputs
from tests._util import SAMPLED, TOL, assert_local, banner, f64, fmt_local, nl2, run_train, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def mlp():
    import backward_gate_up_amd as m

    return m


def _np(inp):
    return {k: v.float().numpy() for k, v in inp.items()}


def _check_full(mlp, inp, fmt, label, check_planes=True):
    banner(f"{label}: GPU fwd+bwd")
    out = run_train(mlp, to_dev(inp))
    f = _np(inp)
    banner(f"{label}: oracle")
    ref = O.bwd(f["dY"], f["X"], f["Wg"], f["Wu"], f["Wd"], keep=check_planes)
    if not check_planes:
        ref["Y"] = O.fwd(f["X"], f["Wg"], f["Wu"], f["Wd"])["Y"]
    tol = TOL[fmt]
    keys = ["Y", "dI", "dWg", "dWu", "dWd"] + (["G", "U", "dG", "dU"] if check_planes else [])
    errs = {}
    for k in keys:
        errs[k] = assert_local(f64(out[k]), ref[k], tol, (label, k))
        banner(f"{label}: {k} {fmt_local(errs[k])}")
    # the backward leaves the A plane untouched
    assert torch.equal(out["A"], out["A_after"])
    # forward epilogue: A within 1 ulp of rnd(SiLU(g) u) from the stored g, u
    if fmt != "fp32":
        a_ref = O.round_to(O.epilogue_fwd(f64(out["G"]), f64(out["U"])), fmt)
        ulp = O.ulp_distance(f64(out["A"]), a_ref, fmt)
        assert int(ulp.max()) <= 1, (label, int(ulp.max()))
    return out, errs


@pytest.mark.parametrize("T,D,H", [
    (1, 64, 64), (3, 64, 128), (5, 136, 200), (40, 264, 520), (64, 200, 136),
    (127, 256, 384), (129, 512, 264), (300, 1024, 2816), (513, 256, 512), (1000, 384, 648), (777, 136, 200),
    # T > 512 with D = 104 and 40: the five-array K loops over D have 2 stages
    # (the second with a K tail) and 1 stage
    (600, 104, 200), (530, 40, 72),
])
def test_ragged_shapes_bf16(mlp, T, D, H):
    inp = make_inputs(T, D, H, seed=T + D + H, dtype="bf16")
    _check_full(mlp, inp, "bf16", f"T={T} D={D} H={H}")


def test_workload_T128(mlp):
    _check_full(mlp, workload_inputs("mlp_1024x2816_T128"), "bf16", "1024x2816 T=128")


def test_workload_T16384(mlp):
    _check_full(mlp, workload_inputs("mlp_1024x2816_T16384"), "bf16", "1024x2816 T=16384")


def test_workload_T32768(mlp):
    _check_full(mlp, workload_inputs("mlp_2048x5632_T32768"), "bf16", "2048x5632 T=32768",
                check_planes=False)


@pytest.mark.parametrize("P", [8])
def test_tensor_parallel_shard_shape(mlp, P):
    """D=4096 and H = 11008 / P, the shape each GPU of a tensor-parallel
    group runs (Wg, Wu split by columns, Wd by rows), at T=4096."""
    H = 11008 // P
    _check_full(mlp, make_inputs(4096, 4096, H, seed=4242 + P, dtype="bf16"), "bf16",
                f"TP shard P={P}: T=4096 D=4096 H={H}", check_planes=False)


def test_weight_gradient_split_remainder_ragged(mlp):
    """Weight gradients with whole rounds of tiles plus split leftovers, on
    ragged edges: at T=8192, D=1032, H=6664 (256 x 256 tiles: 5 x 27 per
    plane), [dWg | dWu] has 270 tiles, one round of 256 on the 256 CUs and
    14 tiles split over K into 8 pieces; dWd's 135 tiles, under one round,
    are all split (3 pieces). Everything against the oracle in full."""
    _check_full(mlp, make_inputs(8192, 1032, 6664, seed=8192, dtype="bf16"), "bf16",
                "split remainder T=8192 D=1032 H=6664", check_planes=False)


def test_fp32_mode_T4096(mlp):
    _check_full(mlp, workload_inputs("mlp_2048x5632_T4096_fp32", dtype="fp32"), "fp32",
                "fp32 2048x5632 T=4096")


def test_fp16_T16384(mlp):
    _check_full(mlp, workload_inputs("mlp_1024x2816_T16384", dtype="fp16"), "fp16",
                "fp16 1024x2816 T=16384")


def test_fp32_and_fp16_ragged(mlp):
    for fmt in ("fp32", "fp16"):
        inp = make_inputs(333, 136, 264, seed=5, dtype=fmt)
        _check_full(mlp, inp, fmt, f"{fmt} T=333 D=136 H=264")


def test_fp32_ragged_large_t(mlp):
    # fp32 above 512 tokens: the down projection has fewer 256 x 256 tiles
    # than CUs and runs on 64-row tiles, here with ragged M (777 = 12 * 64 +
    # 9) and N (136 < 256)
    inp = make_inputs(777, 136, 200, seed=78, dtype="fp32")
    _check_full(mlp, inp, "fp32", "fp32 T=777 D=136 H=200")


def test_fp16_ragged_ring(mlp):
    # T > 512 takes the ring kernels; D and H leave a K tail in every stage
    # (136, 200 = 8 mod 32 and mod 64)
    inp = make_inputs(777, 136, 200, seed=77, dtype="fp16")
    _check_full(mlp, inp, "fp16", "fp16 T=777 D=136 H=200")


def _one_per_block(n, rng, b=32):
    """One index in every b-wide block of range(n) (the last block may be
    partial), drawn at random within the block."""
    starts = np.arange(0, n, b)
    return starts + rng.integers(0, np.minimum(b, n - starts))


def _tiles_touched(idx, n, t=256):
    return set((np.asarray(idx) // t).tolist()) == set(range((n + t - 1) // t))


def _check_sampled(label, got, ref, tol=1e-2):
    """Sampled rows (or transposed sampled columns) against the oracle: each
    sampled line, and each 32- and 256-element segment of it (the footprint
    of a matrix-core block and of a tile), within tol."""
    e = assert_local(got, ref, tol, label, **SAMPLED)
    banner(f"{label} {fmt_local(e)}")


def test_headline_T65536_sampled(mlp):
    """D=4096, H=11008, T=65536 through the same calls the benchmark times.
    Rows: one in every 32-row block (2048 rows) of Y, dI and of the saved
    planes G, U (after fwd) and dG, dU (after bwd). Hidden units: one in every
    32-unit block (344 units) for dWg and dWu (columns) and dWd (rows). Every
    256 x 256 tile of every output is touched, so every tile of dWd and of
    [dWg | dWu] that the library splits over K (the 176 x 4 and 96 x 5 pieces
    of its workspace) is checked too."""
    T, D, H = 65536, 4096, 11008
    banner("T=65536: inputs")
    inp = workload_inputs("mlp_4096x11008_T65536")
    g = to_dev(inp)
    rng = np.random.default_rng(65536)
    rows = _one_per_block(T, rng)
    hs = _one_per_block(H, rng)
    assert _tiles_touched(rows, T) and _tiles_touched(hs, H)
    assert mlp.bwd_workspace_bytes(T, D, H) == (176 * 4) * 256 * 256 * 4
    banner("T=65536: GPU fwd+bwd")
    y, saved = mlp.fwd(g["X"], g["Wg"], g["Wu"], g["Wd"])
    ridx = torch.as_tensor(rows, device="cuda")
    A_s, G_s, U_s = (saved[i].index_select(0, ridx) for i in (0, 1, 2))
    dx, dwg, dwu, dwd = mlp.bwd(g["dY"], g["X"], g["Wg"], g["Wu"], g["Wd"], saved)
    dG_s, dU_s = (saved[i].index_select(0, ridx) for i in (1, 2))
    hidx = torch.as_tensor(hs, device="cuda")
    got = {"Y": y.index_select(0, ridx), "dI": dx.index_select(0, ridx), "G": G_s, "U": U_s, "dG": dG_s,
           "dU": dU_s, "dWg": dwg.index_select(1, hidx).t(), "dWu": dwu.index_select(1, hidx).t(),
           "dWd": dwd.index_select(0, hidx)}
    got = {k: f64(v) for k, v in got.items()}
    a_s = f64(A_s)
    torch.cuda.synchronize()
    del g, y, saved, dx, dwg, dwu, dwd
    f = _np(inp)
    banner("T=65536: oracle rows")
    r = O.rows(rows, f["X"], f["Wg"], f["Wu"], f["Wd"], f["dY"])
    a_ref = O.round_to(O.epilogue_fwd(got["G"], got["U"]), "bf16")
    assert int(O.ulp_distance(a_s, a_ref, "bf16").max()) <= 1
    for k in ("Y", "dI", "G", "U", "dG", "dU"):
        _check_sampled(f"T=65536 {k}", got[k], r[k])
    banner("T=65536: oracle hidden units")
    c = O.cols(hs, f["X"], f["Wg"], f["Wu"], f["Wd"], f["dY"])
    _check_sampled("T=65536 dWg", got["dWg"], c["dWg"].T)
    _check_sampled("T=65536 dWu", got["dWu"], c["dWu"].T)
    _check_sampled("T=65536 dWd", got["dWd"], c["dWd"])


def test_planes_over_2GiB_sampled(mlp):
    """T = 131072, D = 4096, H = 11008: each [T, H] plane of the saved buffer
    is 2.9 GB, past the 2 GiB range of one buffer descriptor (the kernels
    rebase their descriptors per tile and K stage). Sampled rows on both
    sides of byte offset 2^31 in the planes, and sampled hidden units of the
    weight gradients, against the oracle."""
    T, D, H = 131072, 4096, 11008
    banner(f"T={T}: inputs")
    inp = make_inputs(T, D, H, seed=77, dtype="bf16")
    g = to_dev(inp)
    banner(f"T={T}: GPU fwd+bwd")
    y, saved = mlp.fwd(g["X"], g["Wg"], g["Wu"], g["Wd"])
    first_past = (1 << 31) // (H * 2) + 1  # first row starting past 2 GiB in a plane
    rows = np.array([0, 255, first_past - 1, first_past, first_past + 300, T - 257, T - 1])
    G_s, U_s, A_s = (saved[i][rows].clone() for i in (1, 2, 0))
    dx, dwg, dwu, dwd = mlp.bwd(g["dY"], g["X"], g["Wg"], g["Wu"], g["Wd"], saved)
    dG_s, dU_s = saved[1][rows].clone(), saved[2][rows].clone()
    torch.cuda.synchronize()
    del g, saved
    f = _np(inp)
    banner(f"T={T}: oracle rows and hidden units")
    r = O.rows(rows, f["X"], f["Wg"], f["Wu"], f["Wd"], f["dY"])
    a_ref = O.round_to(O.epilogue_fwd(f64(G_s), f64(U_s)), "bf16")
    assert int(O.ulp_distance(f64(A_s), a_ref, "bf16").max()) <= 1
    got = {"Y": y[rows], "dI": dx[rows], "G": G_s, "U": U_s, "dG": dG_s, "dU": dU_s}
    for k, v in got.items():
        _check_sampled(f"T={T} {k}", f64(v), r[k])
    hs = np.array([0, 4999, 11007])
    c = O.cols(hs, f["X"], f["Wg"], f["Wu"], f["Wd"], f["dY"])
    _check_sampled(f"T={T} dWg", f64(dwg[:, hs]).T, c["dWg"].T)
    _check_sampled(f"T={T} dWu", f64(dwu[:, hs]).T, c["dWu"].T)
    _check_sampled(f"T={T} dWd", f64(dwd[hs, :]), c["dWd"])


@pytest.mark.parametrize("D,H", [(1024, 2816), (4096, 11008)])
def test_no_grad_path(mlp, D, H):
    wts = make_inputs(1, D, H, seed=2024 + D, dtype="bf16", with_dy=False)
    Wg, Wu, Wd = (wts[k].cuda() for k in ("Wg", "Wu", "Wd"))
    f = {k: wts[k].float().numpy() for k in ("Wg", "Wu", "Wd")}
    for S in (1, 2, 4, 8, 16, 32, 64, 128, 256, 300):
        X = make_inputs(S, D, H, seed=S, dtype="bf16", with_dy=False)["X"]
        y = mlp.infer(X.cuda(), Wg, Wu, Wd)
        y_train, _ = mlp.fwd(X.cuda(), Wg, Wu, Wd)
        torch.cuda.synchronize()
        e = assert_local(f64(y), O.infer(X.float().numpy(), f["Wg"], f["Wu"], f["Wd"]), 1e-2, ("infer", D, S))
        banner(f"infer D={D} S={S}: {fmt_local(e)}")
        if S > 256:
            # same tiles, same order: the no-grad Y equals the training Y bitwise
            assert torch.equal(y, y_train)
        else:
            # weight streaming (fixed split and summation order):
            # deterministic, and the training forward agrees within the bound
            assert torch.equal(mlp.infer(X.cuda(), Wg, Wu, Wd), y)
            assert nl2(f64(y), f64(y_train)) <= 1e-2


@pytest.mark.parametrize("T,D,H", [(1, 136, 200), (17, 264, 520), (40, 200, 136), (64, 520, 264),
                                   (3, 64, 64), (33, 1032, 2824), (65, 264, 520), (100, 1032, 2824),
                                   (128, 200, 136), (129, 264, 520), (200, 1032, 2824), (255, 520, 264),
                                   (256, 136, 200)])
def test_no_grad_split_k_ragged(mlp, T, D, H):
    """The no-grad weight-streaming kernels (bf16, T <= 256: per-wave rings
    up to 32 tokens, the workgroup-shared ring above, split K in the down
    projection up to 128 tokens) at K not a multiple of 32, N not a multiple
    of 64 and ragged token tiles."""
    inp = make_inputs(T, D, H, seed=T * 7 + D, dtype="bf16", with_dy=False)
    g = to_dev(inp)
    y = mlp.infer(g["X"], g["Wg"], g["Wu"], g["Wd"])
    torch.cuda.synchronize()
    f = _np(inp)
    e = assert_local(f64(y), O.infer(f["X"], f["Wg"], f["Wu"], f["Wd"]), 1e-2, ("split-K infer", T, D, H))
    banner(f"split-K infer T={T} D={D} H={H}: {fmt_local(e)}")
    assert torch.isfinite(y).all()


def test_zero_tokens(mlp):
    inp = make_inputs(0, 64, 128, seed=1, dtype="bf16")
    g = to_dev(inp)
    y, saved = mlp.fwd(g["X"], g["Wg"], g["Wu"], g["Wd"])
    assert y.shape == (0, 64) and saved.numel() == 0
    dwg = torch.full((64, 128), 7.0, dtype=torch.bfloat16, device="cuda")
    dwu = dwg.clone()
    dwd = torch.full((128, 64), 7.0, dtype=torch.bfloat16, device="cuda")
    dx, dwg, dwu, dwd = mlp.bwd(g["dY"], g["X"], g["Wg"], g["Wu"], g["Wd"], saved,
                                dwg=dwg, dwu=dwu, dwd=dwd)
    torch.cuda.synchronize()
    assert dx.shape == (0, 64)
    assert not dwg.any() and not dwu.any() and not dwd.any()
    assert mlp.infer(g["X"], g["Wg"], g["Wu"], g["Wd"]).shape == (0, 64)


@pytest.mark.parametrize("D,H", [(1024, 2816), (4096, 11008)])
def test_no_grad_workspace_contents_do_not_matter(mlp, D, H):
    """The no-grad workspace holds the down projection's arrival counters and
    partials; its contents on entry must not matter (the gate/up launch
    clears the counters). A workspace filled with 0xFF bytes, and one reused
    across shapes and splits, give the same bits as a fresh one."""
    wts = make_inputs(1, D, H, seed=5150 + D, dtype="bf16", with_dy=False)
    Wg, Wu, Wd = (wts[k].cuda() for k in ("Wg", "Wu", "Wd"))
    big = torch.empty(mlp.infer_workspace_bytes(128, D, H), dtype=torch.uint8, device="cuda")
    for S in (128, 7, 64, 1, 100):
        X = make_inputs(S, D, H, seed=S + 11, dtype="bf16", with_dy=False)["X"].cuda()
        n = mlp.infer_workspace_bytes(S, D, H)
        fresh = torch.zeros(n, dtype=torch.uint8, device="cuda")
        y0 = mlp.infer(X, Wg, Wu, Wd, workspace=fresh)
        junk = torch.full((n,), 0xFF, dtype=torch.uint8, device="cuda")
        y1 = mlp.infer(X, Wg, Wu, Wd, workspace=junk)
        y2 = mlp.infer(X, Wg, Wu, Wd, workspace=big[:n])  # reused from the previous shape
        torch.cuda.synchronize()
        banner(f"workspace contents D={D} S={S}")
        assert torch.equal(y0, y1) and torch.equal(y0, y2), (D, S)
