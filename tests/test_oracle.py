"""Pins for the fp64 oracle (CPU only).

Each test checks the oracle against something other than itself: high
precision closed forms, finite differences, identities that follow from the
structure of the MLP, special cases with known answers, brute-force loops,
and the numbers the pages print. A plausible slip in the oracle (a dropped
term, a sign, a transposed operand, a wrong index) fails at least one of them.
"""

import math
from decimal import Decimal, getcontext

import numpy as np
import pytest
from scipy.optimize import brentq

import oracle as O

GOLDEN = __import__("os").path.join(__import__("os").path.dirname(__file__), "golden")


def _rand(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


def _small(T, D, H, seed=0):
    X = _rand((T, D), seed)
    Wg = _rand((D, H), seed + 1, 1 / math.sqrt(D))
    Wu = _rand((D, H), seed + 2, 1 / math.sqrt(D))
    Wd = _rand((H, D), seed + 3, 1 / math.sqrt(H))
    dY = _rand((T, D), seed + 4)
    return X, Wg, Wu, Wd, dY


def _rel(a, b):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    return np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300)


# --------------------------------------------------------------------------
# sigmoid / SiLU / SiLU'
# --------------------------------------------------------------------------

def _dec_silu(g):
    getcontext().prec = 50
    G = Decimal(repr(float(g)))
    s = 1 / (1 + (-G).exp())
    return float(G * s), float(s * (1 + G * (1 - s)))


@pytest.mark.parametrize("g", [-30.0, -7.5, -1.0, -0.5, -1e-3, 0.0, 1e-3, 0.5, 1.0, 2.0, 7.5, 30.0])
def test_silu_against_50_digit_closed_form(g):
    s_ref, ds_ref = _dec_silu(g)
    s = O.silu(np.array([g]))[0]
    ds = O.silu_prime(np.array([g]))[0]
    assert s == pytest.approx(s_ref, rel=1e-14, abs=1e-300)
    assert ds == pytest.approx(ds_ref, rel=1e-14, abs=1e-300)


def test_silu_prime_matches_central_differences():
    g = np.linspace(-30, 30, 6001)
    h = 1e-5
    fd = (O.silu(g + h) - O.silu(g - h)) / (2 * h)
    assert np.max(np.abs(fd - O.silu_prime(g))) < 1e-9
    fd_s = (O.sigmoid(g + h) - O.sigmoid(g - h)) / (2 * h)
    s = O.sigmoid(g)
    assert np.max(np.abs(fd_s - s * (1 - s))) < 1e-9


def test_silu_special_values_and_symmetries():
    assert O.silu(np.array([0.0]))[0] == 0.0
    assert O.silu_prime(np.array([0.0]))[0] == 0.5
    g = np.linspace(-40, 40, 4001)
    # SiLU(g) - SiLU(-g) = g  and  SiLU'(g) + SiLU'(-g) = 1
    assert np.max(np.abs(O.silu(g) - O.silu(-g) - g)) < 1e-12
    assert np.max(np.abs(O.silu_prime(g) + O.silu_prime(-g) - 1.0)) < 1e-14
    # asymptotes
    assert O.silu(np.array([60.0]))[0] == pytest.approx(60.0, rel=1e-15)
    assert -1e-20 < O.silu(np.array([-60.0]))[0] < 0.0


def test_silu_stationary_point():
    # SiLU' = 0 at g*: s(1 + g(1-s)) = 0  =>  g*s = 1 + g  =>  SiLU(g*) = g* + 1
    gs = brentq(lambda z: O.silu_prime(np.array([z]))[0], -2.0, -1.0, xtol=1e-15)
    assert gs == pytest.approx(-1.278464542761074, abs=1e-12)
    assert O.silu(np.array([gs]))[0] == pytest.approx(gs + 1.0, abs=1e-12)


def test_extreme_arguments_do_not_overflow():
    with np.errstate(over="raise", invalid="raise", divide="raise", under="ignore"):
        g = np.array([-1000.0, -745.0, -80.0, 80.0, 745.0, 1000.0])
        s = O.sigmoid(g)
        assert s[0] == 0.0 and s[-1] == 1.0
        assert np.all(np.isfinite(O.silu(g)))
        assert np.all(np.isfinite(O.silu_prime(g)))


# --------------------------------------------------------------------------
# forward / backward against brute force, FD, closed forms, identities
# --------------------------------------------------------------------------

@pytest.mark.parametrize("T,D,H", [(3, 4, 5), (2, 3, 7), (5, 8, 6), (1, 1, 1), (4, 2, 9)])
def test_fwd_bwd_match_brute_force_loops(T, D, H):
    X, Wg, Wu, Wd, dY = _small(T, D, H, seed=T * 100 + D * 10 + H)
    Y = O.fwd(X, Wg, Wu, Wd)["Y"]
    assert _rel(Y, O.fwd_naive(X, Wg, Wu, Wd)) < 1e-13
    b = O.bwd(dY, X, Wg, Wu, Wd)
    n = O.bwd_naive(dY, X, Wg, Wu, Wd)
    for k in ("dI", "dWg", "dWu", "dWd"):
        assert _rel(b[k], n[k]) < 1e-13, k


@pytest.mark.parametrize("T,D,H", [(3, 4, 5), (2, 3, 7)])
def test_bwd_matches_finite_differences_of_loss(T, D, H):
    X, Wg, Wu, Wd, dY = _small(T, D, H, seed=7)
    params = {"X": X, "Wg": Wg, "Wu": Wu, "Wd": Wd}
    grads = O.bwd(dY, X, Wg, Wu, Wd)
    name_to_grad = {"X": "dI", "Wg": "dWg", "Wu": "dWu", "Wd": "dWd"}

    def loss(p):
        return float(np.sum(dY * O.fwd(p["X"], p["Wg"], p["Wu"], p["Wd"])["Y"]))

    h = 1e-6
    for name, arr in params.items():
        fd = np.zeros_like(arr)
        for idx in np.ndindex(arr.shape):
            p_plus = {k: v.copy() for k, v in params.items()}
            p_minus = {k: v.copy() for k, v in params.items()}
            p_plus[name][idx] += h
            p_minus[name][idx] -= h
            fd[idx] = (loss(p_plus) - loss(p_minus)) / (2 * h)
        g = grads[name_to_grad[name]]
        assert np.max(np.abs(fd - g)) <= 1e-7 * max(1.0, np.max(np.abs(g))), name


def test_scalar_closed_form():
    x, wg, wu, wd, dy = 0.7, -1.3, 0.9, 1.7, -0.6
    g, u = x * wg, x * wu
    s = 1 / (1 + math.exp(-g))
    silu, dsilu = g * s, s + g * s * (1 - s)
    y = silu * u * wd
    # hand-derived partials of y = SiLU(x wg) (x wu) wd
    d_wd = silu * u
    d_wu = silu * x * wd
    d_wg = dsilu * x * u * wd
    d_x = dsilu * wg * u * wd + silu * wu * wd
    a = lambda v: np.array([[v]])
    assert O.fwd(a(x), a(wg), a(wu), a(wd))["Y"][0, 0] == pytest.approx(y, rel=1e-15)
    b = O.bwd(a(dy), a(x), a(wg), a(wu), a(wd))
    assert b["dWd"][0, 0] == pytest.approx(dy * d_wd, rel=1e-14)
    assert b["dWu"][0, 0] == pytest.approx(dy * d_wu, rel=1e-14)
    assert b["dWg"][0, 0] == pytest.approx(dy * d_wg, rel=1e-14)
    assert b["dI"][0, 0] == pytest.approx(dy * d_x, rel=1e-14)


def test_homogeneity_identities():
    # Y is linear in Wd and in Wu, so <dWd,Wd> = <dWu,Wu> = <dY,Y>.
    # G is linear in Wg: <dWg,Wg> = <dG,G>; G and U are linear in X:
    # <dI,X> = <dG,G> + <dU,U> = <dWg,Wg> + <dWu,Wu>.
    X, Wg, Wu, Wd, dY = _small(64, 32, 48, seed=3)
    b = O.bwd(dY, X, Wg, Wu, Wd, keep=True)
    ip = lambda a, c: float(np.sum(a * c))
    yy = ip(dY, b["Y"])
    assert ip(b["dWd"], Wd) == pytest.approx(yy, rel=1e-12)
    assert ip(b["dWu"], Wu) == pytest.approx(yy, rel=1e-12)
    assert ip(b["dWg"], Wg) == pytest.approx(ip(b["dG"], b["G"]), rel=1e-12)
    assert ip(b["dI"], X) == pytest.approx(ip(b["dWg"], Wg) + ip(b["dWu"], Wu), rel=1e-12)


def test_linearity_in_dY_and_row_permutation():
    X, Wg, Wu, Wd, dY = _small(16, 8, 12, seed=5)
    dY2 = _rand(dY.shape, 99)
    b1 = O.bwd(dY, X, Wg, Wu, Wd)
    b2 = O.bwd(dY2, X, Wg, Wu, Wd)
    b12 = O.bwd(2.0 * dY - 3.0 * dY2, X, Wg, Wu, Wd)
    for k in b1:
        assert _rel(b12[k], 2.0 * b1[k] - 3.0 * b2[k]) < 1e-13
    perm = np.random.default_rng(1).permutation(16)
    bp = O.bwd(dY[perm], X[perm], Wg, Wu, Wd)
    assert _rel(bp["dI"], b1["dI"][perm]) < 1e-14
    assert _rel(O.fwd(X[perm], Wg, Wu, Wd)["Y"], O.fwd(X, Wg, Wu, Wd)["Y"][perm]) < 1e-14
    for k in ("dWg", "dWu", "dWd"):
        assert _rel(bp[k], b1[k]) < 1e-13


def test_zero_gate_weight_closed_form():
    # Wg = 0: G = 0, SiLU(0) = 0, SiLU'(0) = 1/2 => A = 0, Y = 0, dWd = 0,
    # dU = 0 => dWu = 0, dG = dA*U/2 => dWg = X^T (dA*U)/2, dI = dG Wg^T + dU Wu^T = 0.
    X, Wg, Wu, Wd, dY = _small(6, 4, 5, seed=11)
    Wg = np.zeros_like(Wg)
    f = O.fwd(X, Wg, Wu, Wd)
    b = O.bwd(dY, X, Wg, Wu, Wd)
    assert np.all(f["Y"] == 0)
    assert np.all(b["dWd"] == 0) and np.all(b["dWu"] == 0) and np.all(b["dI"] == 0)
    U = X @ Wu
    dA = dY @ Wd.T
    assert _rel(b["dWg"], 0.5 * X.T @ (dA * U)) < 1e-14


def test_one_hot_input_reproduces_weights():
    # X = I (T = D): G = Wg, U = Wu exactly, Y = (SiLU(Wg) * Wu) @ Wd.
    D, H = 6, 5
    _, Wg, Wu, Wd, _ = _small(D, D, H, seed=13)
    f = O.fwd(np.eye(D), Wg, Wu, Wd, keep=True)
    assert np.array_equal(f["G"], Wg) and np.array_equal(f["U"], Wu)
    s = 1 / (1 + np.exp(-Wg))
    assert _rel(f["Y"], (Wg * s * Wu) @ Wd) < 1e-14


def test_identity_down_projection_passes_dY_through():
    # Wd = I (H = D): Y = A and dA = dY exactly.
    T, D = 7, 6
    X, Wg, Wu, _, dY = _small(T, D, D, seed=17)
    b = O.bwd(dY, X, Wg, Wu, np.eye(D), keep=True)
    assert np.array_equal(b["dA"], dY)
    assert np.array_equal(b["Y"], b["A"])


def test_blocking_over_rows_changes_nothing():
    X, Wg, Wu, Wd, dY = _small(37, 8, 12, seed=19)
    a = O.bwd(dY, X, Wg, Wu, Wd, chunk=4096)
    c = O.bwd(dY, X, Wg, Wu, Wd, chunk=5)
    for k in a:
        assert _rel(c[k], a[k]) < 1e-14
    assert _rel(O.fwd(X, Wg, Wu, Wd, chunk=3)["Y"], O.fwd(X, Wg, Wu, Wd)["Y"]) < 1e-15
    assert np.array_equal(O.infer(X, Wg, Wu, Wd), O.fwd(X, Wg, Wu, Wd)["Y"])


def test_rows_and_cols_match_full_oracle():
    X, Wg, Wu, Wd, dY = _small(40, 16, 24, seed=23)
    full = O.bwd(dY, X, Wg, Wu, Wd, keep=True)
    r = O.rows([0, 7, 39], X, Wg, Wu, Wd, dY)
    assert _rel(r["Y"], full["Y"][[0, 7, 39]]) < 1e-14
    assert _rel(r["dI"], full["dI"][[0, 7, 39]]) < 1e-14
    hs = [0, 5, 23]
    c = O.cols(hs, X, Wg, Wu, Wd, dY, chunk=9)
    assert _rel(c["dWg"], full["dWg"][:, hs]) < 1e-13
    assert _rel(c["dWu"], full["dWu"][:, hs]) < 1e-13
    assert _rel(c["dWd"], full["dWd"][hs, :]) < 1e-13


def test_epilogues_match_forward_and_backward():
    X, Wg, Wu, Wd, dY = _small(9, 8, 10, seed=29)
    b = O.bwd(dY, X, Wg, Wu, Wd, keep=True)
    assert _rel(O.epilogue_fwd(b["G"], b["U"]), b["A"]) < 1e-15
    dG, dU = O.epilogue_bwd(b["dA"], b["G"], b["U"])
    assert _rel(dG, b["dG"]) < 1e-15 and _rel(dU, b["dU"]) < 1e-15
    # closed form at one point: g=1, u=2, dA=3
    s = 1 / (1 + math.e ** -1)
    dg, du = O.epilogue_bwd(np.array([3.0]), np.array([1.0]), np.array([2.0]))
    assert du[0] == pytest.approx(3 * s, rel=1e-15)
    assert dg[0] == pytest.approx(3 * 2 * (s + s * (1 - s)), rel=1e-15)


# --------------------------------------------------------------------------
# rounding and ulp helpers
# --------------------------------------------------------------------------

def test_round_to_ties_and_overflow_by_hand():
    r = O.round_to
    # bf16: 7 fraction bits; 1 + 2^-8 is a tie between 1 and 1 + 2^-7 -> even (1.0)
    assert r(np.array([1 + 2**-8]), "bf16")[0] == 1.0
    assert r(np.array([1 + 3 * 2**-8]), "bf16")[0] == 1 + 2**-6
    # just above the tie: direct rounding goes up (double rounding via fp32 would not)
    assert r(np.array([1 + 2**-8 + 2**-30]), "bf16")[0] == 1 + 2**-7
    assert r(np.array([3.4e38]), "bf16")[0] == np.inf
    assert r(np.array([-3.4e38]), "bf16")[0] == -np.inf
    assert r(np.array([3.3895313892515355e38]), "bf16")[0] == 3.3895313892515355e38
    # fp16: max 65504; 65520 is the tie to 65536 (= overflow) -> inf
    assert r(np.array([65519.0]), "fp16")[0] == 65504.0
    assert r(np.array([65520.0]), "fp16")[0] == np.inf
    # fp16 subnormals: quantum 2^-24; 2^-25 is a tie -> 0; 3*2^-26 -> 2^-24
    assert r(np.array([2.0**-25]), "fp16")[0] == 0.0
    assert r(np.array([3 * 2.0**-26]), "fp16")[0] == 2.0**-24
    assert np.isnan(r(np.array([np.nan]), "bf16")[0])
    assert r(np.array([-0.0]), "bf16")[0] == 0.0


def test_round_to_agrees_with_single_rounding_libraries():
    import torch

    rng = np.random.default_rng(0)
    v = np.concatenate([rng.standard_normal(100000) * 10.0 ** rng.integers(-30, 30, 100000),
                        rng.standard_normal(1000) * 1e-40])
    f32 = v.astype(np.float32).astype(np.float64)   # fp32 values: one rounding to bf16
    ref = torch.from_numpy(f32).float().to(torch.bfloat16).double().numpy()
    assert np.array_equal(O.round_to(f32, "bf16"), ref)
    small = rng.standard_normal(100000) * 10.0 ** rng.integers(-8, 5, 100000)
    assert np.array_equal(O.round_to(small, "fp16"), small.astype(np.float16).astype(np.float64))
    assert np.array_equal(O.round_to(v, "fp32"), v.astype(np.float32).astype(np.float64))


def test_ulp_distance():
    d = O.ulp_distance
    assert d(np.array([0.0]), np.array([-0.0]), "bf16")[0] == 0
    assert d(np.array([1.0]), np.array([1 + 2**-7]), "bf16")[0] == 1
    assert d(np.array([1.0]), np.array([1 - 2**-8]), "bf16")[0] == 1
    assert d(np.array([2.0**-133]), np.array([-(2.0**-133)]), "bf16")[0] == 2
    assert d(np.array([1.0]), np.array([1 + 2**-10]), "fp16")[0] == 1
    assert d(np.array([-2.0]), np.array([-2.0 - 2**-6]), "bf16")[0] == 1


# --------------------------------------------------------------------------
# one-round versus two-round epilogue (xorl PR #51, review thread)
# --------------------------------------------------------------------------

def test_two_round_differs_from_one_round_by_hand():
    # g = 1, u = 1.125 (both bf16): SiLU(1) = 0.7310585786..., product 0.8224409...
    # one round: 0.8224409 / 2^-8 = 210.545 -> 211 * 2^-8 = 0.82421875
    # two rounds: SiLU -> 187 * 2^-8 = 0.73046875; * 1.125 = 0.82177734375 -> 210 * 2^-8
    g, u = np.array([1.0]), np.array([1.125])
    assert O.round_to(O.epilogue_fwd(g, u), "bf16")[0] == 0.82421875
    assert O.epilogue_fwd_two_round(g, u, "bf16")[0] == 0.8203125


def test_two_round_difference_rate_matches_pages():
    # The PR's review reports 27.44% of bf16 outputs differing between the two
    # programs (input distribution unstated); unit-normal bf16 gate/up give ~27.5%.
    rng = np.random.default_rng(0)
    G = O.round_to(rng.standard_normal(1 << 18), "bf16")
    U = O.round_to(rng.standard_normal(1 << 18), "bf16")
    rate = np.mean(O.round_to(O.epilogue_fwd(G, U), "bf16") != O.epilogue_fwd_two_round(G, U, "bf16"))
    assert 0.26 < rate < 0.29


# --------------------------------------------------------------------------
# the pages' printed numbers
# --------------------------------------------------------------------------

def _golden(name):
    rows = []
    with open(f"{GOLDEN}/{name}") as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append([float(v) for v in line.split()])
    return rows


def test_pages_tflops_are_18TDH_over_time():
    for D, H, B, S, ms, tf in _golden("training_timings.txt"):
        flops = 18.0 * B * S * D * H
        assert flops / (ms * 1e-3) / 1e12 == pytest.approx(tf, abs=0.051)
        # and the alternative 6*T*D*H (forward only) or 12*T*D*H would not match
        assert abs(12.0 * B * S * D * H / (ms * 1e-3) / 1e12 - tf) > 5


def test_pages_memory_figures_match_buffer_sizes():
    MiB = float(1 << 20)
    for D, H, S, mb in _golden("infer_memory.txt"):
        T = 1 * S
        assert round((T * H + T * D) * 2 / MiB, 1) == mb      # A + Y only
        assert round((3 * T * H + T * D) * 2 / MiB, 1) != mb  # not if G/U were kept
    for D, H, B, S, mb in _golden("train_memory.txt"):
        T = B * S
        assert (3 * T * H + 3 * T * D) * 2 / MiB == mb
