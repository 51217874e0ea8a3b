"""Plain fp64 definition of the SwiGLU MLP forward, backward and no-grad path.

Test infrastructure (see the package docstring): nothing in the product path
may import or call this module.

Notation follows "[RFC] Full-pipeline SwiGLU MLP with forward/backward
co-optimization" (Liger-Kernel issue #1347), section "Summary":

    G = X @ Wg,  U = X @ Wu,  A = SiLU(G) * U,  Y = A @ Wd          (forward)
    dA = dY @ Wd^T, dWd = A^T @ dY,
    dU = dA * SiLU(G), dG = dA * U * SiLU'(G),
    dWg = X^T @ dG, dWu = X^T @ dU, dI = dG @ Wg^T + dU @ Wu^T       (backward)

with X[T,D], Wg and Wu [D,H], Wd [H,D]. The output set (Y and the four
gradients dI, dWg, dWu, dWd) is the one the same page's section
"Correctness" checks. The no-grad path ("a dedicated no-grad path that does
not save G/U", section "Summary") computes the same Y.

Inputs may be any real numpy array (float32 holds bf16 and fp16 values
exactly); every function converts to float64 first, and nothing is rounded
in between. Long inputs are processed in blocks of rows; rows of Y and dI
depend only on the same row of X and dY, and the weight gradients are sums
over rows, so blocking changes nothing but the fp64 summation order.

Parity status: every function below is pinned by a test in
tests/test_oracle.py against something other than itself (finite
differences, closed forms, identities, special cases, brute-force loops);
see PARITY.
"""

import numpy as np

PARITY = {
    "sigmoid/silu/silu_prime": "pinned: central finite differences, SiLU(0)=0, "
    "SiLU'(0)=1/2, odd/even symmetries, stationary point g*=-1.27846 where SiLU(g*)=g*+1",
    "fwd": "pinned: brute-force loops, scalar closed form, Wg=0 and one-hot-X special cases",
    "bwd": "pinned: central finite differences of <dY,Y>, scalar closed form, "
    "Euler-homogeneity identities, Wg=0 closed form, brute-force loops",
    "infer": "pinned: equals fwd's Y (same definition)",
    "rows/cols": "pinned: equal the corresponding rows/columns of fwd/bwd at small sizes",
    "epilogue_fwd/epilogue_bwd": "pinned: closed forms at chosen points; consistent with fwd/bwd",
    "epilogue_fwd_two_round": "pinned: hand-computed bf16 example and the pages' "
    "reported difference rate versus one-round (about 27%)",
}


def _f64(a):
    return np.asarray(a, dtype=np.float64)


def sigmoid(g):
    """Logistic function 1/(1+exp(-g)), evaluated without overflow.

    For g >= 0 the textbook form is used; for g < 0 the algebraically equal
    exp(g)/(1+exp(g)), so that exp never sees a large positive argument.
    """
    g = _f64(g)
    out = np.empty_like(g)
    pos = g >= 0
    out[pos] = 1.0 / (1.0 + np.exp(-g[pos]))
    e = np.exp(g[~pos])
    out[~pos] = e / (1.0 + e)
    return out


def silu(g):
    """SiLU(g) = g * sigmoid(g)."""
    g = _f64(g)
    return g * sigmoid(g)


def silu_prime(g):
    """d/dg SiLU(g) = s * (1 + g * (1 - s)) with s = sigmoid(g)."""
    g = _f64(g)
    s = sigmoid(g)
    return s * (1.0 + g * (1.0 - s))


def _blocks(T, chunk):
    for t0 in range(0, T, chunk):
        yield t0, min(T, t0 + chunk)


def fwd(X, Wg, Wu, Wd, chunk=4096, keep=False):
    """Forward of the SwiGLU MLP in fp64.

    Returns a dict with Y[T,D]; with keep=True also G, U, A [T,H].
    """
    Wg, Wu, Wd = _f64(Wg), _f64(Wu), _f64(Wd)
    T = X.shape[0]
    D, H = Wg.shape
    Y = np.empty((T, D))
    if keep:
        G = np.empty((T, H))
        U = np.empty((T, H))
        A = np.empty((T, H))
    for t0, t1 in _blocks(T, chunk):
        x = _f64(X[t0:t1])
        g = x @ Wg
        u = x @ Wu
        a = silu(g) * u
        Y[t0:t1] = a @ Wd
        if keep:
            G[t0:t1], U[t0:t1], A[t0:t1] = g, u, a
    out = {"Y": Y}
    if keep:
        out.update(G=G, U=U, A=A)
    return out


def infer(X, Wg, Wu, Wd, chunk=4096):
    """No-grad path: the same Y as the forward, nothing else kept."""
    return fwd(X, Wg, Wu, Wd, chunk=chunk)["Y"]


def bwd(dY, X, Wg, Wu, Wd, chunk=4096, keep=False):
    """Full backward in fp64: dI[T,D], dWg[D,H], dWu[D,H], dWd[H,D].

    Recomputes the forward intermediates per block of rows. With keep=True
    also returns Y, G, U, A, dA, dG, dU for every row.
    """
    Wg, Wu, Wd = _f64(Wg), _f64(Wu), _f64(Wd)
    T = X.shape[0]
    D, H = Wg.shape
    dI = np.empty((T, D))
    dWg = np.zeros((D, H))
    dWu = np.zeros((D, H))
    dWd = np.zeros((H, D))
    kept = {k: [] for k in ("Y", "G", "U", "A", "dA", "dG", "dU")}
    for t0, t1 in _blocks(T, chunk):
        x = _f64(X[t0:t1])
        dy = _f64(dY[t0:t1])
        g = x @ Wg
        u = x @ Wu
        sg = silu(g)
        a = sg * u
        da = dy @ Wd.T
        du = da * sg
        dg = da * u * silu_prime(g)
        dWd += a.T @ dy
        dWg += x.T @ dg
        dWu += x.T @ du
        dI[t0:t1] = dg @ Wg.T + du @ Wu.T
        if keep:
            for k, v in (("Y", a @ Wd), ("G", g), ("U", u), ("A", a),
                         ("dA", da), ("dG", dg), ("dU", du)):
                kept[k].append(v)
    out = {"dI": dI, "dWg": dWg, "dWu": dWu, "dWd": dWd}
    if keep:
        for k, v in kept.items():
            out[k] = np.concatenate(v, axis=0) if v else np.zeros((0, H if k != "Y" else D))
    return out


def rows(idx, X, Wg, Wu, Wd, dY=None):
    """Y and dI restricted to the rows ``idx`` (exact per-row definition).

    Row t of Y depends only on row t of X; row t of dI only on rows t of X
    and dY. Used to check full-size runs on a sample of rows.
    """
    idx = np.asarray(idx)
    Wg, Wu, Wd = _f64(Wg), _f64(Wu), _f64(Wd)
    x = _f64(X[idx])
    g = x @ Wg
    u = x @ Wu
    sg = silu(g)
    a = sg * u
    out = {"Y": a @ Wd, "G": g, "U": u, "A": a}
    if dY is not None:
        dy = _f64(dY[idx])
        da = dy @ Wd.T
        du = da * sg
        dg = da * u * silu_prime(g)
        out.update(dI=dg @ Wg.T + du @ Wu.T, dG=dg, dU=du, dA=da)
    return out


def cols(hidx, X, Wg, Wu, Wd, dY, chunk=8192):
    """Weight-gradient slices for the hidden units ``hidx``.

    Column h of G, U, A, dA, dG, dU only needs column h of Wg and Wu and row
    h of Wd. Then dWg[:, h] = X^T dG[:, h], dWu[:, h] = X^T dU[:, h] and
    dWd[h, :] = A[:, h]^T dY. Returns dWg_cols [D,n], dWu_cols [D,n],
    dWd_rows [n,D] for n = len(hidx).
    """
    hidx = np.asarray(hidx)
    wg = _f64(Wg[:, hidx])
    wu = _f64(Wu[:, hidx])
    wd = _f64(Wd[hidx, :])
    T = X.shape[0]
    D = wg.shape[0]
    n = len(hidx)
    dWg = np.zeros((D, n))
    dWu = np.zeros((D, n))
    dWd = np.zeros((n, D))
    for t0, t1 in _blocks(T, chunk):
        x = _f64(X[t0:t1])
        dy = _f64(dY[t0:t1])
        g = x @ wg
        u = x @ wu
        sg = silu(g)
        a = sg * u
        da = dy @ wd.T
        du = da * sg
        dg = da * u * silu_prime(g)
        dWg += x.T @ dg
        dWu += x.T @ du
        dWd += a.T @ dy
    return {"dWg": dWg, "dWu": dWu, "dWd": dWd}


def epilogue_fwd(g, u):
    """A = SiLU(g) * u from given (stored) g and u, exact in fp64.

    The one-round program of "Scope one-round FP32 SwiGLU to the exact
    Qwen3.5 contract" (xorl PR #51, review thread) computes this in fp32 and
    rounds once to the output dtype; its correctly rounded value is
    ``round_to(epilogue_fwd(g, u), dtype)``.
    """
    return silu(g) * _f64(u)


def epilogue_fwd_two_round(g, u, dtype):
    """The historical two-round program of the same PR: SiLU(g) is rounded
    to the input dtype, then multiplied by u and rounded again."""
    from .rounding import round_to

    s = round_to(silu(g), dtype)
    return round_to(s * _f64(u), dtype)


def epilogue_bwd(dA, g, u):
    """dG = dA * u * SiLU'(g), dU = dA * SiLU(g) from the stored g, u (fp64)."""
    dA, u = _f64(dA), _f64(u)
    return dA * u * silu_prime(g), dA * silu(g)


# ---------------------------------------------------------------------------
# Brute-force versions: explicit loops, independent of the numpy forms above
# (they do not call silu/sigmoid either). Only for tiny shapes.
# ---------------------------------------------------------------------------

def _sig_scalar(z):
    import math

    if z >= 0:
        return 1.0 / (1.0 + math.exp(-z))
    e = math.exp(z)
    return e / (1.0 + e)


def fwd_naive(X, Wg, Wu, Wd):
    X, Wg, Wu, Wd = (np.asarray(v, dtype=np.float64).tolist() for v in (X, Wg, Wu, Wd))
    T, D, H = len(X), len(Wg), len(Wg[0]) if Wg else 0
    Y = [[0.0] * D for _ in range(T)]
    for t in range(T):
        a = []
        for h in range(H):
            g = sum(X[t][d] * Wg[d][h] for d in range(D))
            u = sum(X[t][d] * Wu[d][h] for d in range(D))
            a.append(g * _sig_scalar(g) * u)
        for d in range(D):
            Y[t][d] = sum(a[h] * Wd[h][d] for h in range(H))
    return np.array(Y, dtype=np.float64).reshape(T, D)


def bwd_naive(dY, X, Wg, Wu, Wd):
    """Reverse-mode by hand, one scalar at a time (chain rule written out)."""
    dY, X, Wg, Wu, Wd = (np.asarray(v, dtype=np.float64).tolist()
                         for v in (dY, X, Wg, Wu, Wd))
    T, D, H = len(X), len(Wg), len(Wg[0])
    dI = [[0.0] * D for _ in range(T)]
    dWg = [[0.0] * H for _ in range(D)]
    dWu = [[0.0] * H for _ in range(D)]
    dWd = [[0.0] * D for _ in range(H)]
    for t in range(T):
        for h in range(H):
            g = sum(X[t][d] * Wg[d][h] for d in range(D))
            u = sum(X[t][d] * Wu[d][h] for d in range(D))
            s = _sig_scalar(g)
            a = g * s * u
            # dL/da for this (t, h): Y[t][d] = sum_h a * Wd[h][d]
            da = sum(dY[t][d] * Wd[h][d] for d in range(D))
            for d in range(D):
                dWd[h][d] += a * dY[t][d]
            # a = g*s(g)*u: da/du = g*s ; da/dg = u*(s + g*s*(1-s))
            du = da * g * s
            dg = da * u * (s + g * s * (1.0 - s))
            for d in range(D):
                dWg[d][h] += X[t][d] * dg
                dWu[d][h] += X[t][d] * du
                dI[t][d] += dg * Wg[d][h] + du * Wu[d][h]
    f = lambda v: np.array(v, dtype=np.float64)
    return {"dI": f(dI), "dWg": f(dWg), "dWu": f(dWu), "dWd": f(dWd)}
