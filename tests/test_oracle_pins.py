"""Pins of the fp64 oracle to things other than itself.

Each test reduces the op to a closed form, a textbook/library routine, an
invariant of the mathematics, or exact arithmetic on a tiny case. Together
they are chosen so that a plausible mistake in the oracle fails at least one:

* eps outside the sqrt, or mean over d instead of n*d  -> constant/one-hot/tiny rows
* W transposed, or the wrong flattening k = c*n + i     -> one-hot state
* sigmoid sign, pre/post swapped                        -> gate test
* residual logits read column-major, H^T used in post   -> permutation logits
* no max subtraction                                    -> permutation logits at c = 800
* column pass before row pass, wrong iteration count    -> worked 2x2 example
* dropped bias / dropped post*layer_out term            -> zero row, affinity
"""
import math
import os
from decimal import Decimal, getcontext
from fractions import Fraction

import numpy as np
import pytest
import scipy.special
import torch

import oracle
from deepseek_v4_hyper_amd import workloads as wl

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rng(seed):
    return np.random.Generator(np.random.PCG64(seed))


def rand_case(seed, T, n, d, w_std=0.02):
    g = rng(seed)
    m = wl.n_logits(n)
    X = g.standard_normal((T, n, d))
    W = g.standard_normal((m, n * d)) * w_std
    b = g.standard_normal(m) * 0.3
    lo = g.standard_normal((T, d))
    return X, W, b, lo


def perm_matrix(p):
    n = len(p)
    P = np.zeros((n, n))
    P[np.arange(n), p] = 1.0
    return P


# ---------------------------------------------------------------- RMS norm + fn matvec

@pytest.mark.parametrize("c", [3.0, -0.25, 1e-4])
def test_constant_row_closed_form(c):
    n, d = 4, 16
    _, W, b, _ = rand_case(1, 1, n, d)
    X = np.full((1, n, d), c)
    _, _, z = oracle.pre(X, W, b, eps=1e-6)
    xn = c / math.sqrt(c * c + 1e-6)
    want = np.array([math.fsum(W[j]) * xn + b[j] for j in range(W.shape[0])])
    np.testing.assert_allclose(z[0], want, rtol=1e-12, atol=1e-14)


@pytest.mark.parametrize("n,d,i0,c0", [(4, 8, 2, 5), (2, 12, 1, 3), (4, 6, 0, 5)])
def test_one_hot_state(n, d, i0, c0):
    """Only X[i0][c0] = a is non-zero: r = sqrt(a^2/K + eps), z_j = W[j][i0*d+c0]*a/r + b_j,
    layer_in = pre_i0 * a at column c0 only."""
    a = 1.7
    _, W, b, lo = rand_case(2, 1, n, d)
    X = np.zeros((1, n, d))
    X[0, i0, c0] = a
    layer_in, coeffs, z = oracle.pre(X, W, b)
    r = math.sqrt(a * a / (n * d) + 1e-6)
    k0 = i0 * d + c0
    np.testing.assert_allclose(z[0], W[:, k0] * a / r + b, rtol=1e-13)
    want_li = np.zeros(d)
    want_li[c0] = coeffs[0, i0] * a
    np.testing.assert_allclose(layer_in[0], want_li, rtol=1e-15, atol=0)


def test_rms_and_matvec_match_library_routines():
    X, W, b, _ = rand_case(3, 5, 4, 32)
    _, _, z = oracle.pre(X, W, b, eps=1e-6)
    K = X.shape[1] * X.shape[2]
    xt = torch.from_numpy(X.reshape(5, K))
    xn = torch.nn.functional.rms_norm(xt, [K], eps=1e-6).numpy()
    np.testing.assert_allclose(z, xn @ W.T + b, rtol=1e-12, atol=1e-13)


def test_tiny_rows_see_eps():
    """Near-zero rows: the eps term dominates r; z scales linearly with the row."""
    n, d = 4, 8
    _, W, b, _ = rand_case(4, 1, n, d)
    b = np.zeros_like(b)
    X = rng(5).standard_normal((1, n, d)) * 1e-7
    _, _, z = oracle.pre(X, W, b)
    ss = math.fsum((X.ravel() ** 2).tolist())
    r = math.sqrt(ss / (n * d) + 1e-6)
    np.testing.assert_allclose(z[0], (W @ X.ravel()) / r, rtol=1e-12)
    assert abs(r - 1e-3) < 1e-9


def test_scale_invariance():
    X, W, b, _ = rand_case(6, 3, 4, 32)
    _, c1, _ = oracle.pre(X, W, b)
    _, c2, _ = oracle.pre(X * 1000.0, W, b)
    # relative effect of eps is <= eps / mean(x^2) ~ 1e-6
    np.testing.assert_allclose(c1, c2, atol=1e-6)


# ---------------------------------------------------------------- gates

def test_gates_are_logistic_of_first_2n_logits():
    n, d = 4, 8
    b = np.array([-3.0, -0.5, 0.0, 2.0, 1.0, -1.5, 4.0, 0.25] + [0.0] * 16)
    W = np.zeros((wl.n_logits(n), n * d))
    X = rng(7).standard_normal((2, n, d))
    _, coeffs, z = oracle.pre(X, W, b)
    np.testing.assert_array_equal(z, np.broadcast_to(b, z.shape))
    np.testing.assert_allclose(coeffs[:, :n], scipy.special.expit(b[:n])[None].repeat(2, 0), rtol=1e-15)
    np.testing.assert_allclose(coeffs[:, n:2 * n], scipy.special.expit(b[n:2 * n])[None].repeat(2, 0),
                               rtol=1e-15)
    assert coeffs[0, 2] == 0.5


# ---------------------------------------------------------------- Sinkhorn closed forms

def _perm_closed_form(P, c):
    n = P.shape[0]
    return ((math.expm1(c)) * P + np.ones((n, n))) / (math.exp(c) + n - 1)


@pytest.mark.parametrize("c", [0.0, 1.0, 5.0, 40.0])
@pytest.mark.parametrize("iters", [1, 3, 20])
def test_permutation_logits_closed_form(c, iters):
    P = perm_matrix([1, 2, 3, 0])           # a 4-cycle: P != P^T
    H = oracle.sinkhorn((c * P)[None], iters)[0]
    np.testing.assert_allclose(H, _perm_closed_form(P, c), rtol=1e-13, atol=1e-300)


def test_permutation_logits_need_max_subtraction():
    """exp(800) overflows double; with per-row max subtraction the result is the closed form."""
    P = perm_matrix([2, 0, 3, 1])
    H = oracle.sinkhorn((800.0 * P)[None], 20)[0]
    assert np.all(np.isfinite(H))
    np.testing.assert_array_equal(H, P)     # e^-800 underflows to 0 next to 1


def test_residual_layout_and_post_orientation():
    """Residual logits are row-major (i = output stream); X'[i] = sum_j H[i][j] X[j] + post_i*lo."""
    n, d, c = 4, 6, 3.0
    p = [1, 2, 3, 0]
    P = perm_matrix(p)
    b = np.zeros(wl.n_logits(n))
    b[2 * n:] = (c * P).ravel()
    b[n:2 * n] = [0.1, -0.2, 0.3, -0.4]
    W = np.zeros((wl.n_logits(n), n * d))
    X = rng(8).standard_normal((1, n, d))
    lo = rng(9).standard_normal((1, d))
    _, coeffs, _ = oracle.pre(X, W, b)
    H = coeffs[0, 2 * n:].reshape(n, n)
    Hc = _perm_closed_form(P, c)
    np.testing.assert_allclose(H, Hc, rtol=1e-13)
    assert not np.allclose(Hc, Hc.T)
    out = oracle.post(X, coeffs, lo)
    post = scipy.special.expit(b[n:2 * n])
    want = np.einsum("ij,jc->ic", Hc, X[0]) + post[:, None] * lo[0][None, :]
    np.testing.assert_allclose(out[0], want, rtol=1e-12, atol=1e-14)


def test_worked_2x2_example_pins_order_and_count():
    rows = []
    with open(os.path.join(GOLDEN, "sinkhorn_2x2_worked.txt")) as f:
        for line in f:
            if line.strip() and not line.startswith("#"):
                rows.append(line.split())
    Z = np.array([[0.0, math.log(2.0)], [math.log(3.0), 0.0]])
    assert len(rows) == 2
    for r in rows:
        iters = int(r[0])
        want = np.array([float(Fraction(v)) for v in r[1:]]).reshape(2, 2)
        H = oracle.sinkhorn(Z[None], iters)[0]
        np.testing.assert_allclose(H, want, rtol=1e-14)


def test_additive_logits_give_uniform():
    g = rng(10)
    a, bb = g.standard_normal(4) * 3, g.standard_normal(4) * 3
    Z = a[:, None] + bb[None, :]
    for iters in (1, 20):
        H = oracle.sinkhorn(Z[None], iters)[0]
        np.testing.assert_allclose(H, np.full((4, 4), 0.25), rtol=1e-14)


def test_circulant_logits_give_row_softmax():
    v = np.array([0.3, -1.2, 2.0, 0.7])
    Z = np.stack([np.roll(v, i) for i in range(4)])
    for iters in (1, 5, 20):
        H = oracle.sinkhorn(Z[None], iters)[0]
        np.testing.assert_allclose(H, scipy.special.softmax(Z, axis=1), rtol=1e-13)


def test_zero_logits_and_iters_zero():
    H = oracle.sinkhorn(np.zeros((2, 4, 4)), 20)
    np.testing.assert_array_equal(H, np.full((2, 4, 4), 0.25))
    Z = rng(11).standard_normal((1, 4, 4))
    H0 = oracle.sinkhorn(Z, 0)[0]            # no normalisation: exp(Z - rowmax)
    np.testing.assert_allclose(H0, np.exp(Z[0] - Z[0].max(axis=1, keepdims=True)), rtol=1e-15)


def test_2x2_limit_formula():
    a, b, c, d = 2.0, 0.5, 1.5, 3.0
    Z = np.log(np.array([[a, b], [c, d]]))
    H = oracle.sinkhorn(Z[None], 200)[0]
    p = math.sqrt(a * d) / (math.sqrt(a * d) + math.sqrt(b * c))
    np.testing.assert_allclose(H, [[p, 1 - p], [1 - p, p]], rtol=1e-14)


def test_columns_exact_rows_converge():
    Z = rng(12).standard_normal((64, 4, 4))
    for iters in (1, 2, 20):
        H = oracle.sinkhorn(Z, iters)
        np.testing.assert_allclose(H.sum(axis=1), 1.0, atol=4e-16 * 4)
    H = oracle.sinkhorn(Z, 2000)          # Sinkhorn's theorem: doubly stochastic in the limit
    np.testing.assert_allclose(H.sum(axis=2), 1.0, atol=1e-12)
    np.testing.assert_allclose(H.sum(axis=1), 1.0, atol=1e-12)


# ---------------------------------------------------------------- whole-op invariants

def test_zero_state_row():
    n, d = 4, 16
    _, W, _, lo = rand_case(13, 1, n, d)
    b = np.zeros(wl.n_logits(n))
    X = np.zeros((1, n, d))
    li, coeffs, out = oracle.fused(X, W, b, lo)
    np.testing.assert_array_equal(li, 0.0)
    np.testing.assert_array_equal(coeffs[0, :2 * n], 0.5)
    np.testing.assert_array_equal(coeffs[0, 2 * n:], 0.25)
    np.testing.assert_array_equal(out[0], 0.5 * np.broadcast_to(lo[0], (n, d)))


def test_single_stream_is_identity_residual():
    X, W, b, lo = rand_case(14, 3, 1, 32)
    li, coeffs, out = oracle.fused(X, W, b, lo)
    pre, post, H = coeffs[:, 0], coeffs[:, 1], coeffs[:, 2]
    np.testing.assert_array_equal(H, 1.0)
    np.testing.assert_allclose(li, pre[:, None] * X[:, 0], rtol=1e-15)
    np.testing.assert_allclose(out[:, 0], X[:, 0] + post[:, None] * lo, rtol=1e-15)


def test_stream_permutation_equivariance():
    n, d = 4, 8
    X, W, b, lo = rand_case(15, 3, n, d, w_std=0.3)
    pi = np.array([2, 0, 3, 1])
    Xp = X[:, pi]
    Wb = W[:, :].reshape(W.shape[0], n, d)[:, pi].reshape(W.shape[0], n * d)
    Wp = np.concatenate([Wb[:n][pi], Wb[n:2 * n][pi],
                         Wb[2 * n:].reshape(n, n, -1)[pi][:, pi].reshape(n * n, -1)])
    bp = np.concatenate([b[:n][pi], b[n:2 * n][pi], b[2 * n:].reshape(n, n)[pi][:, pi].ravel()])
    li, c, out = oracle.fused(X, W, b, lo)
    lip, cp, outp = oracle.fused(Xp, Wp, bp, lo)
    np.testing.assert_allclose(lip, li, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(outp, out[:, pi], rtol=1e-12, atol=1e-12)
    H = c[:, 2 * n:].reshape(-1, n, n)
    Hp = cp[:, 2 * n:].reshape(-1, n, n)
    np.testing.assert_allclose(Hp, H[:, pi][:, :, pi], rtol=1e-12, atol=1e-15)


def test_affine_in_layer_out():
    X, W, b, lo = rand_case(16, 2, 4, 8)
    lo2 = rng(17).standard_normal(lo.shape)
    _, c, o1 = oracle.fused(X, W, b, lo)
    _, _, o2 = oracle.fused(X, W, b, lo + lo2)
    post = c[:, 4:8]
    np.testing.assert_allclose(o2 - o1, post[:, :, None] * lo2[:, None, :], rtol=1e-12, atol=1e-14)


def test_nan_stays_in_its_token():
    X, W, b, lo = rand_case(18, 3, 4, 8)
    X[1, 2, 3] = np.nan
    li, c, out = oracle.fused(X, W, b, lo)
    assert np.all(np.isnan(li[1])) and np.all(np.isnan(out[1])) and np.all(np.isnan(c[1]))
    Xc = X.copy()
    Xc[1] = 0
    li2, c2, out2 = oracle.fused(Xc, W, b, lo)
    for t in (0, 2):
        np.testing.assert_array_equal(li[t], li2[t])
        np.testing.assert_array_equal(out[t], out2[t])


# ---------------------------------------------------------------- split-over-d partial sums

def _share(X, W, g, G):
    T, n, d = X.shape
    ds = d // G
    Xs = X[:, :, g * ds:(g + 1) * ds]
    Ws = W.reshape(W.shape[0], n, d)[:, :, g * ds:(g + 1) * ds].reshape(W.shape[0], n * ds)
    return np.ascontiguousarray(Xs), np.ascontiguousarray(Ws)


def test_partials_give_the_pre_logits():
    """The unnormalised dots over 1/r plus the bias are HC-pre's logits, with r
    from the sum of squares (r is one number per token)."""
    X, W, b, _ = rand_case(31, 9, 4, 24)
    m, K, eps = wl.n_logits(4), 4 * 24, 1e-6
    P = oracle.partials(X, W)
    r = np.sqrt(P[:, m] / K + eps)
    z = P[:, :m] / r[:, None] + b
    _, _, logits = oracle.pre(X, W, b, eps=eps)
    np.testing.assert_allclose(z, logits, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(P[:, m], (X.reshape(9, K) ** 2).sum(axis=1), rtol=1e-13)


@pytest.mark.parametrize("n,d,i0,c0", [(4, 8, 2, 5), (2, 12, 1, 3)])
def test_partials_of_one_hot_state(n, d, i0, c0):
    """x = c at stream i0, column c0: the dots are c times W's column i0*d + c0
    and the sum of squares is c^2, exactly (pins W's orientation and the
    flattening k = i*d + c)."""
    m = wl.n_logits(n)
    W = rng(5).standard_normal((m, n * d))
    X = np.zeros((1, n, d))
    X[0, i0, c0] = 2.5
    P = oracle.partials(X, W)
    np.testing.assert_array_equal(P[0, :m], 2.5 * W[:, i0 * d + c0])
    assert P[0, m] == 6.25


@pytest.mark.parametrize("G", [2, 3])
def test_partials_add_over_column_shares(G):
    """Each stream's columns split into G shares: the shares' partial sums add up
    to the whole row's."""
    X, W, b, _ = rand_case(32, 7, 4, 24)
    whole = oracle.partials(X, W)
    parts = sum(oracle.partials(*_share(X, W, g, G)) for g in range(G))
    np.testing.assert_allclose(parts, whole, rtol=1e-12, atol=1e-12)


def test_thread_count_does_not_change_bits():
    X, W, b, lo = rand_case(19, 37, 4, 16)
    nt = oracle.num_threads()
    try:
        oracle.set_threads(1)
        a = oracle.fused(X, W, b, lo)
        oracle.set_threads(4)
        b2 = oracle.fused(X, W, b, lo)
    finally:
        oracle.set_threads(nt)
    for u, v in zip(a, b2):
        np.testing.assert_array_equal(u, v)


def test_chain_with_zero_weights_closed_form():
    """W = 0, b = 0: pre = post = 1/2, H = J/n, so X_{l+1}[i] = mean_j X_l[j] + (S/4 + noise)/2
    with S = sum_j X_l[j] (layer_in = S/2, layer_out = layer_in/2 + noise)."""
    n, d = 4, 8
    X0 = rng(20).standard_normal((1, n, d))
    Ws = [np.zeros((wl.n_logits(n), n * d))] * 3
    noise = rng(21).standard_normal((3, d))
    states = oracle.chain(X0, Ws, np.zeros(wl.n_logits(n)), noise)
    X = X0[0]
    for l in range(3):
        S = X.sum(axis=0)
        X = np.broadcast_to(S / n + 0.5 * (0.25 * S + noise[l]), (n, d))
        np.testing.assert_allclose(states[l + 1][0], X, rtol=1e-13, atol=1e-13)


# ---------------------------------------------------------------- exact brute force

def _decimal_op(X, W, b, lo, eps, iters):
    """Whole op on a tiny case in 50-digit decimal arithmetic (stdlib exp/sqrt)."""
    getcontext().prec = 50
    D = Decimal
    n, d = len(X), len(X[0])
    K, m = n * d, 2 * n + n * n
    x = [D(float(X[i][c])) for i in range(n) for c in range(d)]
    r = (sum(v * v for v in x) / K + D(eps)).sqrt()
    z = [sum(D(float(W[j][k])) * (x[k] / r) for k in range(K)) + D(float(b[j])) for j in range(m)]
    sig = [1 / (1 + (-v).exp()) for v in z]
    Z = [[z[2 * n + i * n + j] for j in range(n)] for i in range(n)]
    M = [[(Z[i][j] - max(Z[i])).exp() for j in range(n)] for i in range(n)]
    for _ in range(iters):
        for i in range(n):
            s = sum(M[i])
            M[i] = [v / s for v in M[i]]
        for j in range(n):
            s = sum(M[i][j] for i in range(n))
            for i in range(n):
                M[i][j] = M[i][j] / s
    li = [sum(sig[i] * D(float(X[i][c])) for i in range(n)) for c in range(d)]
    out = [[sum(M[i][j] * D(float(X[j][c])) for j in range(n)) + sig[n + i] * D(float(lo[c]))
            for c in range(d)] for i in range(n)]
    coeffs = sig[:2 * n] + [M[i][j] for i in range(n) for j in range(n)]
    return li, coeffs, out


@pytest.mark.parametrize("n,d,iters", [(2, 2, 3), (2, 3, 20), (1, 4, 5)])
def test_decimal_brute_force(n, d, iters):
    X, W, b, lo = rand_case(22 + n + d, 1, n, d, w_std=0.8)
    li, c, out = oracle.fused(X, W, b, lo, iters=iters)
    dli, dc, dout = _decimal_op(X[0], W, b, lo[0], 1e-6, iters)
    np.testing.assert_allclose(li[0], [float(v) for v in dli], rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(c[0], [float(v) for v in dc], rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(out[0], [[float(v) for v in row] for row in dout], rtol=1e-13,
                               atol=1e-15)


def test_golden_single_workload_regression():
    """Values written by tests/golden/make_golden.py (calls only the oracle) for the
    single-token workload; catches any later drift of the oracle's arithmetic."""
    path = os.path.join(GOLDEN, "oracle_single_seed0.txt")
    want = np.loadtxt(path)
    case = wl.make_single(0)
    li, c, out = oracle.fused(wl.state_to_f64(case.X, case.dtype), case.W, case.bias,
                              wl.state_to_f64(case.layer_out, case.dtype), case.eps, case.iters)
    _, _, z = oracle.pre(wl.state_to_f64(case.X, case.dtype), case.W, case.bias)
    got = np.concatenate([z[0], c[0], li[0, :8], out[0, :, :8].ravel()])
    np.testing.assert_allclose(got, want, rtol=1e-14, atol=1e-15)
