"""Pins of the float64 oracle against what the pages and the mathematics fix (CPU only).

Every check here is independent of the oracle's own code path: brute-force least squares,
directly summed weighted covariances, closed forms from eigen-decompositions and Chebyshev
polynomials, special cases with textbook answers, and the numbers printed on the pages.
"""
import os

import numpy as np
import pytest

from oracle import (agd_solve, cg_solve, gka_backward_ref, chebyshev_rates, chebyshev_solve, chebyshev_weights,
                    gd_solve, gka_forward_ref, gka_step_ref, ridge_bruteforce, solver_residuals)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand_inputs(rng, B, T, H, D, gate="sigmoid"):
    q = rng.standard_normal((B, T, H, D))
    k = rng.standard_normal((B, T, H, D))
    v = rng.standard_normal((B, T, H, D))
    q /= np.linalg.norm(q, axis=-1, keepdims=True)
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    if gate == "sigmoid":
        g = 1.0 / (1.0 + np.exp(-rng.normal(1.5, 1.0, (B, T, H))))
    elif gate == "with_zeros":
        g = 1.0 / (1.0 + np.exp(-rng.normal(1.5, 1.0, (B, T, H))))
        g[rng.random((B, T, H)) < 0.15] = 0.0
    elif gate == "ones":
        g = np.ones((B, T, H))
    else:
        raise ValueError(gate)
    return q, k, v, g


def _direct_states(k, v, g, t):
    """H_t and U_t for one head summed from eta_{t,i} = prod_{j=i+1}^t gamma_j (no recurrence)."""
    D = k.shape[-1]
    Ht = np.zeros((D, D))
    Ut = np.zeros((D, D))
    for i in range(t + 1):
        eta = np.prod(g[i + 1:t + 1])
        Ht += eta * np.outer(k[i], k[i])
        Ut += eta * np.outer(v[i], k[i])
    return Ht, Ut


def _cheb_T(r, x):
    return np.polynomial.chebyshev.chebval(x, [0.0] * r + [1.0])


def _rel(a, b):
    return np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300)


# ------------------------------------------------------------------------------------------
# 1. the objective: exact mode == brute-force weighted ridge regression
# ------------------------------------------------------------------------------------------

@pytest.mark.parametrize("gate", ["sigmoid", "with_zeros", "ones"])
@pytest.mark.parametrize("D", [1, 4, 16])
def test_exact_mode_matches_bruteforce_ridge(gate, D):
    rng = np.random.default_rng(100 + D)
    T, a = 40, 0.1
    q, k, v, g = _rand_inputs(rng, 1, T, 2, D, gate)
    ref = gka_forward_ref(q, k, v, g, a, iters=1, mode="exact")
    for h in range(2):
        o_bf, hn_bf = ridge_bruteforce(q[0, :, h], k[0, :, h], v[0, :, h], g[0, :, h], a)
        assert _rel(ref["o"][0, :, h], o_bf) < 1e-10
        np.testing.assert_allclose(ref["hnorm"][0, :, h], hn_bf, rtol=1e-12, atol=0)


def test_bruteforce_is_a_minimiser():
    """The brute-force S_t satisfies the normal equations of the weighted objective (sanity of the pin)."""
    rng = np.random.default_rng(7)
    T, D, a = 12, 5, 0.05
    q, k, v, g = _rand_inputs(rng, 1, T, 1, D)
    k0, v0, g0 = k[0, :, 0], v[0, :, 0], g[0, :, 0]
    t = T - 1
    Ht, Ut = _direct_states(k0, v0, g0, t)
    lam = a * np.linalg.norm(Ht)
    # objective f(S) = sum eta ||v - S k||^2 + lam ||S||^2 ; gradient at S* must vanish
    S = Ut @ np.linalg.inv(Ht + lam * np.eye(D))
    grad = -2 * sum(np.prod(g0[i + 1:t + 1]) * np.outer(v0[i] - S @ k0[i], k0[i]) for i in range(t + 1))
    grad += 2 * lam * S
    assert np.abs(grad).max() < 1e-10
    # and the same minimiser gives o_t = S q_t, which the brute force returns
    o_bf, _ = ridge_bruteforce(q[0, :, 0], k0, v0, g0, a)
    assert _rel(o_bf[t], S @ q[0, t, 0]) < 1e-10


# ------------------------------------------------------------------------------------------
# 2. the Frobenius-norm recurrence and the condition-number bound
# ------------------------------------------------------------------------------------------

@pytest.mark.parametrize("gate", ["sigmoid", "with_zeros"])
def test_norm_recurrence_equals_direct_norm(gate):
    rng = np.random.default_rng(11)
    T, D = 48, 8
    q, k, v, g = _rand_inputs(rng, 2, T, 1, D, gate)
    # a nonzero initial state: random PSD h0, any u0, carried n2 = ||h0||_F^2
    Z = rng.standard_normal((2, 1, D, 3 * D))
    h0 = Z @ np.swapaxes(Z, -1, -2) / D
    u0 = rng.standard_normal((2, 1, D, D))
    n20 = np.sum(h0 * h0, axis=(-1, -2))
    ref = gka_forward_ref(q, k, v, g, 0.1, 4, h0=h0, u0=u0, n2_0=n20)
    for b in range(2):
        Hd = h0[b, 0].copy()
        for t in range(T):
            Hd = g[b, t, 0] * Hd + np.outer(k[b, t, 0], k[b, t, 0])
            assert abs(ref["hnorm"][b, t, 0] - np.linalg.norm(Hd)) <= 1e-12 * np.linalg.norm(Hd)
        np.testing.assert_allclose(ref["h"][b, 0], Hd, rtol=0, atol=1e-12 * np.abs(Hd).max())


@pytest.mark.parametrize("a", [0.1, 0.05, 0.02])
def test_condition_number_bound(a):
    rng = np.random.default_rng(int(a * 1000))
    T, D = 32, 6
    q, k, v, g = _rand_inputs(rng, 1, T, 1, D, "with_zeros")
    ref = gka_forward_ref(q, k, v, g, a, 2)
    bound = (a + 1) / a
    for t in range(T):
        Ht, _ = _direct_states(k[0, :, 0], v[0, :, 0], g[0, :, 0], t)
        lam = a * ref["hnorm"][0, t, 0]
        ev = np.linalg.eigvalsh(Ht + lam * np.eye(D))
        assert ev.max() / ev.min() <= bound * (1 + 1e-12)
        # the interval [lam, lam + ||H||_F] used by the solver contains the spectrum
        assert ev.min() >= lam * (1 - 1e-12) and ev.max() <= (lam + ref["hnorm"][0, t, 0]) * (1 + 1e-12)


# ------------------------------------------------------------------------------------------
# 3. Chebyshev mode: closed form, error bound, weight schedule
# ------------------------------------------------------------------------------------------

@pytest.mark.parametrize("r", [1, 2, 3, 8, 10, 12])
def test_chebyshev_mode_matches_polynomial_closed_form(r):
    """x_r = x* - P_r(A) (x* - x_0), P_r(z) = T_r((L+mu-2z)/(L-mu)) / T_r((L+mu)/(L-mu)), x_0 = 0."""
    rng = np.random.default_rng(200 + r)
    T, D, a = 20, 7, 0.05
    q, k, v, g = _rand_inputs(rng, 1, T, 1, D)
    ref = gka_forward_ref(q, k, v, g, a, r)
    k0, v0, g0, q0 = k[0, :, 0], v[0, :, 0], g[0, :, 0], q[0, :, 0]
    for t in range(T):
        Ht, Ut = _direct_states(k0, v0, g0, t)
        n = np.linalg.norm(Ht)
        mu, L = a * n, a * n + n
        A = Ht + mu * np.eye(D)
        w, Q = np.linalg.eigh(A)
        xs = Q @ ((Q.T @ q0[t]) / w)
        P = _cheb_T(r, (L + mu - 2 * w) / (L - mu)) / _cheb_T(r, (L + mu) / (L - mu))
        xr = xs - Q @ (P * (Q.T @ xs))
        assert _rel(ref["o"][0, t, 0], Ut @ xr) < 1e-10


def test_chebyshev_converges_to_exact():
    rng = np.random.default_rng(5)
    q, k, v, g = _rand_inputs(rng, 1, 16, 2, 8)
    ex = gka_forward_ref(q, k, v, g, 0.1, 1, mode="exact")["o"]
    ch = gka_forward_ref(q, k, v, g, 0.1, 80)["o"]
    assert _rel(ch, ex) < 1e-12


@pytest.mark.parametrize("a,r", [(0.1, 8), (0.05, 10), (0.02, 12), (0.02, 3)])
def test_chebyshev_error_bound(a, r):
    """||x_r - x*||_A <= 2 R_a^r / (1 + R_a^{2r}) ||x*||_A for spectrum in [a, 1+a] (kappa=(1+a)/a)."""
    rng = np.random.default_rng(300 + r)
    D = 24
    kappa = (1 + a) / a
    _, ra = chebyshev_rates(kappa)
    bound = 2 * ra ** r / (1 + ra ** (2 * r))
    worst = 0.0
    for trial in range(20):
        Qm, _ = np.linalg.qr(rng.standard_normal((D, D)))
        ev = np.concatenate([[a, 1 + a], rng.uniform(a, 1 + a, D - 2)])
        A = (Qm * ev) @ Qm.T
        b = rng.standard_normal(D)
        xs = np.linalg.solve(A, b)
        xr = chebyshev_solve(A, b, np.array(a), np.array(1 + a), r)
        e = xr - xs
        ratio = np.sqrt(e @ A @ e) / np.sqrt(xs @ A @ xs)
        worst = max(worst, ratio)
        assert ratio <= bound * (1 + 1e-9)
    # the bound is attained in the worst case: equioscillation makes it tight for some rhs
    assert worst > 0.05 * bound


def test_chebyshev_residual_tracking():
    rng = np.random.default_rng(9)
    D, r = 10, 6
    A = np.diag(np.linspace(0.1, 1.1, D))
    b = rng.standard_normal(D)
    res = []
    x = chebyshev_solve(A, b, np.array(0.1), np.array(1.1), r, residuals=res)
    assert len(res) == r + 1
    assert abs(res[0] - np.linalg.norm(b)) < 1e-14
    assert abs(res[-1] - np.linalg.norm(b - A @ x)) < 1e-13


@pytest.mark.parametrize("kappa", [1.5, 11.0, 21.0, 51.0, 500.0])
def test_weight_schedule_lemmas(kappa):
    """Lemma 3: omega_i in [1, 2], non-increasing, above omega*_1; Lemma 4: rate R = rho R_a."""
    rho = (kappa - 1) / (kappa + 1)
    om = np.array([float(w) for w in chebyshev_weights(rho, 40)])
    ostar = 2.0 / (1.0 + np.sqrt(1.0 - rho * rho))
    R, _ = chebyshev_rates(kappa)
    assert om[0] == 2.0
    assert np.all(om >= 1.0) and np.all(om <= 2.0)
    assert np.all(np.diff(om) <= 1e-15)
    assert np.all(om - ostar >= -1e-15)  # strictly above in exact arithmetic; fp64 reaches it
    assert om[1] > ostar
    for i in range(40):
        assert om[i] - ostar <= R ** i * (om[0] - ostar) * (1 + 1e-12)
    # omega* is the fixed point of the update map
    assert abs(4.0 / (4.0 - rho * rho * ostar) - ostar) < 1e-14


def test_lemma4_printed_rates():
    """Reproduce every rate the pages print for kappa = 1.02/0.02 = 51, to the printed digits."""
    rows = []
    with open(os.path.join(GOLDEN, "lemma4_kappa51.txt")) as f:
        for line in f:
            if line.strip() and not line.startswith("#"):
                name, p, val, sig = line.split()
                rows.append((name, int(p), float(val), int(sig)))
    assert len(rows) == 10
    kappa = 1.02 / 0.02
    assert abs(kappa - 51.0) < 1e-12
    R, Ra = chebyshev_rates(kappa)
    for name, p, val, sig in rows:
        got = (R if name == "R" else Ra) ** p
        # the printed value is the computed one cut to `sig` significant digits (the pages round
        # most values and truncate R^30 = 6.5e-5 to 6e-5): within one unit of the last digit
        ulp = 10.0 ** (np.floor(np.log10(val)) - sig + 1)
        assert abs(got - val) < ulp, (name, p, got, val)


# ------------------------------------------------------------------------------------------
# 4. special cases with closed forms
# ------------------------------------------------------------------------------------------

@pytest.mark.parametrize("r", [1, 2, 5, 8, 10])
def test_gamma_zero_closed_form(r):
    """gamma = 0: H_t = k_t k_t^T, lambda = a||k||^2; o_t = (1 - (-1)^r / T_r(1+2a)) v_t k.q / ((1+a)||k||^2)."""
    rng = np.random.default_rng(400 + r)
    a = 0.05
    q, k, v, _ = _rand_inputs(rng, 2, 10, 3, 9)
    k *= rng.uniform(0.5, 2.0, k.shape[:-1])[..., None]  # non-unit keys too
    g = np.zeros(k.shape[:-1])
    ch = gka_forward_ref(q, k, v, g, a, r)["o"]
    ex = gka_forward_ref(q, k, v, g, a, r, mode="exact")["o"]
    kk = np.sum(k * k, -1)
    base = v * (np.sum(k * q, -1) / ((1 + a) * kk))[..., None]
    fac = 1 - (-1) ** r / _cheb_T(r, 1 + 2 * a)
    np.testing.assert_allclose(ex, base, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(ch, fac * base, rtol=1e-12, atol=1e-14)


@pytest.mark.parametrize("r", [1, 4, 9])
def test_scalar_d1_closed_form(r):
    rng = np.random.default_rng(500 + r)
    a, T = 0.1, 30
    q = rng.standard_normal((1, T, 1, 1))
    k = rng.standard_normal((1, T, 1, 1))
    v = rng.standard_normal((1, T, 1, 1))
    g = rng.uniform(0, 1, (1, T, 1))
    out = gka_forward_ref(q, k, v, g, a, r)["o"][0, :, 0, 0]
    h = u = 0.0
    fac = 1 - (-1) ** r / _cheb_T(r, 1 + 2 * a)
    for t in range(T):
        h = g[0, t, 0] * h + k[0, t, 0, 0] ** 2
        u = g[0, t, 0] * u + v[0, t, 0, 0] * k[0, t, 0, 0]
        xs = q[0, t, 0, 0] / (h * (1 + a))
        assert out[t] == pytest.approx(u * fac * xs, rel=1e-12)


def test_zero_keys_give_zero_output():
    rng = np.random.default_rng(13)
    q, k, v, g = _rand_inputs(rng, 1, 12, 2, 4)
    k[:, :5] = 0.0
    for mode in ("cheb", "exact"):
        ref = gka_forward_ref(q, k, v, g, 0.1, 6, mode=mode)
        assert np.all(np.isfinite(ref["o"]))
        assert np.all(ref["o"][:, :5] == 0.0)
        assert np.all(ref["hnorm"][:, :5] == 0.0)
        assert np.all(np.abs(ref["o"][:, 5:]) > 0)


# ------------------------------------------------------------------------------------------
# 5. metamorphic properties
# ------------------------------------------------------------------------------------------

def test_linear_in_v_and_q():
    rng = np.random.default_rng(21)
    q, k, v, g = _rand_inputs(rng, 1, 16, 2, 6)
    q2, _, v2, _ = _rand_inputs(rng, 1, 16, 2, 6)
    f = lambda qq, vv: gka_forward_ref(qq, k, vv, g, 0.05, 7)["o"]
    np.testing.assert_allclose(f(q, 2 * v - 3 * v2), 2 * f(q, v) - 3 * f(q, v2), rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(f(0.5 * q + q2, v), 0.5 * f(q, v) + f(q2, v), rtol=1e-11, atol=1e-12)


def test_heads_and_batches_are_independent():
    rng = np.random.default_rng(22)
    q, k, v, g = _rand_inputs(rng, 2, 10, 3, 5)
    o = gka_forward_ref(q, k, v, g, 0.1, 5)["o"]
    perm = [2, 0, 1]
    op = gka_forward_ref(q[:, :, perm], k[:, :, perm], v[:, :, perm], g[:, :, perm], 0.1, 5)["o"]
    np.testing.assert_array_equal(op, o[:, :, perm])
    o1 = gka_forward_ref(q[1:], k[1:], v[1:], g[1:], 0.1, 5)["o"]
    np.testing.assert_array_equal(o1, o[1:])


def test_split_sequence_with_carried_state():
    rng = np.random.default_rng(23)
    q, k, v, g = _rand_inputs(rng, 2, 30, 2, 6)
    full = gka_forward_ref(q, k, v, g, 0.05, 10)
    p1 = gka_forward_ref(q[:, :13], k[:, :13], v[:, :13], g[:, :13], 0.05, 10)
    p2 = gka_forward_ref(q[:, 13:], k[:, 13:], v[:, 13:], g[:, 13:], 0.05, 10,
                         h0=p1["h"], u0=p1["u"], n2_0=p1["n2"])
    np.testing.assert_allclose(np.concatenate([p1["o"], p2["o"]], 1), full["o"], rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(p2["h"], full["h"], rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(p2["n2"], full["n2"], rtol=1e-12)


def test_step_chain_equals_forward():
    rng = np.random.default_rng(24)
    q, k, v, g = _rand_inputs(rng, 2, 9, 3, 5)
    full = gka_forward_ref(q, k, v, g, 0.1, 8)
    B, T, H, D = q.shape
    h, u, n2 = np.zeros((B, H, D, D)), np.zeros((B, H, D, D)), np.zeros((B, H))
    for t in range(T):
        o, h, u, n2 = gka_step_ref(q[:, t], k[:, t], v[:, t], g[:, t], 0.1, 8, h, u, n2)
        np.testing.assert_allclose(o, full["o"][:, t], rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(h, full["h"], rtol=1e-12, atol=1e-14)


def test_residuals_shape_and_decay():
    rng = np.random.default_rng(25)
    q, k, v, g = _rand_inputs(rng, 1, 8, 2, 6)
    out = gka_forward_ref(q, k, v, g, 0.1, 10, return_residuals=True)
    res = out["residuals"]
    assert res.shape == (1, 8, 2, 11)
    np.testing.assert_allclose(res[..., 0], np.linalg.norm(q, axis=-1), rtol=1e-14)
    assert np.all(res[..., -1] < 0.05 * res[..., 0])


def test_state_only_mode_advances_the_same_state():
    rng = np.random.default_rng(26)
    q, k, v, g = _rand_inputs(rng, 2, 12, 2, 5)
    a = gka_forward_ref(q, k, v, g, 0.1, 4)
    b = gka_forward_ref(q, k, v, g, 0.1, 4, mode="state")
    np.testing.assert_array_equal(a["h"], b["h"])
    np.testing.assert_array_equal(a["u"], b["u"])
    np.testing.assert_array_equal(a["n2"], b["n2"])
    assert np.all(b["o"] == 0)


# ------------------------------------------------------------------------------------------
# write gate beta_t (the beta-augmented recurrence, ai.info summary "Main Findings")
# ------------------------------------------------------------------------------------------

def _rand_beta(rng, shape, zeros=False):
    b = 1.0 / (1.0 + np.exp(-rng.normal(0.5, 1.5, shape)))
    if zeros:
        b[rng.random(shape) < 0.2] = 0.0
    return b


@pytest.mark.parametrize("gate", ["sigmoid", "with_zeros"])
@pytest.mark.parametrize("D", [1, 4, 12])
def test_beta_exact_mode_matches_bruteforce_ridge(gate, D):
    """With beta the objective weighs pair i by beta_i prod_{j>i} gamma_j (brute force)."""
    rng = np.random.default_rng(300 + D)
    T, a = 30, 0.1
    q, k, v, g = _rand_inputs(rng, 1, T, 2, D, gate)
    beta = _rand_beta(rng, (1, T, 2), zeros=True)
    ref = gka_forward_ref(q, k, v, g, a, iters=1, mode="exact", beta=beta)
    for h in range(2):
        o_bf, hn_bf = ridge_bruteforce(q[0, :, h], k[0, :, h], v[0, :, h], g[0, :, h], a,
                                       beta=beta[0, :, h])
        assert _rel(ref["o"][0, :, h], o_bf) < 1e-10
        np.testing.assert_allclose(ref["hnorm"][0, :, h], hn_bf, rtol=1e-12, atol=1e-300)


def test_beta_states_equal_direct_sums():
    rng = np.random.default_rng(310)
    T, D = 17, 6
    q, k, v, g = _rand_inputs(rng, 1, T, 1, D, "with_zeros")
    beta = _rand_beta(rng, (1, T, 1), zeros=True)
    out = gka_forward_ref(q, k, v, g, 0.1, 6, beta=beta)
    Ht = sum(beta[0, i, 0] * np.prod(g[0, i + 1:, 0]) * np.outer(k[0, i, 0], k[0, i, 0]) for i in range(T))
    Ut = sum(beta[0, i, 0] * np.prod(g[0, i + 1:, 0]) * np.outer(v[0, i, 0], k[0, i, 0]) for i in range(T))
    np.testing.assert_allclose(out["h"][0, 0], Ht, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(out["u"][0, 0], Ut, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(out["n2"][0, 0], np.sum(Ht * Ht), rtol=1e-12)


def test_beta_equals_scaled_keys_and_values():
    """beta_t k k^T = (sqrt(beta_t) k)(sqrt(beta_t) k)^T and beta_t v k^T likewise: the gated
    forward equals the plain forward fed sqrt(beta) k and sqrt(beta) v (q unchanged)."""
    rng = np.random.default_rng(311)
    q, k, v, g = _rand_inputs(rng, 2, 20, 3, 8, "with_zeros")
    beta = _rand_beta(rng, (2, 20, 3), zeros=True)
    sb = np.sqrt(beta)[..., None]
    a = gka_forward_ref(q, k, v, g, 0.05, 10, beta=beta)
    b = gka_forward_ref(q, k * sb, v * sb, g, 0.05, 10)
    for key in ("o", "hnorm", "h", "u", "n2"):
        np.testing.assert_allclose(a[key], b[key], rtol=1e-10, atol=1e-13)


def test_beta_ones_is_the_plain_layer():
    rng = np.random.default_rng(312)
    q, k, v, g = _rand_inputs(rng, 1, 15, 2, 6)
    a = gka_forward_ref(q, k, v, g, 0.1, 8)
    b = gka_forward_ref(q, k, v, g, 0.1, 8, beta=np.ones(g.shape))
    for key in ("o", "hnorm", "h", "u", "n2"):
        np.testing.assert_array_equal(a[key], b[key])


def test_beta_zero_token_writes_nothing():
    rng = np.random.default_rng(313)
    q, k, v, g = _rand_inputs(rng, 1, 6, 1, 5)
    beta = np.ones(g.shape)
    beta[0, 3, 0] = 0.0
    before = gka_forward_ref(q[:, :3], k[:, :3], v[:, :3], g[:, :3], 0.1, 8, beta=beta[:, :3])
    after = gka_forward_ref(q[:, :4], k[:, :4], v[:, :4], g[:, :4], 0.1, 8, beta=beta[:, :4])
    np.testing.assert_allclose(after["h"], g[0, 3, 0] * before["h"], rtol=1e-14)
    np.testing.assert_allclose(after["u"], g[0, 3, 0] * before["u"], rtol=1e-14)


def test_beta_step_chain_equals_forward():
    rng = np.random.default_rng(314)
    q, k, v, g = _rand_inputs(rng, 2, 9, 3, 5)
    beta = _rand_beta(rng, g.shape)
    full = gka_forward_ref(q, k, v, g, 0.1, 8, beta=beta)
    B, T, H, D = q.shape
    h, u, n2 = np.zeros((B, H, D, D)), np.zeros((B, H, D, D)), np.zeros((B, H))
    for t in range(T):
        o, h, u, n2 = gka_step_ref(q[:, t], k[:, t], v[:, t], g[:, t], 0.1, 8, h, u, n2,
                                   beta=beta[:, t])
        np.testing.assert_allclose(o, full["o"][:, t], rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(h, full["h"], rtol=1e-12, atol=1e-14)


# ------------------------------------------------------------------------------------------
# residual norms and the comparator solvers of the convergence plot (pith.science page,
# caption of Figure 1 (a); ai.info summary, "Main Findings", the CH-versus-CG bullet)
# ------------------------------------------------------------------------------------------

def _spd(rng, D, lo=0.2, hi=1.0):
    Q, _ = np.linalg.qr(rng.standard_normal((D, D)))
    lam = np.linspace(lo, hi, D)
    return Q @ np.diag(lam) @ Q.T, Q, lam


def test_cg_first_step_is_exact_line_search():
    # x_1 of CG is the steepest-descent step with exact line search: (b.b / b.Ab) b
    rng = np.random.default_rng(40)
    A, _, _ = _spd(rng, 9)
    b = rng.standard_normal(9)
    x1 = cg_solve(A, b, 1)
    np.testing.assert_allclose(x1, (b @ b) / (b @ A @ b) * b, rtol=1e-13)


def test_cg_second_iterate_is_the_krylov_galerkin_solution():
    # x_2 minimises the A-norm error over span{b, A b}: x = V (V^T A V)^-1 V^T b
    rng = np.random.default_rng(41)
    A, _, _ = _spd(rng, 11)
    b = rng.standard_normal(11)
    V = np.stack([b, A @ b], axis=1)
    x_ref = V @ np.linalg.solve(V.T @ A @ V, V.T @ b)
    np.testing.assert_allclose(cg_solve(A, b, 2), x_ref, rtol=1e-10, atol=1e-12)


def test_cg_terminates_after_as_many_steps_as_distinct_eigenvalues():
    rng = np.random.default_rng(42)
    D = 12
    Q, _ = np.linalg.qr(rng.standard_normal((D, D)))
    lam = np.array([0.3] * 4 + [0.7] * 5 + [1.1] * 3)  # three distinct eigenvalues
    A = Q @ np.diag(lam) @ Q.T
    b = rng.standard_normal(D)
    res = []
    cg_solve(A, b, 4, res)
    assert res[2] > 1e-3 * res[0]
    assert res[3] < 1e-12 * res[0]
    assert res[4] < 1e-12 * res[0]  # a converged system stays converged (no 0/0)


def test_gd_residuals_match_the_eigen_closed_form():
    # r_i = (I - c A)^i b with c = 2 / (L + mu)
    rng = np.random.default_rng(43)
    A, Q, lam = _spd(rng, 10, 0.25, 1.25)
    b = rng.standard_normal(10)
    mu, L = 0.25, 1.25
    c = 2.0 / (L + mu)
    res = []
    gd_solve(A, b, mu, L, 7, res)
    for i, r in enumerate(res):
        want = np.linalg.norm(Q @ ((1.0 - c * lam) ** i * (Q.T @ b)))
        assert abs(r - want) <= 1e-12 * np.linalg.norm(b)


def test_agd_residuals_match_the_characteristic_roots():
    # per eigen-mode lambda the error e_i = x* - x_i obeys
    # e_{i+1} = s ((1 + m) e_i - m e_{i-1}),  s = 1 - lambda / L,  e_{-1} = e_0 = x*,
    # so e_i = c1 z1^i + c2 z2^i with z1, z2 the roots of z^2 - (1 + m) s z + m s
    rng = np.random.default_rng(44)
    D = 8
    lam = np.linspace(0.3, 1.0, D)  # strictly inside (mu, L): distinct roots
    A = np.diag(lam)
    b = rng.standard_normal(D)
    mu, L = 0.2, 1.1
    kap = L / mu
    m = (np.sqrt(kap) - 1.0) / (np.sqrt(kap) + 1.0)
    res = []
    agd_solve(A, b, mu, L, 9, res)
    xs = b / lam
    sv = 1.0 - lam / L
    disc = ((1.0 + m) * sv) ** 2 - 4.0 * m * sv + 0j
    z1 = ((1.0 + m) * sv + np.sqrt(disc)) / 2.0
    z2 = ((1.0 + m) * sv - np.sqrt(disc)) / 2.0
    # c1 + c2 = x*, c1 / z1 + c2 / z2 = x*
    c1 = xs * (1.0 - 1.0 / z2) / (1.0 / z1 - 1.0 / z2)
    c2 = xs - c1
    for i, r in enumerate(res):
        e = (c1 * z1 ** i + c2 * z2 ** i).real
        assert abs(r - np.linalg.norm(lam * e)) <= 1e-12 * np.linalg.norm(b)


def test_solver_residuals_use_the_layer_systems():
    # the systems are A = H + a ||H||_F I: CG reaches their solution in D steps, and the
    # Chebyshev residuals are those the layer records for the same token
    rng = np.random.default_rng(45)
    q, k, v, g = _rand_inputs(rng, 1, 9, 1, 6)
    out = gka_forward_ref(q, k, v, g, 0.1, 5, return_residuals=True)
    H = out["h"][0, 0]
    qt = q[0, -1, 0]
    ch = solver_residuals(H, qt, 0.1, 5, "cheb")
    np.testing.assert_allclose(ch, out["residuals"][0, -1, 0], rtol=1e-12)
    cg = solver_residuals(H, qt, 0.1, 6, "cg")
    assert cg[-1] < 1e-10 * cg[0]
    A = H + 0.1 * np.linalg.norm(H) * np.eye(6)
    np.testing.assert_allclose(np.linalg.solve(A, qt), cg_solve(A, qt, 6), rtol=1e-8)
    for s in ("gd", "agd"):
        r = solver_residuals(H, qt, 0.1, 5, s)
        assert r.shape == (6,) and abs(r[0] - np.linalg.norm(qt)) < 1e-14


def test_solver_residuals_on_a_rank_one_state_follow_closed_forms():
    """The gd / agd / cg branches of solver_residuals pinned on the one state whose system has
    its extreme eigenvalues exactly at the layer's interval ends: H = diag(n, 0, ..., 0), so
    ||H||_F = n and A = H + a n I has eigenvalue L = (1 + a) n on e_0 and mu = a n on the rest.
    Textbook facts then fix every residual (kappa = L / mu = (1 + a) / a):
      * GD with step 2 / (L + mu): the residual along any eigenvector shrinks by
        |1 - 2 lambda / (L + mu)| per step, rho = (L - mu) / (L + mu) = 1 / (1 + 2 a) at both ends;
      * Nesterov AGD with step 1 / L: along lambda = L one step solves exactly (x_1 = q / L),
        along lambda = mu the momentum m = (sqrt(kappa) - 1) / (sqrt(kappa) + 1) makes the error
        recurrence critically damped, r_i = (1 + i / sqrt(kappa)) (1 - 1 / sqrt(kappa))^i;
      * CG: two distinct eigenvalues, so the residual vanishes after two steps.
    Swapping mu and L in the AGD call, or a wrong interval, breaks these."""
    a, n, D, iters = 0.1, 2.5, 5, 6
    H = np.zeros((D, D))
    H[0, 0] = n
    e0, e1 = np.eye(D)[0], np.eye(D)[1]
    i = np.arange(iters + 1)
    rho = 1.0 / (1.0 + 2.0 * a)
    for q in (e0, e1, 3.0 * e1):
        np.testing.assert_allclose(solver_residuals(H, q, a, iters, "gd"),
                                   np.linalg.norm(q) * rho ** i, rtol=1e-12)
    r = solver_residuals(H, 2.0 * e0, a, iters, "agd")
    assert r[0] == 2.0 and np.all(r[1:] < 1e-14)
    sk = np.sqrt((1.0 + a) / a)
    np.testing.assert_allclose(solver_residuals(H, e1, a, iters, "agd"),
                               (1.0 + i / sk) * (1.0 - 1.0 / sk) ** i, rtol=1e-10)
    r = solver_residuals(H, e0 + e1, a, 3, "cg")
    assert abs(r[0] - np.sqrt(2.0)) < 1e-14 and r[1] > 1e-3 and r[2] < 1e-13 and r[3] < 1e-13


def test_residuals_of_a_token_with_zero_state_are_q():
    # ||H_t|| = 0 (no key written yet): x_t = 0 is every iterate, so every residual is ||q_t||
    rng = np.random.default_rng(46)
    q, k, v, g = _rand_inputs(rng, 1, 6, 2, 5)
    k[0, :2, 0] = 0.0  # head 0: the first two tokens write nothing
    out = gka_forward_ref(q, k, v, g, 0.1, 6, return_residuals=True)
    res = out["residuals"]
    for t in range(2):
        np.testing.assert_array_equal(res[0, t, 0], np.full(7, np.linalg.norm(q[0, t, 0])))
    assert res[0, 2, 0, -1] < 0.1 * res[0, 2, 0, 0]
    assert np.all(res[0, :, 1, -1] < 0.1 * res[0, :, 1, 0])


def test_step_residuals_match_the_sequence_residuals():
    rng = np.random.default_rng(47)
    q, k, v, g = _rand_inputs(rng, 2, 5, 2, 4)
    full = gka_forward_ref(q, k, v, g, 0.05, 7, return_residuals=True)
    h, u, n2 = np.zeros((2, 2, 4, 4)), np.zeros((2, 2, 4, 4)), np.zeros((2, 2))
    for t in range(5):
        o, h, u, n2, r = gka_step_ref(q[:, t], k[:, t], v[:, t], g[:, t], 0.05, 7, h, u, n2,
                                      return_residuals=True)
        np.testing.assert_allclose(r, full["residuals"][:, t], rtol=1e-12, atol=1e-15)


# ------------------------------------------------------------------------------------------
# backward by implicit differentiation, pinned by finite differences of the forward
# ------------------------------------------------------------------------------------------

def _loss(q, k, v, g, do, a, iters, mode, beta):
    return float(np.sum(gka_forward_ref(q, k, v, g, a, iters, mode=mode, beta=beta)["o"] * do))


def _fd(f, x, idx, h=1e-6):
    xp, xm = x.copy(), x.copy()
    xp[idx] += h
    xm[idx] -= h
    return (f(xp) - f(xm)) / (2 * h)


@pytest.mark.parametrize("gated", [False, True])
def test_backward_matches_finite_differences_of_the_exact_solve(gated):
    # with the exact solve, implicit differentiation is the exact gradient of the forward:
    # central differences of L = sum <do, o> agree for every input
    rng = np.random.default_rng(60)
    B, T, H, D, a = 1, 5, 2, 4, 0.3
    q, k, v, g = _rand_inputs(rng, B, T, H, D)
    do = rng.standard_normal((B, T, H, D))
    beta = rng.uniform(0.2, 1.0, (B, T, H)) if gated else None
    grads = gka_backward_ref(q, k, v, g, do, a, 0, mode="exact", beta=beta)
    L = lambda **kw: _loss(kw.get("q", q), kw.get("k", k), kw.get("v", v), kw.get("g", g), do,
                           a, 0, "exact", kw.get("beta", beta))
    for t in range(T):
        for h in range(H):
            for i in (0, 3):
                idx = (0, t, h, i)
                assert abs(_fd(lambda x: L(q=x), q, idx) - grads["dq"][idx]) < 1e-6
                assert abs(_fd(lambda x: L(k=x), k, idx) - grads["dk"][idx]) < 1e-6
                assert abs(_fd(lambda x: L(v=x), v, idx) - grads["dv"][idx]) < 1e-6
            assert abs(_fd(lambda x: L(g=x), g, (0, t, h)) - grads["dgamma"][0, t, h]) < 1e-6
            if gated:
                assert abs(_fd(lambda x: L(beta=x), beta, (0, t, h)) - grads["dbeta"][0, t, h]) < 1e-6


def test_query_gradient_of_the_chebyshev_forward_is_the_solve():
    # Lemma 2: x_t is a fixed polynomial of A_t applied to q_t, so the gradient of the
    # Chebyshev forward with respect to q_t is that polynomial applied to U_t^T do_t --
    # the implicit gradient with the same solver -- exactly, not only in the limit
    rng = np.random.default_rng(61)
    B, T, H, D, a, r = 1, 6, 2, 5, 0.05, 6
    q, k, v, g = _rand_inputs(rng, B, T, H, D)
    do = rng.standard_normal((B, T, H, D))
    grads = gka_backward_ref(q, k, v, g, do, a, r, mode="cheb")
    for t in range(T):
        for i in range(D):
            idx = (0, t, 1, i)
            fd = _fd(lambda x: _loss(x, k, v, g, do, a, r, "cheb", None), q, idx)
            assert abs(fd - grads["dq"][idx]) < 1e-7


def test_backward_special_cases():
    rng = np.random.default_rng(62)
    B, T, H, D = 1, 6, 2, 4
    q, k, v, g = _rand_inputs(rng, B, T, H, D)
    do = rng.standard_normal((B, T, H, D))
    # zero upstream gradient: all gradients vanish
    z = gka_backward_ref(q, k, v, g, np.zeros_like(do), 0.1, 5)
    assert all(np.all(z[n] == 0) for n in z)
    # beta = 1 gives the ungated gradients, bit for bit in dq, dk, dv, dgamma
    a1 = gka_backward_ref(q, k, v, g, do, 0.1, 5)
    b1 = gka_backward_ref(q, k, v, g, do, 0.1, 5, beta=np.ones((B, T, H)))
    for n in ("dq", "dk", "dv", "dgamma", "dbeta"):
        np.testing.assert_array_equal(a1[n], b1[n])
    # a token before any key is written (||H_t|| = 0) has dq_t = 0
    k2 = k.copy()
    k2[0, :2, 0] = 0.0
    c = gka_backward_ref(q, k2, v, g, do, 0.1, 5)
    assert np.all(c["dq"][0, :2, 0] == 0.0)
