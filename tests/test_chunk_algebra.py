"""Float64 check of the chunk-wise algebra the HIP kernels implement (CPU only).

The kernels never form a per-token H_t. Inside a chunk of C tokens that starts from the state
(H0, U0, ||H0||^2) they use, with cl_t the in-chunk inclusive prefix sum of log gamma,
Gam_t = exp(cl_t) and the causal decay mask M_ts = exp(cl_t - cl_s) [s <= t]:

  H_t x      = Gam_t H0 x + sum_s M_ts (k_s . x) k_s
  ||H_t||^2  = Gam_t^2 ||H0||^2 + 2 Gam_t sum_s M_ts k_s^T H0 k_s + sum_{s,u} M_ts M_tu (k_s . k_u)^2
  U_t x      = Gam_t U0 x + sum_s M_ts (k_s . x) v_s
  carry      H0 <- Gam_C H0 + K^T diag(w) K,  U0 <- Gam_C U0 + V^T diag(w) K,  w_s = exp(cl_C - cl_s)

and they run the Chebyshev iteration on the system scaled by 1/||H_t||_F (spectrum in [a, 1+a],
so the step 2/(1+2a) and the weights are the same for every token). Sequence segments are
summarised from a zero state and combined by an affine scan. This file re-derives all of that in
plain numpy and checks it against the sequential oracle; it is a model of the design, written
here in the tests, and shares nothing with either the oracle or the HIP sources.
"""
import numpy as np
import pytest

from oracle import gka_forward_ref

LOG_FLOOR = -200.0


def _chunked_head(q, k, v, g, a, r, C, H0, U0, n20):
    T, D = q.shape
    c = 2.0 / (1.0 + 2.0 * a)
    rho = 1.0 / (1.0 + 2.0 * a)
    om = [2.0]
    for _ in range(1, r):
        om.append(4.0 / (4.0 - rho * rho * om[-1]))
    out = np.zeros((T, D))
    hn = np.zeros(T)
    for c0 in range(0, T, C):
        Q, K, V = q[c0:c0 + C], k[c0:c0 + C], v[c0:c0 + C]
        lg = np.where(g[c0:c0 + C] > 0, np.log(np.maximum(g[c0:c0 + C], 1e-300)), LOG_FLOOR)
        cl = np.cumsum(lg)
        Gam = np.exp(cl)
        M = np.tril(np.exp(np.minimum(cl[:, None] - cl[None, :], 0.0)))
        G = K @ K.T
        u = np.einsum("sd,de,se->s", K, H0, K)
        n2 = Gam ** 2 * n20 + 2 * Gam * (M @ u) + np.einsum("ts,su,tu->t", M, G * G, M)
        n = np.sqrt(n2)
        zero = n2 == 0
        ninv = np.where(zero, 0.0, 1.0 / np.where(zero, 1.0, n))
        s = Gam * ninv
        Mh = M * ninv[:, None]
        Qz = np.where(zero[:, None], 0.0, Q)

        def apply(X):
            return s[:, None] * (X @ H0) + ((X @ K.T) * Mh) @ K + a * X

        X = _residual_chebyshev(Qz, apply, c, om, r)
        out[c0:c0 + C] = s[:, None] * (X @ U0.T) + ((X @ K.T) * Mh) @ V
        hn[c0:c0 + C] = n
        w = np.exp(cl[-1] - cl)
        H0 = Gam[-1] * H0 + (K * w[:, None]).T @ K
        U0 = Gam[-1] * U0 + (V * w[:, None]).T @ K
        n20 = n2[-1]
    return out, hn, H0, U0, n20


def _residual_chebyshev(Q, apply, c, om, r):
    """Chebyshev iteration on the residuals R_i = Q - A X_i with X_r = sum_i beta_i R_i.

    Same iterates as x_{i+1} = x_{i-1} + omega_i (x_i - x_{i-1} + c (q - A x_i)) in exact
    arithmetic; beta follows from x_0 = 0, x_1 = c r_0 and that recurrence.
    """
    prev, cur = [], [c]
    for i in range(1, r):
        cur, prev = [(1 - om[i]) * (prev[j] if j < len(prev) else 0.0) + om[i] * cur[j]
                     for j in range(i)] + [om[i] * c], cur
    R, Rp = Q.copy(), None
    X = cur[0] * R
    for i in range(r - 1):
        AR = apply(R)
        Rn = R - c * AR if i == 0 else Rp + om[i] * (R - Rp - c * AR)
        Rp, R = R, Rn
        X = X + cur[i + 1] * R
    return X


S0 = 0.7390851332151607  # the rescaling's start value s_0 = s_1 (the fixed point of cos)


def _rescaled_chebyshev(Q, apply, a, c, om, r):
    """The same iteration on rescaled residuals Rt_i = R_i / s_i, s_0 = s_1 = S0 and
    s_{i+1} = (1 - omega_i) s_{i-1}: the R_{i-1} term then needs no multiply,
    Rt_{i+1} = Rt_{i-1} + krs_i Rt_i + kys_i (A - a I) Rt_i and x_r = sum_i beta_i s_i Rt_i.
    The iteration stops before a step whose |1 - omega_i| is below 2^-64 (from then on every
    residual is below 2^-64 of the first). Returns X and the number of iterations run.
    """
    prev, cur = [], [c]
    for i in range(1, r):
        cur, prev = [(1 - om[i]) * (prev[j] if j < len(prev) else 0.0) + om[i] * cur[j]
                     for j in range(i)] + [om[i] * c], cur
    R, Rp = Q / S0, np.zeros_like(Q)
    X = cur[0] * S0 * R
    s, ratio = S0, 1.0
    for i in range(r - 1):
        w = 1.0 if i == 0 else om[i]
        kp = 0.0 if i == 0 else 1.0 - om[i]
        if i >= 1 and abs(kp) < 2.0 ** -64:
            return X, i + 1
        rn = 1.0 if i == 0 else kp / ratio
        krs, kys = w * (1.0 - c * a) / rn, -w * c / rn
        Rn = Rp + krs * R + kys * (apply(R) - a * R)
        Rp, R = R, Rn
        s, ratio = s * rn, rn
        X = X + cur[i + 1] * s * R
    return X, r


@pytest.mark.parametrize("a,r", [(0.02, 12), (0.05, 10), (0.1, 8), (1.0, 6), (0.05, 1),
                                 (0.05, 2), (0.02, 64), (1e13, 10)])
def test_rescaled_residual_recurrence(a, r):
    """The rescaled residual form the bf16 walk runs gives the iterate of the plain residual
    form (and, for huge a, stops early at no visible cost)."""
    rng = np.random.default_rng(7)
    D, n = 12, 5
    Bm = rng.standard_normal((D, D))
    Hn = Bm @ Bm.T
    Hn /= np.linalg.norm(Hn)  # the normalised system: spectrum in [a, 1 + a]
    Q = rng.standard_normal((n, D))
    apply = lambda X: X @ Hn + a * X
    c = 2.0 / (1.0 + 2.0 * a)
    rho = 1.0 / (1.0 + 2.0 * a)
    om = [2.0]
    for _ in range(1, r):
        om.append(4.0 / (4.0 - rho * rho * om[-1]))
    ref = _residual_chebyshev(Q, apply, c, om, r)
    got, used = _rescaled_chebyshev(Q, apply, a, c, om, r)
    assert np.linalg.norm(got - ref) <= 1e-12 * np.linalg.norm(ref)
    assert used == r if a < 1e6 else used < r


def _inputs(seed, T, D, gate_mu=2.0, zeros=False):
    rng = np.random.default_rng(seed)
    q, k, v = (rng.standard_normal((T, D)) for _ in range(3))
    q /= np.linalg.norm(q, axis=1, keepdims=True)
    k /= np.linalg.norm(k, axis=1, keepdims=True)
    g = 1.0 / (1.0 + np.exp(-rng.normal(gate_mu, 1.0, T)))
    if zeros:
        g[rng.random(T) < 0.1] = 0.0
    return q, k, v, g


@pytest.mark.parametrize("C", [4, 8, 16])
@pytest.mark.parametrize("zeros", [False, True])
def test_chunked_form_matches_sequential_oracle(C, zeros):
    T, D, a, r = 48, 8, 0.05, 10
    q, k, v, g = _inputs(C + 10 * zeros, T, D, zeros=zeros)
    ref = gka_forward_ref(q[None, :, None], k[None, :, None], v[None, :, None], g[None, :, None], a, r)
    o, hn, H, U, n2 = _chunked_head(q, k, v, g, a, r, C, np.zeros((D, D)), np.zeros((D, D)), 0.0)
    assert np.linalg.norm(o - ref["o"][0, :, 0]) < 1e-10 * np.linalg.norm(o)
    np.testing.assert_allclose(hn, ref["hnorm"][0, :, 0], rtol=1e-12)
    np.testing.assert_allclose(H, ref["h"][0, 0], rtol=1e-11, atol=1e-13)
    np.testing.assert_allclose(U, ref["u"][0, 0], rtol=1e-11, atol=1e-13)
    assert n2 == pytest.approx(ref["n2"][0, 0], rel=1e-12)


def test_segment_summaries_and_scan_reproduce_the_carry():
    T, D, C, S = 64, 6, 8, 4
    q, k, v, g = _inputs(3, T, D, zeros=True)
    Z = np.zeros((D, D))
    Hs, Us = np.eye(D) * 0.3, np.ones((D, D)) * 0.1  # arbitrary start state
    _, _, Hend, Uend, _ = _chunked_head(q, k, v, g, 0.1, 3, C, Hs, Us, np.sum(Hs * Hs))
    # per-segment summaries from a zero state and the segment's total gate product
    seg = T // S
    summ = []
    for si in range(S):
        sl = slice(si * seg, (si + 1) * seg)
        _, _, dH, dU, _ = _chunked_head(q[sl], k[sl], v[sl], g[sl], 0.1, 1, C, Z, Z, 0.0)
        lg = np.where(g[sl] > 0, np.log(np.maximum(g[sl], 1e-300)), LOG_FLOOR)
        summ.append((np.exp(lg.sum()), dH, dU))
    H, U = Hs, Us
    for G, dH, dU in summ:
        H, U = G * H + dH, G * U + dU
    np.testing.assert_allclose(H, Hend, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(U, Uend, rtol=1e-12, atol=1e-14)


@pytest.mark.parametrize("regime,mu,a,r", [("figure_shape", 3.0, 0.05, 10),
                                             ("long_memory", 4.0, 0.02, 12),
                                             ("short_memory", -1.0, 0.02, 12),
                                             ("no_memory", None, 0.05, 10)])
def test_fp16_operand_rounding_budget(regime, mu, a, r):
    """fp16 matrix-core operands, rounded where the kernels round them, stay well inside the 2e-2
    bar in every gate regime (and ||H_t||_F inside 1e-3).

    Rounded to fp16 (round to nearest even): the keys and values (exact for bf16 inputs in
    fp16's normal range), the copies H0/n0 and U0/n0 of the chunk-start state, the residual
    operand of every product in the loop and the masked products P' (in the loop and in the
    output). Split into hi + lo fp16 parts: the iterate X in both output products, and the
    gate-weighted keys of the carry (so the float32 state is accurate to float32). Rounding the
    plain iterate instead of the residual costs up to (1+a)/a times the unit error; so does
    rounding X to one fp16 part in the output when H_t is nearly low-rank (short gate memory:
    about 6e-3 here at a = 0.02, against about 4e-4 with the split).
    """
    from test_ridge_regression_amd.workloads import round_bf16

    rb = lambda x: round_bf16(x).astype(np.float64)
    rh = lambda x: np.asarray(x).astype(np.float16).astype(np.float64)
    split = lambda x: rh(x) + rh(x - rh(x))
    T, D, C = 384, 64, 64
    rng = np.random.default_rng(42)
    q, k, v = (rng.standard_normal((T, D)) for _ in range(3))
    q, k = rb(q / np.linalg.norm(q, axis=1, keepdims=True)), rb(k / np.linalg.norm(k, axis=1, keepdims=True))
    v = rb(v)
    g = np.zeros(T) if mu is None else \
        (1.0 / (1.0 + np.exp(-rng.normal(mu, 1.0, T)))).astype(np.float32).astype(np.float64)
    ref = gka_forward_ref(q[None, :, None], k[None, :, None], v[None, :, None], g[None, :, None], a, r)
    cst = 2.0 / (1.0 + 2.0 * a)
    rho = 1.0 / (1.0 + 2.0 * a)
    om = [2.0]
    for _ in range(1, r):
        om.append(4.0 / (4.0 - rho * rho * om[-1]))
    H0 = np.zeros((D, D))
    U0 = np.zeros((D, D))
    n20 = 0.0
    out = np.zeros((T, D))
    hn = np.zeros(T)
    for c0 in range(0, T, C):
        Q, K, V = q[c0:c0 + C], rh(k[c0:c0 + C]), rh(v[c0:c0 + C])
        cl = np.cumsum(np.where(g[c0:c0 + C] > 0, np.log2(np.maximum(g[c0:c0 + C], 1e-300)), -160.0))
        Gam = 2.0 ** cl
        M = np.tril(2.0 ** np.minimum(cl[:, None] - cl[None, :], 0.0))
        n0 = np.sqrt(n20)
        n0inv = 1.0 / n0 if n0 > 0 else 0.0
        Hh, Uh = rh(H0 * n0inv), rh(U0 * n0inv)
        n2 = Gam ** 2 * n20 + 2 * Gam * n0 * (M @ np.einsum("sd,de,se->s", K, Hh, K)) + \
            np.einsum("ts,su,tu->t", M, (K @ K.T) ** 2, M)
        n = np.sqrt(n2)
        s, Mh = Gam * n0 / n, M / n[:, None]

        def apply(R):
            Rh = rh(R)
            return s[:, None] * (Rh @ Hh) + rh((Rh @ K.T) * Mh) @ K + a * R

        X, _ = _rescaled_chebyshev(Q, apply, a, cst, om, r)  # the bf16 walk's form
        Xs = split(X)
        out[c0:c0 + C] = s[:, None] * (Xs @ Uh.T) + rh((Xs @ K.T) * Mh) @ V
        hn[c0:c0 + C] = n
        wK = split(K * (2.0 ** (cl[-1] - cl))[:, None])
        H0 = Gam[-1] * H0 + wK.T @ K
        U0 = Gam[-1] * U0 + V.T @ wK
        n20 = n2[-1]
    err = np.linalg.norm(out - ref["o"][0, :, 0]) / np.linalg.norm(ref["o"][0, :, 0])
    errh = np.max(np.abs(hn - ref["hnorm"][0, :, 0]) / ref["hnorm"][0, :, 0])
    assert err < 1e-2, (regime, err)
    assert errh < 1e-4, (regime, errh)
