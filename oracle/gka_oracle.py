"""Plain float64 CPU oracle of the Gated KalmaNet (GKA) forward pass.

TEST INFRASTRUCTURE ONLY. Only the tests, the package's smoke check and the bench's CPU-baseline
leg may import this module. The GPU library never calls it and shares no code with it.

What it computes, token by token and head by head (the pages name the pieces; the order below
is the plainest reading that all of them support):

  ridge objective   S_t = argmin_S  sum_{i<=t} eta_{t,i} ||v_i - S k_i||^2 + lambda_t ||S||_F^2,
                    o_t = S_t q_t           (ai.info summary, "Main Findings", the KF objective
                                             "Eq. 3"; pith.science page, appendix fragment
                                             "No weighting", which sets eta_i = 1 in (3))
  closed form       (H_t + lambda_t I) x_t = q_t,  o_t = U_t x_t
                                            (ai.info summary, "Methodology in Plain English")
  gated weights     eta_{t,i} = prod_{j=i+1}^{t} gamma_j, gamma_j in [0, 1]
                                            (pith.science page, appendix fragment "Adaptive
                                             weighting (gating)"), i.e.
                    H_t = gamma_t H_{t-1} + k_t k_t^T,  U_t = gamma_t U_{t-1} + v_t k_t^T
  adaptive ridge    lambda_t = a ||H_t||_F, so kappa_t <= (a+1)/a
                                            (ai.info summary, "Key Contributions" 2 and
                                             "Main Findings")
  Frobenius norm    ||H_t||_F^2 = gamma_t^2 ||H_{t-1}||_F^2 + 2 gamma_t k_t^T H_{t-1} k_t
                                  + ||k_t||^4   (expanding the square of the update above)
  solver            Chebyshev Iteration on the spectral interval [mu, L] = [lambda_t,
                    lambda_t + ||H_t||_F] (H_t is PSD, so its largest eigenvalue is at most
                    ||H_t||_F), with the weight schedule omega_i = 4 / (4 - rho^2 omega_{i-1}),
                    rho = (L - mu)/(L + mu), omega_0 = 2 (pith.science page, appendix fragments
                    around Lemma 3 -- omega_i in [1, 2] and non-increasing -- and Lemma 4 with
                    kappa = L/mu); the three-term Chebyshev semi-iterative form of Golub and
                    Van Loan, "Matrix Computations" (cited in the pages' reference list)
  exact mode        Cholesky solve of the same SPD system, for the pins only (the pages'
                    exact-solver reference, ai.info summary "Key Contributions" 2)
  residuals         optionally ||q_t - A_t x_i|| for i = 0..iters, the quantity of the pages'
                    convergence plot (pith.science page, caption of Figure 1 (a); ai.info
                    summary, "Main Findings", the bullet comparing CH with CG)
  backward          gradients of L = sum_t <do_t, o_t> by implicit differentiation of the solve
                    (ai.info summary, "Methodology in Plain English" and "Main Findings": the
                    backward re-runs the solver on the upstream gradient; Lemma 2: the query
                    gradient is that solve), through the adaptive ridge lambda_t = a ||H_t||_F
                    and back through the gated recurrences (derivation in gka_backward_ref)
  comparators       conjugate gradient, gradient descent and accelerated gradient descent on
                    the same systems (the solvers CH is compared with in those two passages),
                    for the convergence comparison only; the layer itself uses CH

  write gate        optional beta_t in [0, 1] scaling the token's write (ai.info summary, "Main
                    Findings", the beta_t-augmented variant; its "Future Directions" call it the
                    released default): H_t = gamma_t H_{t-1} + beta_t k_t k_t^T and
                    U_t = gamma_t U_{t-1} + beta_t v_t k_t^T, i.e. weights eta_{t,i} beta_i in
                    the ridge objective; beta = None means beta_t = 1 (the paper's experiments)

Readings taken where the pages are silent (each also listed in the design notes):
  * x_0 = 0 and x_1 = c q (one Richardson step); "iters = r" means the iterate x_r is returned,
    i.e. r - 1 matrix-vector products with A;
  * gamma_t decays the state before token t writes (the gating fragment's eta_{t,i});
  * when ||H_t||_F = 0 (only possible when every weighted key so far is zero, hence U_t = 0)
    the solve is defined as x_t = 0 and o_t = 0; every iterate is then 0, so every residual
    q_t - A_t x_i is q_t;
  * the initial state is zero unless the caller passes one.

Everything is float64 and vectorised only across independent (batch, head) pairs; the loop
over tokens is the plain sequential recurrence.
"""
from __future__ import annotations

from typing import Optional

import numpy as np


# ------------------------------------------------------------------------------------------
# Chebyshev Iteration
# ------------------------------------------------------------------------------------------

def chebyshev_weights(rho, iters: int):
    """Weight schedule omega_0..omega_{iters-1}: omega_0 = 2, omega_i = 4 / (4 - rho^2 omega_{i-1}).

    Follows the weight-schedule update on the pith.science page (Lemma 3 and the map used in
    the proof of Lemma 4). ``rho`` may be an array (one value per system).
    """
    rho = np.asarray(rho, dtype=np.float64)
    omegas = [np.full(rho.shape, 2.0)]
    for _ in range(1, iters):
        omegas.append(4.0 / (4.0 - rho * rho * omegas[-1]))
    return omegas


def chebyshev_rates(kappa: float):
    """Rates of Lemma 4 (pith.science page): R_a = (sqrt(k)-1)/(sqrt(k)+1), R = (k-1)/(k+1) * R_a."""
    ra = (np.sqrt(kappa) - 1.0) / (np.sqrt(kappa) + 1.0)
    rho = (kappa - 1.0) / (kappa + 1.0)
    return rho * ra, ra


def chebyshev_solve(A: np.ndarray, b: np.ndarray, mu: np.ndarray, L: np.ndarray, iters: int,
                    residuals: Optional[list] = None) -> np.ndarray:
    """Chebyshev Iteration for A x = b with spectrum(A) in [mu, L]; batched over leading axes.

    A: [..., D, D], b: [..., D], mu, L: [...]. Returns the iterate x_iters.
    Starts at x_0 = 0; x_1 = x_0 + c (b - A x_0) = c b with c = 2/(L+mu); then for i >= 1
      x_{i+1} = x_{i-1} + omega_i (x_i - x_{i-1} + c (b - A x_i)).
    If ``residuals`` is a list, ||b - A x_i|| for i = 0..iters is appended to it.
    """
    c = (2.0 / (L + mu))[..., None]
    rho = (L - mu) / (L + mu)
    omegas = chebyshev_weights(rho, iters)
    x_prev = np.zeros_like(b)
    x = c * b
    if residuals is not None:
        residuals.append(np.linalg.norm(b, axis=-1))
        residuals.append(np.linalg.norm(b - np.einsum("...ij,...j->...i", A, x), axis=-1))
    for i in range(1, iters):
        r = b - np.einsum("...ij,...j->...i", A, x)
        w = omegas[i][..., None]
        x_next = x_prev + w * (x - x_prev + c * r)
        x_prev, x = x, x_next
        if residuals is not None:
            residuals.append(np.linalg.norm(b - np.einsum("...ij,...j->...i", A, x), axis=-1))
    return x


# ------------------------------------------------------------------------------------------
# Comparator solvers (convergence comparison only; x_0 = 0 and residuals[i] = ||b - A x_i||)
# ------------------------------------------------------------------------------------------

def _matvec(A, x):
    return np.einsum("...ij,...j->...i", A, x)


def cg_solve(A: np.ndarray, b: np.ndarray, iters: int, residuals: Optional[list] = None):
    """Conjugate gradient (Hestenes-Stiefel) for SPD A; iterate x_i after i steps (i products
    with A). A system whose residual is exactly 0 stays where it is."""
    x = np.zeros_like(b)
    r = b.copy()
    p = r.copy()
    rr = np.einsum("...i,...i->...", r, r)
    if residuals is not None:
        residuals.append(np.sqrt(rr))
    for _ in range(iters):
        Ap = _matvec(A, p)
        pAp = np.einsum("...i,...i->...", p, Ap)
        alpha = np.where(rr > 0.0, rr / np.where(pAp > 0.0, pAp, 1.0), 0.0)[..., None]
        x = x + alpha * p
        r = r - alpha * Ap
        rr_new = np.einsum("...i,...i->...", r, r)
        beta = np.where(rr > 0.0, rr_new / np.where(rr > 0.0, rr, 1.0), 0.0)[..., None]
        p = r + beta * p
        rr = rr_new
        if residuals is not None:
            residuals.append(np.linalg.norm(b - _matvec(A, x), axis=-1))
    return x


def gd_solve(A: np.ndarray, b: np.ndarray, mu, L, iters: int,
             residuals: Optional[list] = None):
    """Gradient descent on 1/2 x^T A x - b^T x with the fixed step c = 2 / (L + mu) (the
    optimal constant step for spectrum in [mu, L]): x_{i+1} = x_i + c (b - A x_i). Its first
    iterate equals CH's x_1."""
    c = (2.0 / (np.asarray(L, np.float64) + np.asarray(mu, np.float64)))[..., None]
    x = np.zeros_like(b)
    if residuals is not None:
        residuals.append(np.linalg.norm(b, axis=-1))
    for _ in range(iters):
        x = x + c * (b - _matvec(A, x))
        if residuals is not None:
            residuals.append(np.linalg.norm(b - _matvec(A, x), axis=-1))
    return x


def agd_solve(A: np.ndarray, b: np.ndarray, mu, L, iters: int,
              residuals: Optional[list] = None):
    """Accelerated gradient descent (Nesterov's constant-momentum scheme for an L-smooth,
    mu-strongly convex objective, here 1/2 x^T A x - b^T x): y_i = x_i + m (x_i - x_{i-1}),
    x_{i+1} = y_i + (b - A y_i) / L, m = (sqrt(kappa) - 1) / (sqrt(kappa) + 1), kappa = L / mu,
    x_{-1} = x_0 = 0."""
    L = np.asarray(L, np.float64)
    kappa = L / np.asarray(mu, np.float64)
    m = ((np.sqrt(kappa) - 1.0) / (np.sqrt(kappa) + 1.0))[..., None]
    step = (1.0 / L)[..., None]
    x_prev = np.zeros_like(b)
    x = np.zeros_like(b)
    if residuals is not None:
        residuals.append(np.linalg.norm(b, axis=-1))
    for _ in range(iters):
        y = x + m * (x - x_prev)
        x_prev, x = x, y + step * (b - _matvec(A, y))
        if residuals is not None:
            residuals.append(np.linalg.norm(b - _matvec(A, x), axis=-1))
    return x


SOLVERS = ("cheb", "cg", "gd", "agd")


def solver_residuals(H: np.ndarray, q: np.ndarray, a: float, iters: int, solver: str):
    """Residual norms ||q - A x_i||, i = 0..iters, of one solver on the layer's systems
    A = H + a ||H||_F I with the layer's interval [mu, L] = [a ||H||_F, (1 + a) ||H||_F].
    H: [..., D, D] PSD with ||H||_F > 0, q: [..., D]. Returns [..., iters + 1]."""
    H = np.asarray(H, np.float64)
    q = np.asarray(q, np.float64)
    n = np.linalg.norm(H, axis=(-2, -1))
    A = H + (a * n)[..., None, None] * np.eye(H.shape[-1])
    mu, L = a * n, (1.0 + a) * n
    res: list = []
    if solver == "cheb":
        chebyshev_solve(A, q, mu, L, iters, res)
    elif solver == "cg":
        cg_solve(A, q, iters, res)
    elif solver == "gd":
        gd_solve(A, q, mu, L, iters, res)
    elif solver == "agd":
        agd_solve(A, q, mu, L, iters, res)
    else:
        raise ValueError(f"unknown solver {solver!r}")
    return np.stack(res, axis=-1)


def cholesky_solve(A: np.ndarray, b: np.ndarray) -> np.ndarray:
    """Exact solve of the SPD system A x = b through its Cholesky factor (batched)."""
    Lc = np.linalg.cholesky(A)
    y = np.linalg.solve(Lc, b[..., None])
    return np.linalg.solve(np.swapaxes(Lc, -1, -2), y)[..., 0]


# ------------------------------------------------------------------------------------------
# One token of the recurrence
# ------------------------------------------------------------------------------------------

def _token(H, U, n2, q, k, v, g, a, iters, mode, residuals=None, b=None):
    """Advance (H, U, n2) by one token for every system and return (H, U, n2, x, o).

    H, U: [N, D, D]; n2, g: [N]; q, k, v: [N, D]; b: [N] write gate or None (= 1).
    With the write gate the update is H <- g H + b k k^T, U <- g U + b v k^T, so that
    ||H||^2 <- g^2 ||H||^2 + 2 g b k^T H k + b^2 ||k||^4 (the square of the update, expanded).
    """
    if b is None:
        b = np.ones_like(g)
    kHk = np.einsum("ni,nij,nj->n", k, H, k)
    kk = np.einsum("ni,ni->n", k, k)
    n2 = g * g * n2 + 2.0 * g * b * kHk + (b * kk) ** 2
    H = g[:, None, None] * H + b[:, None, None] * (k[:, :, None] * k[:, None, :])
    U = g[:, None, None] * U + b[:, None, None] * (v[:, :, None] * k[:, None, :])
    if mode == "state":  # advance the state only (no solve); o is returned as zeros
        return H, U, n2, np.zeros_like(q), np.zeros_like(q)
    n = np.sqrt(n2)
    lam = a * n
    D = H.shape[-1]
    zero = n2 == 0.0
    A = H + lam[:, None, None] * np.eye(D)
    if zero.any():  # degenerate systems: keep the solver finite, the result is forced to 0
        A = np.where(zero[:, None, None], np.eye(D), A)
    if mode == "cheb":
        mu = np.where(zero, 1.0, lam)
        L = np.where(zero, 1.0, lam + n)
        rl = [] if residuals is not None else None
        x = chebyshev_solve(A, q, mu, L, iters, rl)
        if residuals is not None:  # x_t = 0 for ||H_t|| = 0: every residual is q_t
            qn = np.linalg.norm(q, axis=-1)
            residuals.extend(np.where(zero, qn, r) for r in rl)
    elif mode == "exact":
        x = cholesky_solve(A, q)
    else:
        raise ValueError(f"unknown mode {mode!r}")
    x = np.where(zero[:, None], 0.0, x)
    o = np.einsum("nij,nj->ni", U, x)
    return H, U, n2, x, o


# ------------------------------------------------------------------------------------------
# Public entry points
# ------------------------------------------------------------------------------------------

def gka_forward_ref(q, k, v, gamma, a: float, iters: int, mode: str = "cheb",
                    h0=None, u0=None, n2_0=None, return_residuals: bool = False, beta=None):
    """Sequential forward over a whole sequence.

    ``mode``: "cheb" (Chebyshev Iteration, as the layer), "exact" (Cholesky solve), or
    "state" (advance H, U, ||H||^2 only; o is all zeros).

    q, k, v: [B, T, H, D]; gamma and the optional write gate beta: [B, T, H] (beta None: all
    ones); optional initial state h0, u0 [B, H, D, D]
    (U indexed [value dim][key dim]) and n2_0 [B, H] (= ||h0||_F^2 as carried by the caller).
    Returns a dict with o [B,T,H,D], hnorm [B,T,H] (= ||H_t||_F from the recurrence),
    h, u [B,H,D,D] and n2 [B,H] (final state), and optionally residuals
    [B, T, H, iters+1] (||q_t - A_t x_i|| for i = 0..iters, Chebyshev mode only).
    """
    q, k, v = (np.asarray(x, dtype=np.float64) for x in (q, k, v))
    gamma = np.asarray(gamma, dtype=np.float64)
    B, T, Hh, D = q.shape
    N = B * Hh

    def heads(x):  # [B,T,H,...] -> [B*H, T, ...]
        return np.moveaxis(x, 2, 1).reshape((N, T) + x.shape[3:])

    qh, kh, vh, gh = heads(q), heads(k), heads(v), heads(gamma)
    bh = None if beta is None else heads(np.asarray(beta, dtype=np.float64))
    H = np.zeros((N, D, D)) if h0 is None else np.asarray(h0, np.float64).reshape(N, D, D).copy()
    U = np.zeros((N, D, D)) if u0 is None else np.asarray(u0, np.float64).reshape(N, D, D).copy()
    n2 = np.zeros(N) if n2_0 is None else np.asarray(n2_0, np.float64).reshape(N).copy()
    o = np.empty((N, T, D))
    hn = np.empty((N, T))
    res = np.empty((N, T, iters + 1)) if return_residuals else None
    for t in range(T):
        rl = [] if return_residuals else None
        H, U, n2, _, o[:, t] = _token(H, U, n2, qh[:, t], kh[:, t], vh[:, t], gh[:, t], a, iters,
                                      mode, rl, None if bh is None else bh[:, t])
        hn[:, t] = np.sqrt(n2)
        if return_residuals:
            res[:, t] = np.stack(rl, axis=-1)

    def unheads(x):  # [B*H, T, ...] -> [B,T,H,...]
        return np.moveaxis(x.reshape((B, Hh, T) + x.shape[2:]), 1, 2)

    out = dict(o=unheads(o), hnorm=unheads(hn), h=H.reshape(B, Hh, D, D),
               u=U.reshape(B, Hh, D, D), n2=n2.reshape(B, Hh))
    if return_residuals:
        out["residuals"] = unheads(res)
    return out


def gka_step_ref(q, k, v, gamma, a: float, iters: int, h, u, n2, mode: str = "cheb",
                 beta=None, return_residuals: bool = False):
    """One recurrent decode step: update the carried state with the token, then solve.

    q, k, v: [B, H, D]; gamma and the optional write gate beta: [B, H]; h, u: [B, H, D, D];
    n2: [B, H].
    Returns (o [B,H,D], h, u, n2) -- new arrays, inputs untouched -- and, with
    ``return_residuals``, a fifth entry [B, H, iters+1]: ||q - A x_i|| for i = 0..iters.
    """
    q, k, v = (np.asarray(x, dtype=np.float64) for x in (q, k, v))
    B, Hh, D = q.shape
    N = B * Hh
    rl = [] if return_residuals else None
    H2, U2, n22, _, o = _token(np.asarray(h, np.float64).reshape(N, D, D),
                               np.asarray(u, np.float64).reshape(N, D, D),
                               np.asarray(n2, np.float64).reshape(N),
                               q.reshape(N, D), k.reshape(N, D), v.reshape(N, D),
                               np.asarray(gamma, np.float64).reshape(N), a, iters, mode, rl,
                               None if beta is None else np.asarray(beta, np.float64).reshape(N))
    out = (o.reshape(B, Hh, D), H2.reshape(B, Hh, D, D), U2.reshape(B, Hh, D, D),
           n22.reshape(B, Hh))
    if return_residuals:
        out = out + (np.stack(rl, axis=-1).reshape(B, Hh, iters + 1),)
    return out


def ridge_bruteforce(q, k, v, gamma, a: float, beta=None):
    """Solve the weighted ridge objective directly for one head, by least squares.

    q, k, v: [T, D]; gamma (and the optional write gate beta): [T]. For every t the weights
    eta_{t,i} = beta_i prod_{j=i+1}^{t} gamma_j are formed as plain products,
    H_t = sum_i eta_{t,i} k_i k_i^T is summed directly,
    lambda_t = a ||H_t||_F, and
        min_S  sum_{i<=t} eta_{t,i} ||v_i - S k_i||^2 + lambda_t ||S||_F^2
    is solved as the stacked least-squares problem [sqrt(eta_i) k_i^T ; sqrt(lambda_t) I] S^T
    ~= [sqrt(eta_i) v_i^T ; 0]. Returns o [T, D] with o_t = S_t q_t and hnorm [T].
    """
    q, k, v = (np.asarray(x, dtype=np.float64) for x in (q, k, v))
    gamma = np.asarray(gamma, dtype=np.float64)
    T, D = k.shape
    beta = np.ones(T) if beta is None else np.asarray(beta, dtype=np.float64)
    o = np.zeros((T, D))
    hn = np.zeros(T)
    for t in range(T):
        eta = np.array([beta[i] * np.prod(gamma[i + 1:t + 1]) for i in range(t + 1)])
        Ht = sum(eta[i] * np.outer(k[i], k[i]) for i in range(t + 1))
        hn[t] = np.linalg.norm(Ht, "fro")
        lam = a * hn[t]
        X = np.vstack([np.sqrt(eta)[:, None] * k[:t + 1], np.sqrt(lam) * np.eye(D)])
        Y = np.vstack([np.sqrt(eta)[:, None] * v[:t + 1], np.zeros((D, D))])
        St, *_ = np.linalg.lstsq(X, Y, rcond=None)  # St = S^T, [D_k, D_v]
        o[t] = St.T @ q[t]
    return o, hn


# ------------------------------------------------------------------------------------------
# Backward pass by implicit differentiation
# ------------------------------------------------------------------------------------------

def gka_backward_ref(q, k, v, gamma, do, a: float, iters: int, mode: str = "cheb", beta=None):
    """Gradients of L = sum_t <do_t, o_t> with respect to q, k, v, gamma (and beta).

    The solve x_t = A_t^-1 q_t, A_t = H_t + a ||H_t||_F I (symmetric), is differentiated
    implicitly: with g_t = U_t^T do_t (= dL/dx_t) and y_t = A_t^-1 g_t (the same solver on the
    upstream gradient, ``mode`` "cheb" or "exact"),
        dq_t = y_t,
        dL/dA_t = -y_t x_t^T, and A_t depends on H_t directly and through lambda_t, whose
        derivative is a H_t / ||H_t||_F; so the local gradients of the statistics are
        G_t = -y_t x_t^T + c_t H_t,  c_t = -a (y_t . x_t) / ||H_t||_F,   W_t = do_t x_t^T.
    Back through H_t = gamma_t H_{t-1} + beta_t k_t k_t^T (and U_t likewise) the total
    gradients obey Gb_t = G_t + gamma_{t+1} Gb_{t+1}, Wb_t = W_t + gamma_{t+1} Wb_{t+1}, and
        dk_t = beta_t ((Gb_t + Gb_t^T) k_t + Wb_t^T v_t),   dv_t = beta_t Wb_t k_t,
        dbeta_t = k_t^T Gb_t k_t + v_t^T Wb_t k_t,
        dgamma_t = <Gb_t, H_{t-1}> + <Wb_t, U_{t-1}>.
    A token with ||H_t||_F = 0 has x_t = 0 by definition: it contributes nothing and dq_t = 0.
    Shapes as gka_forward_ref (zero initial state); do: [B, T, H, D]. Returns a dict with dq,
    dk, dv [B, T, H, D], dgamma and dbeta [B, T, H].
    """
    q, k, v, do = (np.asarray(x, dtype=np.float64) for x in (q, k, v, do))
    gamma = np.asarray(gamma, dtype=np.float64)
    B, T, Hh, D = q.shape
    N = B * Hh

    def heads(x):
        return np.moveaxis(x, 2, 1).reshape((N, T) + x.shape[3:])

    qh, kh, vh, gh, dh = heads(q), heads(k), heads(v), heads(gamma), heads(do)
    bh = np.ones((N, T)) if beta is None else heads(np.asarray(beta, dtype=np.float64))
    # forward, keeping every state
    Hs = np.zeros((N, T + 1, D, D))  # Hs[:, t + 1] = H_t, Hs[:, 0] = the zero initial state
    Us = np.zeros((N, T + 1, D, D))
    for t in range(T):
        kk = kh[:, t, :, None] * kh[:, t, None, :]
        vk = vh[:, t, :, None] * kh[:, t, None, :]
        Hs[:, t + 1] = gh[:, t, None, None] * Hs[:, t] + bh[:, t, None, None] * kk
        Us[:, t + 1] = gh[:, t, None, None] * Us[:, t] + bh[:, t, None, None] * vk
    dq = np.zeros((N, T, D))
    G = np.zeros((N, T, D, D))
    W = np.zeros((N, T, D, D))
    eye = np.eye(D)
    for t in range(T):
        H, U = Hs[:, t + 1], Us[:, t + 1]
        n = np.linalg.norm(H, axis=(-2, -1))
        live = n > 0.0
        ns = np.where(live, n, 1.0)
        A = np.where(live[:, None, None], H + (a * ns)[:, None, None] * eye, eye)
        g = np.einsum("nij,ni->nj", U, dh[:, t])  # U^T do
        if mode == "cheb":
            mu, L = np.where(live, a * ns, 1.0), np.where(live, (1.0 + a) * ns, 1.0)
            x = chebyshev_solve(A, qh[:, t], mu, L, iters)
            y = chebyshev_solve(A, g, mu, L, iters)
        elif mode == "exact":
            x, y = cholesky_solve(A, qh[:, t]), cholesky_solve(A, g)
        else:
            raise ValueError(f"unknown mode {mode!r}")
        x = np.where(live[:, None], x, 0.0)
        y = np.where(live[:, None], y, 0.0)
        c = -a * np.einsum("ni,ni->n", y, x) / ns
        dq[:, t] = y
        G[:, t] = -y[:, :, None] * x[:, None, :] + c[:, None, None] * H
        W[:, t] = dh[:, t, :, None] * x[:, None, :]
    dk = np.zeros((N, T, D))
    dv = np.zeros((N, T, D))
    dgam = np.zeros((N, T))
    dbet = np.zeros((N, T))
    Gb = np.zeros((N, D, D))
    Wb = np.zeros((N, D, D))
    for t in range(T - 1, -1, -1):
        gn = gh[:, t + 1, None, None] if t + 1 < T else 0.0
        Gb = G[:, t] + gn * Gb
        Wb = W[:, t] + gn * Wb
        kt, vt = kh[:, t], vh[:, t]
        Gs = Gb + np.swapaxes(Gb, -1, -2)
        dk[:, t] = bh[:, t, None] * (np.einsum("nij,nj->ni", Gs, kt) + np.einsum("nij,ni->nj", Wb, vt))
        dv[:, t] = bh[:, t, None] * np.einsum("nij,nj->ni", Wb, kt)
        dbet[:, t] = np.einsum("ni,nij,nj->n", kt, Gb, kt) + np.einsum("ni,nij,nj->n", vt, Wb, kt)
        dgam[:, t] = np.einsum("nij,nij->n", Gb, Hs[:, t]) + np.einsum("nij,nij->n", Wb, Us[:, t])

    def unheads(x):
        return np.moveaxis(x.reshape((B, Hh, T) + x.shape[2:]), 1, 2)

    return dict(dq=unheads(dq), dk=unheads(dk), dv=unheads(dv), dgamma=unheads(dgam),
                dbeta=unheads(dbet))
