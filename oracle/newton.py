"""Naive Newton evaluation with a dense block-bidiagonal solve (oracle; test infrastructure only).

The T-step recurrence is unfolded into one system of equations, one per timestep's
state (ParaRNN overview, "Core Idea"; DEER poses the states as the solution of a
fixed-point problem, "Towards Scalable and Stable Parallelization of Nonlinear
RNNs", abstract):

    R_t(H) = f(H_{t-1}, x_t) - H_t = 0,   t = 1..T,   H_0 = h0.

Each Newton iteration computes the residual and the Jacobian at every step, then
solves the linearised system (ParaRNN overview, "Core Idea" step 2 and "Newton's
Iteration").  The system matrix is block lower-bidiagonal: identity blocks on the
diagonal and -J_t = -df(H_{t-1}, x_t)/dH_{t-1} just below it, because each step
depends only on its input and the previous state.  Here it is assembled densely
(T*S x T*S per batch element) and handed to LAPACK -- slow on purpose, so that the
HIP path's scan has an independent check.

Options:
* jac_mode: FULL (exact Jacobian), DIAG (its diagonal: quasi-DEER), ZERO (no
  Jacobian; a fixed-point sweep, test only).
* jac_every: the Jacobian is recomputed only when k % jac_every == 0 and reused
  otherwise (ParaRNN overview, "Newton's Iteration": recomputing the Jacobian only
  every few steps).  The residual is always fresh.
* refresh_ratio = theta >= 0 (adaptive refresh: the ParaRNN overview, "Newton's
  Iteration", names recomputing the Jacobian only every few steps; choosing when by the
  residual is this reading's own rule, not the page's): the Jacobian is also recomputed
  at iteration k >= 2 when the update before last contracted the residual by less than
  theta, rho_{k-1} > theta rho_{k-2};
  jac_every is then the largest age (k - last refresh) a Jacobian may reach.  The rule
  looks one update back because a fused pass must take its Jacobian before it learns
  its own residual.  theta = inf gives the fixed schedule, theta = 0 refreshes at every
  k >= 2.

* bounded = True (a safeguard of this reading's own, not the pages': "Towards Scalable and
  Stable Parallelization of Nonlinear RNNs", abstract and summary "Problem", says
  undamped Newton can be numerically unstable and diverge): after each update the new
  iterate is projected onto the box that every state of the recurrence lies in
  (``state_bounds``), and a component the step made NaN keeps its previous value.  The
  true states lie inside the box, so the projection never moves them: the exact-prefix
  property below still holds, and so does the fixed point.

* jac_rank = r (dense GRU): the Jacobian's recurrent-matrix factors are the rank-r
  truncations of ``oracle.lowrank`` (with jac_mode FULL; r = D is Newton, r = 0 the
  diagonal approximation).

Readings where the pages are silent: initial guess H = 0; stop when the max-abs
residual (NaN counted as +inf) is <= tol, testing *before* each update so the
returned iterate is the one whose residual was checked; one shared loop for all
batch elements; tol < 0 never stops early.
"""
from __future__ import annotations

import numpy as np

from .cells import CELL_LSTM_DIAG, approx_jacobian, cell_jacobian, cell_step
from .damped import damped_step
from .lowrank import lowrank_matrix
from .scan import scan_loop
from .sequential import project

STATUS_OK = 0
STATUS_NOT_CONVERGED = 1
STATUS_NONFINITE = 2


def max_abs(r) -> float:
    """max |r| over all entries; any NaN makes it +inf; an empty array gives 0."""
    a = np.abs(np.asarray(r, dtype=np.float64))
    if a.size == 0:
        return 0.0
    if np.isnan(a).any():
        return float("inf")
    return float(a.max())


def state_bounds(cell: int, h0, T: int):
    """Bounds [B, T, S] with |s_t| <= bound for every state s_1..s_T the recurrence can reach
    from h0, per component.

    GRU cells: h' = (1 - z) n + z h is a convex combination of n (|n| < 1, a tanh) and h, so
    |h'_i| <= max(1, |h_i|) <= max(1, |h0_i|).  LSTM: h' = o tanh(c') with 0 < o < 1, so
    |h'| < 1; c' = f c + i g with 0 < f, i < 1 and |g| < 1, so |c'| < |c| + 1 and
    |c_t| < |c0| + t.
    """
    h0 = np.asarray(h0, dtype=np.float64)
    B, S = h0.shape
    if cell == CELL_LSTM_DIAG:
        D = S // 2
        t = np.arange(1, T + 1, dtype=np.float64)[None, :, None]
        c = np.abs(h0[:, None, :D]) + t
        h = np.ones((B, T, D))
        return np.concatenate([c, h], axis=2)
    return np.broadcast_to(np.maximum(1.0, np.abs(h0))[:, None, :], (B, T, S)).copy()


def project_states(cell: int, h0, H_new, H_old):
    """The projected update: NaN components keep their previous value, then every component
    is clipped to its state bound."""
    H = np.where(np.isnan(H_new), H_old, H_new)
    bound = state_bounds(cell, h0, H.shape[1])
    return np.clip(H, -bound, bound)


def _previous_states(h0, H):
    """P_t = H_{t-1} (with H_0 = h0) for every step: [B, T, S]."""
    return np.concatenate([h0[:, None, :], H[:, :-1, :]], axis=1)


def newton_dense(cell: int, W, U, b_x, b_h, x, h0, max_iters: int, tol: float,
                 jac_mode: int, jac_every: int = 1, gx=None, solver: str = "dense",
                 damping: float = 0.0, refresh_ratio=None, bounded: bool = False, jac_rank=None):
    """Returns dict(states [B,T,S], iters, status, rhos[list], jac_evals, refreshes[list
    of the iterations that recomputed the Jacobian]).

    solver="dense" assembles the block-bidiagonal matrix and calls LAPACK (only for
    T*S up to a few thousand); solver="loop" solves the same system by forward
    substitution (``scan_loop``), which the tests pin to the dense solve.

    damping = lam > 0 takes the damped (Levenberg-Marquardt / ELK) step of
    ``oracle.damped`` instead: solver="dense" solves its normal equations with LAPACK,
    solver="loop" runs the Kalman filter and smoother.
    """
    if jac_every < 1:
        raise ValueError("jac_every must be >= 1")
    if refresh_ratio is not None and not refresh_ratio >= 0:
        raise ValueError("refresh_ratio must be >= 0 (or None)")
    U = np.asarray(U, dtype=np.float64)
    b_h = None if b_h is None else np.asarray(b_h, dtype=np.float64)
    h0 = np.asarray(h0, dtype=np.float64)
    if gx is None:
        gx = project(W, x, b_x)
    B, T, GD = gx.shape
    S = h0.shape[1]
    U_jac = None if jac_rank is None else lowrank_matrix(cell, U, jac_rank)
    H = np.zeros((B, T, S))
    rhos = []
    Jhat = None
    jac_evals = 0
    refreshes = []
    k = 0
    while True:
        P = _previous_states(h0, H)
        F = cell_step(cell, U, b_h, P.reshape(B * T, S), gx.reshape(B * T, GD)).reshape(B, T, S)
        r = F - H
        rho = max_abs(r)
        rhos.append(rho)
        if not np.isfinite(rho):
            return dict(states=H, iters=k, status=STATUS_NONFINITE, rhos=rhos, jac_evals=jac_evals,
                        refreshes=refreshes)
        if rho <= tol:
            return dict(states=H, iters=k, status=STATUS_OK, rhos=rhos, jac_evals=jac_evals,
                        refreshes=refreshes)
        if k == max_iters:
            return dict(states=H, iters=k, status=STATUS_NOT_CONVERGED, rhos=rhos,
                        jac_evals=jac_evals, refreshes=refreshes)
        aged = not refreshes or k - refreshes[-1] >= jac_every
        slow = refresh_ratio is not None and k >= 2 and rhos[k - 1] > refresh_ratio * rhos[k - 2]
        if aged or slow:
            refreshes.append(k)
            J = cell_jacobian(cell, U, b_h, P.reshape(B * T, S), gx.reshape(B * T, GD), U_jac=U_jac)
            Jhat = approx_jacobian(J, jac_mode).reshape(B, T, S, S)
            jac_evals += 1
        Hn = np.empty_like(H)
        with np.errstate(over="ignore", invalid="ignore"):
            for b in range(B):
                if damping > 0:
                    Hn[b] = H[b] + damped_step(Jhat[b], r[b], damping, "dense" if solver == "dense" else "kalman")
                    continue
                if solver == "loop":
                    Hn[b] = H[b] + scan_loop(Jhat[b], r[b])
                    continue
                A = np.eye(T * S)
                for t in range(1, T):
                    A[t * S:(t + 1) * S, (t - 1) * S:t * S] = -Jhat[b, t]
                delta = np.linalg.solve(A, r[b].reshape(T * S))
                Hn[b] = H[b] + delta.reshape(T, S)
        H = project_states(cell, h0, Hn, H) if bounded else Hn
        k += 1
