"""Damped (Levenberg-Marquardt) Newton steps for the unfolded recurrence -- ELK / quasi-ELK
(oracle; test infrastructure only).

[ELK] "Towards Scalable and Stable Parallelization of Nonlinear RNNs" (abstract; summary
page, "Approach" and "Limitations"): Newton's method on the unfolded recurrence is
stabilised with a Levenberg-Marquardt trust region whose linear-Gaussian MAP solve is a
Kalman filter and smoother; with the diagonal Jacobian the combination is quasi-ELK; the
trust-region strength is a hyperparameter to sweep.

Reading (the pages print no formula).  With the current iterate's residuals r_t and
Jacobian estimates J_t, the damped step D minimises

    sum_t |D_t - J_t D_{t-1} - r_t|^2 + lam * sum_t |D_t|^2,      D_0 = 0,

that is the Levenberg-Marquardt step (A^T A + lam I) D = A^T r for the block
lower-bidiagonal A of the Newton system (A D = r is the undamped step; lam = 0 gives
it back).  The same D is the smoothed mean of the linear-Gaussian state-space model

    D_t = J_t D_{t-1} + r_t + w_t,   w_t ~ N(0, I)        (dynamics)
    0   = D_t + v_t,                 v_t ~ N(0, I / lam)   (pseudo-observation)

computed by a Kalman filter forward and a Rauch-Tung-Striebel smoother backward.  Both
are implemented here, independently, so that each checks the other.  The step is always
accepted (no adaptive trust region), and the iteration stops on the same max-abs
residual test as the undamped one.
"""
from __future__ import annotations

import numpy as np


def _as_dense(J):
    """[T, S, S] from dense [T, S, S] or diagonal [T, S] Jacobians."""
    J = np.asarray(J, dtype=np.float64)
    if J.ndim == 2:
        T, S = J.shape
        out = np.zeros((T, S, S))
        idx = np.arange(S)
        out[:, idx, idx] = J
        return out
    return J


def lm_step_dense(J, r, lam: float):
    """The damped step by its definition: assemble A (identity blocks on the diagonal, -J_t
    below it), then solve (A^T A + lam I) D = A^T r with LAPACK.  J: [T, S, S] or [T, S];
    r: [T, S].  Returns D [T, S]."""
    J = _as_dense(J)
    r = np.asarray(r, dtype=np.float64)
    T, S = r.shape
    A = np.eye(T * S)
    for t in range(1, T):
        A[t * S:(t + 1) * S, (t - 1) * S:t * S] = -J[t]
    M = A.T @ A + lam * np.eye(T * S)
    return np.linalg.solve(M, A.T @ r.reshape(T * S)).reshape(T, S)


def lm_step_kalman(J, r, lam: float):
    """The damped step as a Kalman filter (prediction J P J^T + I, pseudo-observation 0
    with variance 1/lam) and an RTS smoother.  lam > 0.  Returns D [T, S]."""
    if lam <= 0:
        raise ValueError("the Kalman form needs lam > 0 (lam = 0 is the undamped step)")
    J = _as_dense(J)
    r = np.asarray(r, dtype=np.float64)
    T, S = r.shape
    I = np.eye(S)
    m = np.zeros(S)
    P = np.zeros((S, S))
    ms, Ps, mp, Pp = (np.zeros((T, S)), np.zeros((T, S, S)), np.zeros((T, S)), np.zeros((T, S, S)))
    for t in range(T):
        # the step before the first one is known exactly (D_0 = 0): J_0 never matters
        Pm = J[t] @ P @ J[t].T + I if t > 0 else I.copy()
        mm = J[t] @ m + r[t] if t > 0 else r[t].copy()
        K = lam * Pm @ np.linalg.inv(lam * Pm + I)
        m = (I - K) @ mm
        P = (I - K) @ Pm
        ms[t], Ps[t], mp[t], Pp[t] = m, P, mm, Pm
    D = np.zeros((T, S))
    D[T - 1] = ms[T - 1]
    for t in range(T - 2, -1, -1):
        G = Ps[t] @ J[t + 1].T @ np.linalg.inv(Pp[t + 1])
        D[t] = ms[t] + G @ (D[t + 1] - mp[t + 1])
    return D


def damped_step(J, r, lam: float, solver: str = "kalman"):
    """Damped step for one batch element ("kalman" or "dense"); lam = 0 is the Newton step."""
    if lam == 0:
        from .scan import scan_loop
        return scan_loop(np.asarray(J, dtype=np.float64), np.asarray(r, dtype=np.float64))
    if solver == "dense":
        return lm_step_dense(J, r, lam)
    if solver == "kalman":
        return lm_step_kalman(J, r, lam)
    raise ValueError(f"unknown solver {solver}")
