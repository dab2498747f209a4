"""Cells and their exact Jacobians (oracle; test infrastructure only).

The pages name GRU and LSTM cells and ParaRNN's "adaptations" of them (ParaRNN
overview, "Experimental Results"; Danieli talk, "Abstract") but print no equations.
Readings used here:

* GRU (dense recurrent matrix U, gate blocks r, z, n, "linear before reset"):
    gh = U h + b_h
    r = sigmoid(gx_r + gh_r),  z = sigmoid(gx_z + gh_z)
    n = tanh(gx_n + r * gh_n)
    h' = (1 - z) * n + z * h
  This is the form in which the recurrent product for all three gates is one
  contraction that does not depend on r.
* GRU with elementwise recurrent weights (diagonal recurrence): U = diag(u_g) per
  gate, so gh_g = u_g * h + b_hg; otherwise identical.
* LSTM with elementwise recurrent weights, gate blocks (i, f, o, g), state s = (c, h):
    a_k = gx_k + u_k * h + b_hk
    i, f, o = sigmoid(a_i), sigmoid(a_f), sigmoid(a_o);  g = tanh(a_g)
    c' = f * c + i * g;   h' = o * tanh(c')

The Jacobian of the step map with respect to the previous state is derived below by
the chain rule (each Newton iteration evaluates it at every step; ParaRNN overview,
"Technical Implementation / Newton's Iteration").  ``approx_jacobian`` applies the
quasi-Newton diagonal approximation ("Towards Scalable and Stable Parallelization of
Nonlinear RNNs", abstract; scime summary, "Approach") or drops the Jacobian entirely
(a Picard/Jacobi fixed-point sweep, used only as a test mode).

All functions work on batched rows: ``h`` is [N, S], ``gx`` is [N, G*D]; they keep the
dtype of their inputs (float64 for the oracle, float32 for the conditioning floor).
"""
from __future__ import annotations

import numpy as np

CELL_GRU = 0
CELL_GRU_DIAG = 1
CELL_LSTM_DIAG = 2

JAC_FULL = 0
JAC_DIAG = 1
JAC_ZERO = 2


def gates_of(cell: int) -> int:
    return 4 if cell == CELL_LSTM_DIAG else 3


def state_size(cell: int, D: int) -> int:
    return 2 * D if cell == CELL_LSTM_DIAG else D


def _sigmoid(a):
    one = a.dtype.type(1)
    return one / (one + np.exp(-a))


def _recurrent(cell, U, b_h, h):
    """gh = U h + b_h for every gate block: [N, G*D]."""
    if cell == CELL_GRU:
        gh = h @ U.T
    else:
        G, D = U.shape
        gh = (h[:, None, :] * U[None, :, :]).reshape(h.shape[0], G * D)
    if b_h is not None:
        gh = gh + b_h
    return gh


def _gru_parts(cell, U, b_h, h, gx):
    D = h.shape[1]
    gh = _recurrent(cell, U, b_h, h)
    r = _sigmoid(gx[:, 0:D] + gh[:, 0:D])
    z = _sigmoid(gx[:, D:2 * D] + gh[:, D:2 * D])
    ghn = gh[:, 2 * D:3 * D]
    n = np.tanh(gx[:, 2 * D:3 * D] + r * ghn)
    return r, z, n, ghn


def _lstm_parts(U, b_h, s, gx):
    D = s.shape[1] // 2
    c, h = s[:, :D], s[:, D:]
    a = gx + _recurrent(CELL_LSTM_DIAG, U, b_h, h)
    i = _sigmoid(a[:, 0:D])
    f = _sigmoid(a[:, D:2 * D])
    o = _sigmoid(a[:, 2 * D:3 * D])
    g = np.tanh(a[:, 3 * D:4 * D])
    c_new = f * c + i * g
    tau = np.tanh(c_new)
    return c, h, i, f, o, g, c_new, tau


def cell_step(cell: int, U, b_h, s, gx):
    """One step of the recurrence: s' = f(s, gx) for every row.  s [N, S], gx [N, G*D]."""
    if cell in (CELL_GRU, CELL_GRU_DIAG):
        r, z, n, _ = _gru_parts(cell, U, b_h, s, gx)
        one = s.dtype.type(1)
        return (one - z) * n + z * s
    if cell == CELL_LSTM_DIAG:
        _, _, _, _, o, _, c_new, tau = _lstm_parts(U, b_h, s, gx)
        return np.concatenate([c_new, o * tau], axis=1)
    raise ValueError(f"unknown cell {cell}")


def cell_jacobian(cell: int, U, b_h, s, gx, U_jac=None):
    """Exact Jacobian d f(s, gx) / d s as dense [N, S, S] (row = output component).

    U_jac (dense GRU only): take the Jacobian's matrix factors from U_jac instead of U,
    with the gates still computed from U -- the low-rank approximation of
    ``oracle.lowrank``; U_jac = U is the exact Jacobian."""
    N, S = s.shape
    one = s.dtype.type(1)
    if cell in (CELL_GRU, CELL_GRU_DIAG):
        D = S
        r, z, n, ghn = _gru_parts(cell, U, b_h, s, gx)
        # d h'/d h = diag(z) + diag(h - n) dz/dh + diag(1 - z) dn/dh
        #   dz/dh = diag(z (1 - z)) U_z
        #   dn/dh = diag(1 - n^2) [diag(r) U_n + diag(ghn) dr/dh],  dr/dh = diag(r (1 - r)) U_r
        cz = (s - n) * z * (one - z)
        cn = (one - z) * (one - n * n)
        if cell == CELL_GRU:
            Um = U if U_jac is None else np.asarray(U_jac, dtype=s.dtype)
            Ur, Uz, Un = Um[0:D], Um[D:2 * D], Um[2 * D:3 * D]
        else:
            Ur, Uz, Un = np.diag(U[0]), np.diag(U[1]), np.diag(U[2])
        J = (cz[:, :, None] * Uz[None]
             + (cn * r)[:, :, None] * Un[None]
             + (cn * ghn * r * (one - r))[:, :, None] * Ur[None])
        J = J + z[:, :, None] * np.eye(D, dtype=s.dtype)[None]
        return J
    if cell == CELL_LSTM_DIAG:
        D = S // 2
        c, h, i, f, o, g, c_new, tau = _lstm_parts(U, b_h, s, gx)
        ui, uf, uo, ug = U[0], U[1], U[2], U[3]
        # c' = f c + i g: d c'/d c = f;  d c'/d h = c f(1-f) u_f + g i(1-i) u_i + i (1-g^2) u_g
        kappa = c * f * (one - f) * uf + g * i * (one - i) * ui + i * (one - g * g) * ug
        # h' = o tanh(c'): d h'/d c = o (1 - tau^2) f;
        #                  d h'/d h = tau o(1-o) u_o + o (1 - tau^2) kappa
        dtau = o * (one - tau * tau)
        J = np.zeros((N, S, S), dtype=s.dtype)
        idx = np.arange(D)
        J[:, idx, idx] = f
        J[:, idx, D + idx] = kappa
        J[:, D + idx, idx] = dtau * f
        J[:, D + idx, D + idx] = tau * o * (one - o) * uo + dtau * kappa
        return J
    raise ValueError(f"unknown cell {cell}")


def approx_jacobian(J, mode: int):
    """Apply a Jacobian mode to exact dense Jacobians [N, S, S].

    FULL keeps J; DIAG keeps its diagonal (quasi-DEER); ZERO drops it (fixed-point sweep).
    """
    if mode == JAC_FULL:
        return J
    if mode == JAC_DIAG:
        d = np.diagonal(J, axis1=1, axis2=2)
        out = np.zeros_like(J)
        idx = np.arange(J.shape[1])
        out[:, idx, idx] = d
        return out
    if mode == JAC_ZERO:
        return np.zeros_like(J)
    raise ValueError(f"unknown jac mode {mode}")
