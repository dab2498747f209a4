"""Gradients through the evaluated sequence: backpropagation through time (oracle; test
infrastructure only).

Training through the parallel evaluation needs the gradients of a loss with respect to
the inputs, parameters and initial state ("Parallelizing non-linear sequential models
over the sequence length", abstract: training sequential models with the parallel
algorithm; scime summary of "Towards Scalable and Stable Parallelization of Nonlinear
RNNs", "Measured effects": the diagonal approximation also in the backward pass).  The
block lower-triangular system of the recurrence is solved backwards as well as forwards
(ParaRNN overview, "Newton's Iteration": forward and backward substitution): with
g_t = dL/ds_t the explicit loss gradient at each state, the adjoint obeys

    lam_t = g_t + J_{t+1}^T lam_{t+1},     lam_T = g_T,

a linear recurrence run backwards in time, and every parameter gradient is a sum over
steps of what lam_t sends back through the cell.  This module is the plain definition:
a sequential loop from the last step to the first, each step's vector-Jacobian product
written out from the cell equations of ``oracle.cells`` by the chain rule, in fp64.  It
is pinned by central finite differences of L = sum_t <g_t, s_t> (tests).

Layouts follow the library: x [B, T, D_in], W [G*D, D_in], U (GRU [3D, D]; diagonal
cells [G, D]), b_x and b_h [G*D], h0 [B, S], states and g [B, T, S].
"""
from __future__ import annotations

import numpy as np

from .cells import CELL_GRU, CELL_GRU_DIAG, CELL_LSTM_DIAG, JAC_DIAG, JAC_FULL, _recurrent, _sigmoid, cell_jacobian
from .sequential import project


def cell_vjp(cell: int, U, b_h, s, gx, lam):
    """One step's vector-Jacobian products at previous states s [N, S] and inputs gx
    [N, G*D], for lam [N, S] = dL/ds' (total): returns (dprev [N, S] = (ds'/ds)^T lam,
    dgx [N, G*D] = dL/d(pre-activations), dgh [N, G*D] = dL/d(U s + b_h))."""
    one = 1.0
    if cell in (CELL_GRU, CELL_GRU_DIAG):
        D = s.shape[1]
        gh = _recurrent(cell, U, b_h, s)
        r = _sigmoid(gx[:, :D] + gh[:, :D])
        z = _sigmoid(gx[:, D:2 * D] + gh[:, D:2 * D])
        ghn = gh[:, 2 * D:]
        n = np.tanh(gx[:, 2 * D:] + r * ghn)
        # h' = (1 - z) n + z h
        dn = lam * (one - z)
        da_n = dn * (one - n * n)              # n = tanh(a_n), a_n = gx_n + r gh_n
        da_z = lam * (s - n) * z * (one - z)   # z = sigmoid(a_z)
        da_r = da_n * ghn * r * (one - r)      # r enters a_n through r gh_n
        dgx = np.concatenate([da_r, da_z, da_n], axis=1)
        dgh = np.concatenate([da_r, da_z, da_n * r], axis=1)
        if cell == CELL_GRU:
            dprev = lam * z + dgh @ U
        else:
            dprev = lam * z + (dgh.reshape(-1, 3, D) * U[None]).sum(axis=1)
        return dprev, dgx, dgh
    if cell == CELL_LSTM_DIAG:
        D = s.shape[1] // 2
        c, h = s[:, :D], s[:, D:]
        a = gx + _recurrent(cell, U, b_h, h)
        i, f, o = _sigmoid(a[:, :D]), _sigmoid(a[:, D:2 * D]), _sigmoid(a[:, 2 * D:3 * D])
        g = np.tanh(a[:, 3 * D:])
        tau = np.tanh(f * c + i * g)
        lc, lh = lam[:, :D], lam[:, D:]
        # c' = f c + i g,  h' = o tanh(c'): c' is reached directly and through h'
        dcn = lc + lh * o * (one - tau * tau)
        da = np.concatenate([dcn * g * i * (one - i), dcn * c * f * (one - f), lh * tau * o * (one - o),
                             dcn * i * (one - g * g)], axis=1)
        dh = (da.reshape(-1, 4, D) * U[None]).sum(axis=1)
        return np.concatenate([dcn * f, dh], axis=1), da, da
    raise ValueError(f"unknown cell {cell}")


def bptt(cell: int, W, U, b_x, b_h, x, h0, states, g, jac_mode: int = JAC_FULL):
    """Gradients of L = sum_{b,t} <g[b,t], states[b,t]> where states solve the recurrence
    from h0 (the states are taken as given: the converged evaluation).  Returns dict(dx,
    dW, dU, db_x, db_h, dh0, dgx [B, T, G*D], lam [B, T, S]).

    jac_mode = JAC_DIAG is the diagonal approximation in the backward pass ("Towards
    Scalable and Stable Parallelization of Nonlinear RNNs", summary page, "Measured
    effects": diagonal Jacobians "including in the backward pass"): the adjoint recursion
    carries diag(J_{t+1}) * lam_{t+1} instead of J_{t+1}^T lam_{t+1} (dh0 likewise), while
    every step still sends its lam_t back through the cell's gates exactly.  With a
    diagonal Jacobian (GRU_DIAG) it is the exact gradient."""
    W = np.asarray(W, dtype=np.float64)
    U = np.asarray(U, dtype=np.float64)
    x = np.asarray(x, dtype=np.float64)
    h0 = np.asarray(h0, dtype=np.float64)
    H = np.asarray(states, dtype=np.float64)
    g = np.asarray(g, dtype=np.float64)
    gx = project(W, x, b_x)
    B, T, S = H.shape
    GD = gx.shape[2]
    dgx = np.zeros((B, T, GD))
    lam_all = np.zeros((B, T, S))
    dU = np.zeros_like(U)
    db_h = np.zeros(GD)
    carry = np.zeros((B, S))                     # J_{t+1}^T lam_{t+1}
    for t in range(T - 1, -1, -1):
        lam = g[:, t] + carry
        prev = H[:, t - 1] if t > 0 else h0
        dprev, dgx_t, dgh = cell_vjp(cell, U, b_h, prev, gx[:, t], lam)
        lam_all[:, t] = lam
        dgx[:, t] = dgx_t
        db_h += dgh.sum(axis=0)
        if cell == CELL_GRU:
            dU += dgh.T @ prev                   # gh = U h: dU[m, j] = sum dgh[m] h[j]
        elif cell == CELL_GRU_DIAG:
            dU += (dgh.reshape(B, 3, S) * prev[:, None, :]).sum(axis=0)
        else:
            D = S // 2
            dU += (dgh.reshape(B, 4, D) * prev[:, None, D:]).sum(axis=0)
        if jac_mode == JAC_DIAG:
            J = cell_jacobian(cell, U, b_h, prev, gx[:, t])
            carry = np.einsum("nii->ni", J) * lam
        else:
            carry = dprev
    flat = dgx.reshape(B * T, GD)
    return dict(dx=(flat @ W).reshape(B, T, -1), dW=flat.T @ x.reshape(B * T, -1), dU=dU,
                db_x=flat.sum(axis=0), db_h=db_h, dh0=carry, dgx=dgx, lam=lam_all)
