"""Sequential evaluation: the plain definition of what the parallel methods compute.

Oracle; test infrastructure only.  The recurrence s_t = f(s_{t-1}, x_t) is evaluated
one step after another (the "naive sequential application" baseline of the Danieli
talk abstract; the sequential evaluation baseline of "Towards Scalable and Stable
Parallelization of Nonlinear RNNs").  Parallel Newton methods converge to exactly
these states ("Parallelizing non-linear sequential models over the sequence length",
abstract).

Output convention: ``states[:, t]`` is s_{t+1}, the state after consuming x_t; h0 is
not part of the output.
"""
from __future__ import annotations

import numpy as np

from .cells import CELL_GRU, CELL_GRU_DIAG, CELL_LSTM_DIAG, cell_step, gates_of


def project(W, x, b_x=None, t_chunk: int = 4096, dtype=np.float64):
    """Input projection gx[b, t, :] = W x[b, t] + b_x, computed in ``dtype``.

    Each timestep depends only on its own input and the previous state (ParaRNN
    overview, "Newton's Iteration"), so this product is taken once for all steps.  A
    library matrix product does the arithmetic; chunking over T bounds memory.
    """
    W = np.asarray(W, dtype=dtype)
    B, T, _ = x.shape
    out = np.empty((B, T, W.shape[0]), dtype=dtype)
    for t0 in range(0, T, t_chunk):
        xs = np.asarray(x[:, t0:t0 + t_chunk], dtype=dtype)
        out[:, t0:t0 + t_chunk] = xs @ W.T
    if b_x is not None:
        out += np.asarray(b_x, dtype=dtype)
    return out


def sequential(cell: int, W, U, b_x, b_h, x, h0, dtype=np.float64, gx=None):
    """States [B, T, S] of the recurrence, one step at a time, in ``dtype``."""
    U = np.asarray(U, dtype=dtype)
    b_h = None if b_h is None else np.asarray(b_h, dtype=dtype)
    if gx is None:
        gx = project(W, x, b_x, dtype=dtype)
    B, T = gx.shape[:2]
    s = np.array(h0, dtype=dtype, copy=True)
    out = np.empty((B, T, s.shape[1]), dtype=dtype)
    for t in range(T):
        s = cell_step(cell, U, b_h, s, gx[:, t])
        out[:, t] = s
    return out


def restrict_channels(cell: int, D: int, W, U, b_x, b_h, h0, channels):
    """Sub-problem made of a subset of channels of a diagonal-recurrence cell.

    With elementwise recurrent weights a channel's gates read only that channel's
    state, so the trajectory of a channel subset is the trajectory of the sub-problem
    built from those channels' rows of W, u, the biases and h0.  Used to check very
    large workloads on sampled channels.  Returns (W, U, b_x, b_h, h0, D_sub).
    """
    if cell not in (CELL_GRU_DIAG, CELL_LSTM_DIAG):
        raise ValueError("only diagonal-recurrence cells decouple channels")
    ch = np.asarray(channels)
    G = gates_of(cell)
    rows = (np.arange(G)[:, None] * D + ch[None, :]).reshape(-1)
    Wc = W[rows]
    Uc = U[:, ch]
    bxc = None if b_x is None else b_x[rows]
    bhc = None if b_h is None else b_h[rows]
    if cell == CELL_LSTM_DIAG:
        h0c = np.concatenate([h0[:, ch], h0[:, D + ch]], axis=1)
    else:
        h0c = h0[:, ch]
    return Wc, Uc, bxc, bhc, h0c, len(ch)


def output_channel_columns(cell: int, D: int, channels):
    """Columns of the full [.., S] state that a channel subset occupies (c then h for LSTM)."""
    ch = np.asarray(channels)
    if cell == CELL_LSTM_DIAG:
        return np.concatenate([ch, D + ch])
    if cell == CELL_GRU:
        raise ValueError("dense GRU channels are coupled")
    return ch
