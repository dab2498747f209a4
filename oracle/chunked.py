"""Chunked Newton evaluation of a long sequence (oracle; test infrastructure only).

ParaRNN overview page, "Experimental Results" (long sequences): the memory that the
stored hidden states take during the Newton iteration is kept in check by chunking,
together with gradient checkpointing.

Reading (the page gives no procedure): the sequence is cut into consecutive chunks of
``chunk_len`` steps (the last may be shorter); chunk c is evaluated by the same Newton
iteration as a whole sequence (``newton_dense``, with the same max_iters, tol, Jacobian
options and damping, its stopping test shared by the batch), from the initial state h0
for the first chunk and from the returned state at the previous chunk's last step for
the others.  Aggregates: the worst status (non-finite > not converged > converged),
the sum of the chunks' iterations, the chunks' residual histories one after another;
after a non-finite chunk the later chunks are not evaluated (their states are left 0).
"""
from __future__ import annotations

import numpy as np

from .newton import STATUS_NONFINITE, STATUS_NOT_CONVERGED, STATUS_OK, newton_dense
from .sequential import project

_RANK = {STATUS_OK: 0, STATUS_NOT_CONVERGED: 1, STATUS_NONFINITE: 2}


def newton_chunked(cell: int, W, U, b_x, b_h, x, h0, max_iters: int, tol: float, jac_mode: int,
                   chunk_len: int, jac_every: int = 1, solver: str = "loop", damping: float = 0.0):
    """Returns dict(states [B,T,S], iters, status, rhos, chunks) -- ``chunks`` lists each
    chunk's (t0, length, iters, status)."""
    if chunk_len < 1:
        raise ValueError("chunk_len must be >= 1")
    gx = project(W, x, b_x)
    B, T, _ = gx.shape
    h0 = np.asarray(h0, dtype=np.float64)
    S = h0.shape[1]
    states = np.zeros((B, T, S))
    rhos, chunks = [], []
    iters, status = 0, STATUS_OK
    start = h0
    for t0 in range(0, T, chunk_len):
        t1 = min(T, t0 + chunk_len)
        r = newton_dense(cell, W, U, b_x, b_h, None, start, max_iters, tol, jac_mode, jac_every,
                         gx=gx[:, t0:t1], solver=solver, damping=damping)
        states[:, t0:t1] = r["states"]
        rhos += list(r["rhos"])
        iters += r["iters"]
        chunks.append((t0, t1 - t0, r["iters"], r["status"]))
        if _RANK[r["status"]] > _RANK[status]:
            status = r["status"]
        if r["status"] == STATUS_NONFINITE:
            break
        start = r["states"][:, -1]
    return dict(states=states, iters=iters, status=status, rhos=rhos, chunks=chunks)
