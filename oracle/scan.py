"""The linear recurrence that each Newton iteration solves (oracle; test infrastructure only).

d_t = A_t d_{t-1} + b_t with d_{-1} = 0 is forward substitution on the block
lower-bidiagonal system (ParaRNN overview, "Newton's Iteration": block
lower-triangular Jacobian, forward substitution).  Viewing each step as the affine
map e_t(d) = A_t d + b_t, composition (A2, b2) o (A1, b1) = (A2 A1, A2 b1 + b2) is
associative, which is what lets a parallel associative scan replace the loop (scime
summary of "Towards Scalable and Stable Parallelization of Nonlinear RNNs", "Builds
on": parallel associative scan).

``A`` is either dense [T, S, S] or diagonal [T, S]; ``b`` is [T, S].
"""
from __future__ import annotations

import numpy as np


def _apply(A, v):
    if A.ndim == v.ndim:          # diagonal: elementwise
        return A * v
    return np.einsum("...ij,...j->...i", A, v)


def compose(e2, e1):
    """(A2, b2) o (A1, b1) = (A2 A1, A2 b1 + b2): apply e1 first, then e2."""
    A2, b2 = e2
    A1, b1 = e1
    if A2.shape == b2.shape:      # diagonal elements
        return A2 * A1, A2 * b1 + b2
    return A2 @ A1, _apply(A2, b1) + b2


def scan_loop(A, b):
    """Sequential loop: returns d [T, S]."""
    T = b.shape[0]
    d = np.zeros_like(b)
    prev = np.zeros_like(b[0])
    for t in range(T):
        prev = _apply(A[t], prev) + b[t]
        d[t] = prev
    return d


def scan_doubling(A, b):
    """Recursive-doubling (Hillis-Steele) inclusive scan of affine maps: returns d [T, S].

    After the round with offset o, element t holds e_t o ... o e_{max(0, t-2o+1)}; the
    b-part of the full prefix applied to d_{-1} = 0 is d_t.
    """
    A = np.array(A, copy=True)
    b = np.array(b, copy=True)
    T = b.shape[0]
    o = 1
    while o < T:
        A_new = A.copy()
        b_new = b.copy()
        for t in range(o, T):
            A_new[t], b_new[t] = compose((A[t], b[t]), (A[t - o], b[t - o]))
        A, b = A_new, b_new
        o *= 2
    return b
