"""Low-rank approximation of the dense GRU's Jacobian (oracle; test infrastructure only).

ParaRNN overview page, "Technical Implementation / Newton's Iteration": to keep the cost
down at scale, the Newton iteration may use approximate Jacobians, recomputed only
every few steps or replaced by low-rank approximations.  The page gives no form; the
reading used here:

    J_t = diag(z) + diag(al) U_z + diag(be) U_r + diag(ga) U_n        (exact, oracle.cells)

keeps its structure, with each gate block U_g of the recurrent matrix replaced by its
best rank-r approximation (a truncated singular value decomposition, Eckart-Young)
whose diagonal is then reset to U_g's own, so that the Jacobian's diagonal stays exact:

    U~_g = sum_{i<r} s_i u_i v_i^T,    U^_g = U~_g - diag(U~_g) + diag(U_g)

The gates themselves are still computed from U.  r = D gives U^ = U (Newton, DEER); r = 0
gives a zero off-diagonal, i.e. the diagonal approximation (quasi-DEER).
"""
from __future__ import annotations

import numpy as np

from .cells import CELL_GRU


def truncated(Ug, rank: int):
    """Best rank-r approximation of one square block (library SVD)."""
    Ug = np.asarray(Ug, dtype=np.float64)
    u, sv, vt = np.linalg.svd(Ug)
    r = max(0, min(rank, len(sv)))
    return (u[:, :r] * sv[:r]) @ vt[:r]


def lowrank_matrix(cell: int, U, rank: int):
    """U^ [3D, D]: every gate block truncated to rank r, its diagonal reset to U's own."""
    if cell != CELL_GRU:
        raise ValueError("the low-rank Jacobian is defined for the GRU with a dense recurrent matrix")
    U = np.asarray(U, dtype=np.float64)
    D = U.shape[1]
    out = np.empty_like(U)
    for g in range(3):
        blk = U[g * D:(g + 1) * D]
        t = truncated(blk, rank)
        idx = np.arange(D)
        t[idx, idx] = blk[idx, idx]
        out[g * D:(g + 1) * D] = t
    return out
