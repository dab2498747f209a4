"""Pins of the oracle's low-rank Jacobian for the dense GRU (oracle.lowrank,
newton_dense(..., jac_rank=r)).

Fixed independently of the oracle's own code:
* Eckart-Young: the rank-r truncation of a block is exactly sigma_{r+1} away from it in
  the spectral norm and has rank r (a wrong ordering of the singular values, or a
  dropped factor, fails here);
* the two ends of the family: r = D is Newton with the exact Jacobian (autograd fixes
  that Jacobian, tests/test_oracle_cells.py), r = 0 is the diagonal approximation;
* the Jacobian's diagonal is the exact one at every rank;
* Newton's exact-prefix property (any Jacobian estimate: the first k states are exact
  after k updates) and the fixed point (the sequential trajectory).
"""
import numpy as np
import pytest
import torch

import oracle as O
from nonlinear_rnn_evaluation_amd import workloads as WL


def _problem(B=2, T=50, D=6, D_in=3, seed=0):
    p = WL.random_problem(WL.CELL_GRU, B, T, D, D_in, seed=seed, bias_std=0.3, h0_std=0.4)
    return {k: (None if v is None else WL.as_f64(v)) for k, v in p.items()}


@pytest.mark.parametrize("rank", [0, 1, 3, 5, 6])
def test_truncation_meets_eckart_young(rank):
    rng = np.random.default_rng(rank)
    A = rng.normal(size=(6, 6))
    t = O.truncated(A, rank)
    sv = np.linalg.svd(A, compute_uv=False)
    assert np.linalg.matrix_rank(t, tol=1e-10) == rank
    err = np.linalg.norm(A - t, 2)
    expect = sv[rank] if rank < 6 else 0.0
    assert abs(err - expect) < 1e-12


@pytest.mark.parametrize("rank", [0, 2, 6])
def test_lowrank_matrix_keeps_each_block_diagonal_and_truncates_the_rest(rank):
    q = _problem()
    D = 6
    Uh = O.lowrank_matrix(WL.CELL_GRU, q["U"], rank)
    for g in range(3):
        blk, hb = q["U"][g * D:(g + 1) * D], Uh[g * D:(g + 1) * D]
        assert np.array_equal(np.diag(blk), np.diag(hb))
        t = O.truncated(blk, rank)
        off = ~np.eye(D, dtype=bool)
        assert np.allclose(hb[off], t[off], atol=1e-14)


def test_full_rank_is_newton_and_rank_zero_is_the_diagonal_approximation():
    q = _problem()
    args = (WL.CELL_GRU, q["W"], q["U"], q["b_x"], q["b_h"], q["x"], q["h0"], 5, -1.0)
    full = O.newton_dense(*args, WL.JAC_FULL, solver="loop")
    diag = O.newton_dense(*args, WL.JAC_DIAG, solver="loop")
    r_full = O.newton_dense(*args, WL.JAC_FULL, solver="loop", jac_rank=6)
    r_zero = O.newton_dense(*args, WL.JAC_FULL, solver="loop", jac_rank=0)
    assert np.abs(r_full["states"] - full["states"]).max() < 1e-12
    assert np.allclose(r_full["rhos"], full["rhos"], rtol=1e-10, atol=1e-15)
    assert np.abs(r_zero["states"] - diag["states"]).max() < 1e-12


def test_lowrank_jacobian_diagonal_is_exact_and_full_rank_matches_autograd():
    q = _problem(B=1, T=1, D=5, D_in=2, seed=3)
    D = 5
    s = np.random.default_rng(4).normal(size=(1, D))
    gx = O.project(q["W"], q["x"][:, :1], q["b_x"])[0]
    Jx = O.cell_jacobian(WL.CELL_GRU, q["U"], q["b_h"], s, gx)
    for r in (0, 2, 5):
        Jr = O.cell_jacobian(WL.CELL_GRU, q["U"], q["b_h"], s, gx, U_jac=O.lowrank_matrix(WL.CELL_GRU, q["U"], r))
        assert np.allclose(np.diag(Jr[0]), np.diag(Jx[0]), atol=1e-14)
    # full rank against autograd on the torch GRU cell (the exact Jacobian)
    cell = torch.nn.GRUCell(2, D, bias=True).double()
    with torch.no_grad():
        cell.weight_ih.copy_(torch.from_numpy(q["W"]))
        cell.weight_hh.copy_(torch.from_numpy(q["U"]))
        cell.bias_ih.copy_(torch.from_numpy(q["b_x"]))
        cell.bias_hh.copy_(torch.from_numpy(q["b_h"]))
    xt = torch.from_numpy(q["x"][0, :1])
    Ja = torch.autograd.functional.jacobian(lambda h: cell(xt, h), torch.from_numpy(s)).reshape(D, D).numpy()
    Jr = O.cell_jacobian(WL.CELL_GRU, q["U"], q["b_h"], s, gx, U_jac=O.lowrank_matrix(WL.CELL_GRU, q["U"], D))
    assert np.abs(Jr[0] - Ja).max() < 1e-12


@pytest.mark.parametrize("rank", [1, 3])
@pytest.mark.parametrize("k", [1, 4, 9])
def test_exact_prefix_with_a_lowrank_jacobian(rank, k):
    q = _problem(T=40, seed=5)
    seq = O.sequential(WL.CELL_GRU, q["W"], q["U"], q["b_x"], q["b_h"], q["x"], q["h0"])
    r = O.newton_dense(WL.CELL_GRU, q["W"], q["U"], q["b_x"], q["b_h"], q["x"], q["h0"], k, -1.0, WL.JAC_FULL,
                       solver="loop", jac_rank=rank)
    assert np.abs(r["states"][:, :k] - seq[:, :k]).max() < 1e-12
    assert np.abs(r["states"][:, k:] - seq[:, k:]).max() > 1e-9   # not converged by accident


@pytest.mark.parametrize("rank", [0, 2, 4, 6])
def test_lowrank_newton_converges_to_the_sequential_trajectory(rank):
    q = _problem(T=80, seed=6)
    seq = O.sequential(WL.CELL_GRU, q["W"], q["U"], q["b_x"], q["b_h"], q["x"], q["h0"])
    r = O.newton_dense(WL.CELL_GRU, q["W"], q["U"], q["b_x"], q["b_h"], q["x"], q["h0"], 80, 1e-11, WL.JAC_FULL,
                       solver="loop", jac_rank=rank)
    assert r["status"] == O.STATUS_OK
    assert np.abs(r["states"] - seq).max() < 1e-9
