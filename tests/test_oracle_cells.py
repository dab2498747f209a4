"""Pins for the oracle's cells and Jacobians (CPU).

The pages print no cell equations, so the cells are pinned to independent library
implementations: torch's GRUCell / LSTMCell (fp64) for the step maps, torch autograd
for the Jacobians, and central finite differences as brute force.
"""
import numpy as np
import pytest
import torch

import oracle as O




def _rand(rng, *shape, scale=1.0):
    return rng.normal(0.0, scale, size=shape)


def _gru_torch(W, U_dense, b_x, b_h):
    D = U_dense.shape[1]
    cell = torch.nn.GRUCell(W.shape[1], D, bias=True, dtype=torch.float64)
    with torch.no_grad():
        cell.weight_ih.copy_(torch.from_numpy(W))
        cell.weight_hh.copy_(torch.from_numpy(U_dense))
        cell.bias_ih.copy_(torch.from_numpy(b_x))
        cell.bias_hh.copy_(torch.from_numpy(b_h))
    return cell


def _diag_stack(u):
    return np.concatenate([np.diag(row) for row in u], axis=0)


LSTM_PERM = [0, 1, 3, 2]   # torch blocks (i, f, g, o) taken from ours (i, f, o, g)


def _blocks(a, D, perm):
    return np.concatenate([a[p * D:(p + 1) * D] for p in perm], axis=0)


def _lstm_torch(W, u, b_x, b_h):
    G, D = u.shape
    cell = torch.nn.LSTMCell(W.shape[1], D, bias=True, dtype=torch.float64)
    with torch.no_grad():
        cell.weight_ih.copy_(torch.from_numpy(_blocks(W, D, LSTM_PERM)))
        cell.weight_hh.copy_(torch.from_numpy(_blocks(_diag_stack(u), D, LSTM_PERM)))
        cell.bias_ih.copy_(torch.from_numpy(_blocks(b_x, D, LSTM_PERM)))
        cell.bias_hh.copy_(torch.from_numpy(_blocks(b_h, D, LSTM_PERM)))
    return cell


@pytest.mark.parametrize("D,D_in", [(4, 2), (7, 5), (16, 16)])
def test_gru_step_matches_torch_grucell(D, D_in):
    rng = np.random.default_rng(1)
    W, U = _rand(rng, 3 * D, D_in, scale=0.7), _rand(rng, 3 * D, D, scale=0.7)
    b_x, b_h = _rand(rng, 3 * D, scale=0.3), _rand(rng, 3 * D, scale=0.3)
    x, h = _rand(rng, 9, D_in), _rand(rng, 9, D, scale=0.8)
    ref = _gru_torch(W, U, b_x, b_h)(torch.from_numpy(x), torch.from_numpy(h)).detach().numpy()
    gx = x @ W.T + b_x
    got = O.cell_step(O.CELL_GRU, U, b_h, h, gx)
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-14)


def test_gru_diag_step_matches_grucell_with_diagonal_recurrence():
    rng = np.random.default_rng(2)
    D, D_in = 6, 3
    W, u = _rand(rng, 3 * D, D_in), rng.uniform(-1, 1, size=(3, D))
    b_x, b_h = _rand(rng, 3 * D, scale=0.3), _rand(rng, 3 * D, scale=0.3)
    x, h = _rand(rng, 5, D_in), _rand(rng, 5, D)
    ref = _gru_torch(W, _diag_stack(u), b_x, b_h)(torch.from_numpy(x), torch.from_numpy(h))
    got = O.cell_step(O.CELL_GRU_DIAG, u, b_h, h, x @ W.T + b_x)
    np.testing.assert_allclose(got, ref.detach().numpy(), rtol=0, atol=1e-14)


def test_lstm_diag_step_matches_lstmcell_with_diagonal_recurrence():
    rng = np.random.default_rng(3)
    D, D_in = 5, 4
    W, u = _rand(rng, 4 * D, D_in), rng.uniform(-1, 1, size=(4, D))
    b_x, b_h = _rand(rng, 4 * D, scale=0.3), _rand(rng, 4 * D, scale=0.3)
    x = _rand(rng, 7, D_in)
    c, h = _rand(rng, 7, D), _rand(rng, 7, D)
    h_t, c_t = _lstm_torch(W, u, b_x, b_h)(torch.from_numpy(x), (torch.from_numpy(h), torch.from_numpy(c)))
    got = O.cell_step(O.CELL_LSTM_DIAG, u, b_h, np.concatenate([c, h], 1), x @ W.T + b_x)
    np.testing.assert_allclose(got[:, :D], c_t.detach().numpy(), rtol=0, atol=1e-14)
    np.testing.assert_allclose(got[:, D:], h_t.detach().numpy(), rtol=0, atol=1e-14)


def _autograd_jac(fn, s):
    J = torch.autograd.functional.jacobian(fn, torch.from_numpy(s))
    return J.detach().numpy()


@pytest.mark.parametrize("cell", [O.CELL_GRU, O.CELL_GRU_DIAG, O.CELL_LSTM_DIAG])
def test_jacobian_matches_autograd_of_torch_cells(cell):
    rng = np.random.default_rng(4 + cell)
    D, D_in = 5, 3
    G = O.gates_of(cell)
    S = O.state_size(cell, D)
    W = _rand(rng, G * D, D_in)
    U = _rand(rng, G * D, D) if cell == O.CELL_GRU else rng.uniform(-1, 1, size=(G, D))
    b_x, b_h = _rand(rng, G * D, scale=0.3), _rand(rng, G * D, scale=0.3)
    x = _rand(rng, 1, D_in)
    s = _rand(rng, 1, S, scale=0.7)
    J = O.cell_jacobian(cell, U, b_h, s, x @ W.T + b_x)[0]
    xt = torch.from_numpy(x)
    if cell == O.CELL_LSTM_DIAG:
        tc = _lstm_torch(W, U, b_x, b_h)

        def fn(st):
            h_new, c_new = tc(xt, (st[:, D:], st[:, :D]))
            return torch.cat([c_new, h_new], 1)
    else:
        Ud = U if cell == O.CELL_GRU else _diag_stack(U)
        tc = _gru_torch(W, Ud, b_x, b_h)

        def fn(st):
            return tc(xt, st)
    ref = _autograd_jac(fn, s)[0, :, 0, :]
    np.testing.assert_allclose(J, ref, rtol=0, atol=1e-14)


@pytest.mark.parametrize("cell", [O.CELL_GRU, O.CELL_GRU_DIAG, O.CELL_LSTM_DIAG])
def test_jacobian_matches_central_differences(cell):
    rng = np.random.default_rng(10 + cell)
    D = 4
    G = O.gates_of(cell)
    S = O.state_size(cell, D)
    U = _rand(rng, G * D, D) if cell == O.CELL_GRU else rng.uniform(-1, 1, size=(G, D))
    b_h = _rand(rng, G * D, scale=0.3)
    gx = _rand(rng, 3, G * D)
    s = _rand(rng, 3, S, scale=0.7)
    J = O.cell_jacobian(cell, U, b_h, s, gx)
    eps = 1e-6
    for j in range(S):
        e = np.zeros(S)
        e[j] = eps
        col = (O.cell_step(cell, U, b_h, s + e, gx) - O.cell_step(cell, U, b_h, s - e, gx)) / (2 * eps)
        np.testing.assert_allclose(J[:, :, j], col, rtol=0, atol=1e-8)


def test_diagonal_cells_have_no_channel_mixing():
    """Elementwise recurrence: exact GRU_DIAG Jacobian is diagonal; LSTM's is 2x2 per channel."""
    rng = np.random.default_rng(20)
    D = 6
    gx = _rand(rng, 2, 3 * D)
    s = _rand(rng, 2, D)
    J = O.cell_jacobian(O.CELL_GRU_DIAG, rng.uniform(-1, 1, (3, D)), None, s, gx)
    off = J - np.einsum("nii->ni", J)[:, :, None] * np.eye(D)
    assert np.abs(off).max() == 0.0
    gx = _rand(rng, 2, 4 * D)
    s = _rand(rng, 2, 2 * D)
    J = O.cell_jacobian(O.CELL_LSTM_DIAG, rng.uniform(-1, 1, (4, D)), None, s, gx)
    mask = np.zeros((2 * D, 2 * D), bool)
    for d in range(D):
        for a in (d, D + d):
            for b in (d, D + d):
                mask[a, b] = True
    assert np.abs(J[:, ~mask]).max() == 0.0


def test_approx_jacobian_modes():
    rng = np.random.default_rng(21)
    J = rng.normal(size=(3, 4, 4))
    np.testing.assert_array_equal(O.approx_jacobian(J, O.JAC_FULL), J)
    Jd = O.approx_jacobian(J, O.JAC_DIAG)
    np.testing.assert_array_equal(np.einsum("nii->ni", Jd), np.einsum("nii->ni", J))
    np.testing.assert_array_equal(Jd - np.einsum("nii->ni", Jd)[:, :, None] * np.eye(4), 0)
    np.testing.assert_array_equal(O.approx_jacobian(J, O.JAC_ZERO), 0)
