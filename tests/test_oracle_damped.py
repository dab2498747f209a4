"""Pins for the damped (Levenberg-Marquardt / ELK) step of the oracle (CPU).

What fixes them, independently of the oracle's formulas:
* the step is defined as the minimiser of |A D - r|^2 + lam |D|^2 ("Towards Scalable
  and Stable Parallelization of Nonlinear RNNs", abstract: a Levenberg-Marquardt trust
  region); two independent derivations of it -- the normal equations solved by LAPACK,
  and a Kalman filter with an RTS smoother (the linear-Gaussian MAP view the same page
  names) -- must agree;
* special cases: lam = 0 is the undamped Newton step (forward substitution); one step
  (T = 1) has the closed form r / (1 + lam); two scalar steps are solved by hand below;
  lam -> infinity shrinks the step to A^T r / lam (a gradient step);
* a zero residual gives a zero step, so the damped iteration's fixed point is the
  sequential trajectory (DEER abstract: no loss of output accuracy).
"""
import numpy as np
import pytest

import oracle as O
from nonlinear_rnn_evaluation_amd import workloads as WL


def _rand(T, S, diag, seed):
    rng = np.random.default_rng(seed)
    J = rng.normal(size=(T, S)) if diag else 0.6 * rng.normal(size=(T, S, S))
    return J, rng.normal(size=(T, S))


@pytest.mark.parametrize("S,diag", [(1, True), (4, True), (3, False)])
@pytest.mark.parametrize("lam", [0.05, 1.0, 20.0])
def test_normal_equations_and_kalman_smoother_agree(S, diag, lam):
    J, r = _rand(9, S, diag, seed=S * 7 + int(lam * 10))
    np.testing.assert_allclose(O.lm_step_kalman(J, r, lam), O.lm_step_dense(J, r, lam), rtol=0, atol=1e-12)


@pytest.mark.parametrize("S,diag", [(1, True), (3, False)])
def test_zero_damping_is_the_newton_step(S, diag):
    J, r = _rand(8, S, diag, seed=3)
    dense = O.lm_step_dense(J, r, 0.0)
    newton = O.scan_loop(J, r)
    np.testing.assert_allclose(dense, newton, rtol=0, atol=1e-12)
    np.testing.assert_allclose(O.damped_step(J, r, 0.0), newton, rtol=0, atol=0)


@pytest.mark.parametrize("lam", [0.3, 4.0])
def test_single_step_closed_form(lam):
    r = np.array([[0.7, -1.3, 2.0]])
    J = np.array([[0.5, 0.1, -0.4]])   # never used: D_0 is known
    want = r / (1.0 + lam)
    np.testing.assert_allclose(O.lm_step_dense(J, r, lam), want, rtol=0, atol=1e-14)
    np.testing.assert_allclose(O.lm_step_kalman(J, r, lam), want, rtol=0, atol=1e-14)


def test_two_scalar_steps_by_hand():
    # minimise (d1 - r1)^2 + (d2 - j d1 - r2)^2 + lam (d1^2 + d2^2):
    #   (1 + j^2 + lam) d1 - j d2 = r1 - j r2
    #   -j d1 + (1 + lam) d2     = r2
    j, r1, r2, lam = 0.8, 1.5, -0.4, 0.6
    a11, a12, a21, a22 = 1 + j * j + lam, -j, -j, 1 + lam
    c1, c2 = r1 - j * r2, r2
    det = a11 * a22 - a12 * a21
    d1 = (c1 * a22 - a12 * c2) / det
    d2 = (a11 * c2 - a21 * c1) / det
    J = np.array([[0.0], [j]])
    r = np.array([[r1], [r2]])
    for f in (O.lm_step_dense, O.lm_step_kalman):
        np.testing.assert_allclose(f(J, r, lam)[:, 0], [d1, d2], rtol=0, atol=1e-14)


def test_large_damping_is_a_scaled_gradient_step():
    J, r = _rand(6, 2, True, seed=11)
    lam = 1e7
    # A^T r: (A^T r)_t = r_t - J_{t+1} r_{t+1}
    atr = r.copy()
    atr[:-1] -= J[1:] * r[1:]
    np.testing.assert_allclose(lam * O.lm_step_kalman(J, r, lam), atr, rtol=0, atol=1e-5)


@pytest.mark.parametrize("cell,mode", [(O.CELL_GRU_DIAG, O.JAC_FULL), (O.CELL_LSTM_DIAG, O.JAC_DIAG),
                                       (O.CELL_LSTM_DIAG, O.JAC_FULL), (O.CELL_GRU, O.JAC_DIAG)])
def test_damped_iteration_converges_to_the_sequential_trajectory(cell, mode):
    p = {k: WL.as_f64(v) for k, v in WL.random_problem(cell, 2, 40, 3, 2, seed=5, bias_std=0.3,
                                                        h0_std=0.5).items()}
    seq = O.sequential(cell, p["W"], p["U"], p["b_x"], p["b_h"], p["x"], p["h0"])
    for solver in ("dense", "loop"):
        res = O.newton_dense(cell, p["W"], p["U"], p["b_x"], p["b_h"], p["x"], p["h0"], 400, 1e-11, mode,
                             solver=solver, damping=0.2)
        assert res["status"] == O.STATUS_OK
        assert np.abs(res["states"] - seq).max() < 1e-9
        # damping slows it down relative to the undamped iteration
        und = O.newton_dense(cell, p["W"], p["U"], p["b_x"], p["b_h"], p["x"], p["h0"], 400, 1e-11, mode,
                             solver=solver)
        assert und["iters"] < res["iters"]


def test_damped_fixed_iterations_agree_between_solvers():
    cell = O.CELL_LSTM_DIAG
    p = {k: WL.as_f64(v) for k, v in WL.random_problem(cell, 2, 30, 3, 2, seed=8, bias_std=0.3,
                                                        h0_std=0.5, u_scale=2.0).items()}
    a = O.newton_dense(cell, p["W"], p["U"], p["b_x"], p["b_h"], p["x"], p["h0"], 4, -1.0, O.JAC_DIAG,
                       solver="dense", damping=0.7)
    b = O.newton_dense(cell, p["W"], p["U"], p["b_x"], p["b_h"], p["x"], p["h0"], 4, -1.0, O.JAC_DIAG,
                       solver="loop", damping=0.7)
    np.testing.assert_allclose(a["states"], b["states"], rtol=0, atol=1e-11)
