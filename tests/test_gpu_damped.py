"""GPU parity of the damped (quasi-ELK) evaluation against the CPU oracle.

The oracle's damped step (oracle.damped: Kalman filter + RTS smoother, itself pinned
against the normal equations of the Levenberg-Marquardt step) is iterated with the same
stopping rule as the HIP path.  Bars as for the undamped path: fp32 state against the
fp64 oracle at max-abs 1e-4, per iteration and at convergence.  Sizes span several
1024-step tiles with a ragged tail (the kernel's tile is 256 threads x 4 steps); a tile's
last step takes its smoother coefficients from the next tile's first, so lengths one past
a tile boundary are covered too.  The diagonal LSTM runs quasi-ELK (diagonal of its 2x2
Jacobian: two scalar filters per channel, for c and for h) and ELK proper (the exact 2x2
block: one 2-state filter per channel).
"""
import math

import numpy as np
import pytest
import torch

import oracle as O
from nonlinear_rnn_evaluation_amd import pnr
from nonlinear_rnn_evaluation_amd import workloads as WL

pytestmark = pytest.mark.gpu

DEV = "cuda"
CELL = WL.CELL_GRU_DIAG


def _np(t):
    return t.detach().to("cpu").to(torch.float64).numpy()


def _run(p, max_iters, tol, mode, lam, cell=CELL):
    d = {k: (None if v is None else v.to(DEV)) for k, v in p.items()}
    return pnr.evaluate(cell, d["W"], d["U"], d["x"], b_x=d["b_x"], b_h=d["b_h"], h0=d["h0"],
                        max_iters=max_iters, tol=tol, jac_mode=mode, damping=lam)


def _f64(p):
    return {k: WL.as_f64(v) for k, v in p.items()}


def _problem(T, D=5, B=2, seed=0, x_dtype=WL.DT_F32, cell=CELL):
    return WL.random_problem(cell, B, T, D, 3, seed=seed, x_dtype=x_dtype, state_dtype=WL.DT_F32,
                             bias_std=0.2, h0_std=0.3)


@pytest.mark.parametrize("T", [37, 1024, 2 * 1024 + 300])
@pytest.mark.parametrize("mode", [WL.JAC_FULL, WL.JAC_DIAG])
@pytest.mark.parametrize("lam", [0.05, 1.0])
def test_fixed_iterations_match_damped_oracle(T, mode, lam):
    p = _problem(T, seed=T % 97)
    q = _f64(p)
    print(f"# damped fixed iterations T={T} mode={mode} lam={lam}", flush=True)
    got = _run(p, 3, -1.0, mode, lam)
    ref = O.newton_dense(CELL, q["W"], q["U"], q["b_x"], q["b_h"], q["x"], q["h0"], 3, -1.0, mode,
                         solver="loop", damping=lam)
    assert got["status"] == pnr.NOT_CONVERGED and got["iters"] == 3
    np.testing.assert_allclose(_np(got["h"]), ref["states"], rtol=0, atol=1e-4)
    np.testing.assert_allclose(got["history"], ref["rhos"], rtol=1e-3, atol=1e-5)


def test_converged_damped_equals_sequential():
    p = _problem(3000, D=7, B=3, seed=4)
    q = _f64(p)
    got = _run(p, 200, 1e-6, WL.JAC_FULL, 0.3)
    assert got["status"] == pnr.OK, (got["status"], got["history"][-3:])
    ref = O.sequential(CELL, q["W"], q["U"], q["b_x"], q["b_h"], q["x"], q["h0"])
    assert np.abs(_np(got["h"]) - ref).max() < 1e-4
    # damping costs iterations against the undamped step on the same problem
    d = {k: (None if v is None else v.to(DEV)) for k, v in p.items()}
    und = pnr.evaluate(CELL, d["W"], d["U"], d["x"], b_x=d["b_x"], b_h=d["b_h"], h0=d["h0"],
                       max_iters=200, tol=1e-6, jac_mode=WL.JAC_FULL)
    assert und["status"] == pnr.OK and und["iters"] < got["iters"]


def test_vanishing_damping_gives_the_newton_iterates():
    p = _problem(1500, seed=9)
    d = {k: (None if v is None else v.to(DEV)) for k, v in p.items()}
    und = pnr.evaluate(CELL, d["W"], d["U"], d["x"], b_x=d["b_x"], b_h=d["b_h"], h0=d["h0"],
                       max_iters=2, tol=-1.0, jac_mode=WL.JAC_FULL)
    got = _run(p, 2, -1.0, WL.JAC_FULL, 1e-7)
    np.testing.assert_allclose(_np(got["h"]), _np(und["h"]), rtol=0, atol=1e-4)


def test_bf16_inputs_and_zero_iterations():
    p = _problem(1300, seed=2, x_dtype=WL.DT_BF16)
    q = _f64(p)
    got = _run(p, 2, -1.0, WL.JAC_DIAG, 0.5)
    ref = O.newton_dense(CELL, q["W"], q["U"], q["b_x"], q["b_h"], q["x"], q["h0"], 2, -1.0, WL.JAC_DIAG,
                         solver="loop", damping=0.5)
    np.testing.assert_allclose(_np(got["h"]), ref["states"], rtol=0, atol=1e-4)
    zero = _run(p, 0, 1e-5, WL.JAC_DIAG, 0.5)
    assert zero["iters"] == 0 and np.abs(_np(zero["h"])).max() == 0.0


def test_damped_nonfinite_input_reports_nonfinite():
    p = _problem(700, seed=3)
    p["x"][1, 123, 2] = float("nan")
    got = _run(p, 10, 1e-6, WL.JAC_FULL, 0.5)
    assert got["status"] == pnr.NONFINITE and got["iters"] == 0
    assert math.isinf(got["residual"])


LSTM = WL.CELL_LSTM_DIAG


@pytest.mark.parametrize("T", [1, 37, 1023, 1025, 2 * 1024 + 300])
@pytest.mark.parametrize("lam", [0.05, 1.0])
def test_lstm_fixed_iterations_match_damped_oracle(T, lam):
    p = _problem(T, D=4, seed=T % 89, cell=LSTM)
    q = _f64(p)
    print(f"# damped LSTM fixed iterations T={T} lam={lam}", flush=True)
    got = _run(p, 3, -1.0, WL.JAC_DIAG, lam, cell=LSTM)
    ref = O.newton_dense(LSTM, q["W"], q["U"], q["b_x"], q["b_h"], q["x"], q["h0"], 3, -1.0, WL.JAC_DIAG,
                         solver="loop", damping=lam)
    assert got["status"] == pnr.NOT_CONVERGED and got["iters"] == 3
    np.testing.assert_allclose(_np(got["h"]), ref["states"], rtol=0, atol=1e-4)
    np.testing.assert_allclose(got["history"], ref["rhos"], rtol=1e-3, atol=1e-5)


def test_lstm_damped_step_matches_normal_equations():
    """One damped step from the zero guess against the Levenberg-Marquardt normal equations
    solved densely (a short sequence, so the dense solve stays small)."""
    p = _problem(150, D=3, B=2, seed=21, cell=LSTM)
    q = _f64(p)
    got = _run(p, 1, -1.0, WL.JAC_DIAG, 0.3, cell=LSTM)
    ref = O.newton_dense(LSTM, q["W"], q["U"], q["b_x"], q["b_h"], q["x"], q["h0"], 1, -1.0, WL.JAC_DIAG,
                         solver="dense", damping=0.3)
    np.testing.assert_allclose(_np(got["h"]), ref["states"], rtol=0, atol=1e-4)


def test_lstm_converged_damped_equals_sequential():
    p = _problem(2500, D=6, B=3, seed=5, cell=LSTM)
    q = _f64(p)
    got = _run(p, 300, 1e-6, WL.JAC_DIAG, 0.2, cell=LSTM)
    assert got["status"] == pnr.OK, (got["status"], got["history"][-3:])
    ref = O.sequential(LSTM, q["W"], q["U"], q["b_x"], q["b_h"], q["x"], q["h0"])
    assert np.abs(_np(got["h"]) - ref).max() < 1e-4


@pytest.mark.parametrize("T", [1, 37, 1023, 1025, 2 * 1024 + 300])
@pytest.mark.parametrize("lam", [0.05, 1.0])
def test_lstm_elk_fixed_iterations_match_damped_oracle(T, lam):
    """ELK proper: the exact 2x2 Jacobian block per channel (the oracle's Kalman filter and
    smoother run on the dense block-diagonal Jacobian)."""
    p = _problem(T, D=4, seed=T % 83, cell=LSTM)
    q = _f64(p)
    print(f"# ELK LSTM fixed iterations T={T} lam={lam}", flush=True)
    got = _run(p, 3, -1.0, WL.JAC_FULL, lam, cell=LSTM)
    ref = O.newton_dense(LSTM, q["W"], q["U"], q["b_x"], q["b_h"], q["x"], q["h0"], 3, -1.0, WL.JAC_FULL,
                         solver="loop", damping=lam)
    assert got["status"] == pnr.NOT_CONVERGED and got["iters"] == 3
    np.testing.assert_allclose(_np(got["h"]), ref["states"], rtol=0, atol=1e-4)
    np.testing.assert_allclose(got["history"], ref["rhos"], rtol=1e-3, atol=1e-5)


def test_lstm_elk_step_matches_normal_equations():
    """One ELK step from the zero guess against the Levenberg-Marquardt normal equations of
    the dense block-bidiagonal system, solved by LAPACK."""
    p = _problem(150, D=3, B=2, seed=22, cell=LSTM)
    q = _f64(p)
    got = _run(p, 1, -1.0, WL.JAC_FULL, 0.3, cell=LSTM)
    ref = O.newton_dense(LSTM, q["W"], q["U"], q["b_x"], q["b_h"], q["x"], q["h0"], 1, -1.0, WL.JAC_FULL,
                         solver="dense", damping=0.3)
    np.testing.assert_allclose(_np(got["h"]), ref["states"], rtol=0, atol=1e-4)


def test_lstm_elk_vanishing_damping_gives_the_newton_iterates():
    p = _problem(1500, D=3, B=2, seed=23, cell=LSTM)
    d = {k: (None if v is None else v.to(DEV)) for k, v in p.items()}
    newton = pnr.evaluate(LSTM, d["W"], d["U"], d["x"], b_x=d["b_x"], b_h=d["b_h"], h0=d["h0"],
                          max_iters=2, tol=-1.0, jac_mode=WL.JAC_FULL)
    got = _run(p, 2, -1.0, WL.JAC_FULL, 1e-7, cell=LSTM)
    np.testing.assert_allclose(_np(got["h"]), _np(newton["h"]), rtol=0, atol=1e-4)


def test_lstm_elk_converged_equals_sequential():
    p = _problem(2500, D=6, B=3, seed=6, cell=LSTM)
    q = _f64(p)
    got = _run(p, 300, 1e-6, WL.JAC_FULL, 0.2, cell=LSTM)
    assert got["status"] == pnr.OK, (got["status"], got["history"][-3:])
    ref = O.sequential(LSTM, q["W"], q["U"], q["b_x"], q["b_h"], q["x"], q["h0"])
    assert np.abs(_np(got["h"]) - ref).max() < 1e-4


# Dense GRU (quasi-ELK): the iteration against the oracle's Kalman-smoother step with the
# diagonal of the dense Jacobian.  The device loop cuts the sequence into chunks of 16
# steps (one MFMA row tile) that cross waves only through their boundary values, so the
# lengths span one partial chunk, exactly one, many with a ragged last one, and (B = 3,
# T = 11000: 2064 chunks) more chunks than a full grid has waves; D = 1, 7 and 40 leave
# most of the 64 padded channels of the recurrent product empty.
GRU = WL.CELL_GRU


@pytest.mark.parametrize("B,D,T", [(2, 16, 37), (2, 16, 1000), (2, 64, 333), (2, 40, 1500), (2, 1, 17),
                                   (2, 7, 5), (1, 64, 16), (3, 8, 11000)])
@pytest.mark.parametrize("lam", [0.05, 1.0])
def test_dense_gru_fixed_iterations_match_damped_oracle(B, D, T, lam):
    p = WL.random_problem(GRU, B, T, D, 5, seed=D + T, x_dtype=WL.DT_F32, state_dtype=WL.DT_F32, bias_std=0.2,
                          h0_std=0.3, w_std=0.7 / math.sqrt(D))
    q = _f64(p)
    print(f"# damped dense GRU B={B} D={D} T={T} lam={lam}", flush=True)
    got = _run(p, 3, -1.0, WL.JAC_DIAG, lam, cell=GRU)
    ref = O.newton_dense(GRU, q["W"], q["U"], q["b_x"], q["b_h"], q["x"], q["h0"], 3, -1.0, WL.JAC_DIAG,
                         solver="loop", damping=lam)
    assert got["status"] == pnr.NOT_CONVERGED and got["iters"] == 3
    np.testing.assert_allclose(_np(got["h"]), ref["states"], rtol=0, atol=1e-4)
    np.testing.assert_allclose(got["history"], ref["rhos"], rtol=1e-3, atol=1e-5)


def test_dense_gru_damped_converges_to_the_sequential_states():
    p = WL.random_problem(GRU, 3, 2000, 64, 8, seed=3, x_dtype=WL.DT_F32, state_dtype=WL.DT_F32, bias_std=0.2,
                          h0_std=0.3, w_std=0.7 / math.sqrt(64))
    q = _f64(p)
    got = _run(p, 200, 1e-6, WL.JAC_DIAG, 0.1, cell=GRU)
    assert got["status"] == pnr.OK, (got["status"], got["history"][-3:])
    ref = O.sequential(GRU, q["W"], q["U"], q["b_x"], q["b_h"], q["x"], q["h0"])
    assert np.abs(_np(got["h"]) - ref).max() < 1e-4
    # damped chunks of the same problem
    d = {k: (None if v is None else v.to(DEV)) for k, v in p.items()}
    ch = pnr.evaluate(GRU, d["W"], d["U"], d["x"], b_x=d["b_x"], b_h=d["b_h"], h0=d["h0"], max_iters=200, tol=1e-6,
                      jac_mode=WL.JAC_DIAG, damping=0.1, chunk_len=700)
    assert ch["status"] == pnr.OK and np.abs(_np(ch["h"]) - ref).max() < 1e-4


def test_dense_gru_damped_edge_cases():
    p = WL.random_problem(GRU, 1, 300, 16, 3, seed=9, x_dtype=WL.DT_F32, state_dtype=WL.DT_F32, bias_std=0.2)
    zero = _run(p, 0, 1e-5, WL.JAC_DIAG, 0.5, cell=GRU)
    assert zero["iters"] == 0 and np.abs(_np(zero["h"])).max() == 0.0
    p["x"][0, 77, 1] = float("nan")
    bad = _run(p, 10, 1e-6, WL.JAC_DIAG, 0.5, cell=GRU)
    assert bad["status"] == pnr.NONFINITE and bad["iters"] == 0
    with pytest.raises(pnr.PnrError):
        _run(p, 2, -1.0, WL.JAC_FULL, 0.5, cell=GRU)
