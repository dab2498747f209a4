"""GPU parity of chunked evaluation (pnr_eval_chunked) against the chunked CPU oracle.

Each chunk runs the same Newton loop as a whole-sequence call, from the state the
previous chunk returned at its last step, so the oracle (oracle.newton_chunked, pinned on
the CPU) is compared iterate by iterate: fixed iterations per chunk (tol < 0), several
chunks with a ragged last one, B = 1 (chunks passed in place) and B > 1 (chunks staged
through contiguous buffers), undamped and damped.  Bars as for the undamped path: fp32
state against the fp64 oracle at max-abs 1e-4.
"""
import numpy as np
import pytest
import torch

import oracle as O
from nonlinear_rnn_evaluation_amd import pnr
from nonlinear_rnn_evaluation_amd import workloads as WL

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _np(t):
    return t.detach().to("cpu").to(torch.float64).numpy()


def _run(cell, p, max_iters, tol, mode, chunk_len, damping=None, every=1):
    d = {k: (None if v is None else v.to(DEV)) for k, v in p.items()}
    return pnr.evaluate(cell, d["W"], d["U"], d["x"], b_x=d["b_x"], b_h=d["b_h"], h0=d["h0"],
                        max_iters=max_iters, tol=tol, jac_mode=mode, jac_every=every, damping=damping,
                        chunk_len=chunk_len)


def _f64(p):
    return {k: WL.as_f64(v) for k, v in p.items()}


CASES = [
    # cell, B, T, D, D_in, x dtype, mode, chunk
    (WL.CELL_GRU_DIAG, 1, 3000, 6, 5, WL.DT_F32, WL.JAC_FULL, 1024),
    (WL.CELL_GRU_DIAG, 3, 2500, 5, 3, WL.DT_F32, WL.JAC_FULL, 700),
    (WL.CELL_LSTM_DIAG, 1, 2100, 4, 3, WL.DT_F32, WL.JAC_FULL, 512),
    (WL.CELL_LSTM_DIAG, 2, 1300, 3, 8, WL.DT_BF16, WL.JAC_DIAG, 300),
    (WL.CELL_GRU, 2, 1200, 64, 9, WL.DT_F32, WL.JAC_DIAG, 500),
    (WL.CELL_GRU, 1, 900, 16, 4, WL.DT_F32, WL.JAC_FULL, 256),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "cell%d_B%d_T%d_D%d_m%d_L%d" % (c[0], c[1], c[2], c[3],
                                                                                     c[6], c[7]))
def test_fixed_iterations_per_chunk_match_the_oracle(case):
    cell, B, T, D, Din, xd, mode, L = case
    p = WL.random_problem(cell, B, T, D, Din, seed=T + D, x_dtype=xd, state_dtype=WL.DT_F32, bias_std=0.2,
                          h0_std=0.3, w_std=0.5 / np.sqrt(max(Din, D)))
    q = _f64(p)
    print(f"# chunked fixed iterations {case}", flush=True)
    got = _run(cell, p, 3, -1.0, mode, L)
    ref = O.newton_chunked(cell, q["W"], q["U"], q["b_x"], q["b_h"], q["x"], q["h0"], 3, -1.0, mode, L)
    n_chunks = -(-T // L)
    assert got["status"] == pnr.NOT_CONVERGED and got["iters"] == 3 * n_chunks
    assert len(got["history"]) == 4 * n_chunks
    np.testing.assert_allclose(_np(got["h"]), ref["states"], rtol=0, atol=1e-4)
    np.testing.assert_allclose(got["history"], ref["rhos"], rtol=1e-3, atol=1e-5)


@pytest.mark.parametrize("cell,mode", [(WL.CELL_GRU_DIAG, WL.JAC_FULL), (WL.CELL_LSTM_DIAG, WL.JAC_DIAG)])
@pytest.mark.parametrize("B", [1, 2])
def test_damped_chunks_match_the_oracle(cell, mode, B):
    T, L = 2300, 1000
    p = WL.random_problem(cell, B, T, 4, 3, seed=7 + B, x_dtype=WL.DT_F32, state_dtype=WL.DT_F32, bias_std=0.2,
                          h0_std=0.3)
    q = _f64(p)
    got = _run(cell, p, 2, -1.0, mode, L, damping=0.2)
    ref = O.newton_chunked(cell, q["W"], q["U"], q["b_x"], q["b_h"], q["x"], q["h0"], 2, -1.0, mode, L,
                           damping=0.2)
    np.testing.assert_allclose(_np(got["h"]), ref["states"], rtol=0, atol=1e-4)
    np.testing.assert_allclose(got["history"], ref["rhos"], rtol=1e-3, atol=1e-5)


@pytest.mark.parametrize("B", [1, 3])
def test_converged_chunks_equal_the_sequential_states(B):
    cell = WL.CELL_LSTM_DIAG
    p = WL.random_problem(cell, B, 5000, 8, 6, seed=11, x_dtype=WL.DT_F32, state_dtype=WL.DT_F32, bias_std=0.3,
                          h0_std=0.3)
    q = _f64(p)
    got = _run(cell, p, 64, 1e-6, WL.JAC_FULL, 1024, every=2)
    assert got["status"] == pnr.OK
    ref = O.sequential(cell, q["W"], q["U"], q["b_x"], q["b_h"], q["x"], q["h0"])
    assert np.abs(_np(got["h"]) - ref).max() < 1e-4


def test_one_chunk_is_bitwise_the_unchunked_call():
    cell = WL.CELL_GRU_DIAG
    p = WL.random_problem(cell, 2, 1500, 7, 5, seed=13, x_dtype=WL.DT_F32, state_dtype=WL.DT_F32, bias_std=0.2,
                          h0_std=0.3)
    d = {k: (None if v is None else v.to(DEV)) for k, v in p.items()}
    a = pnr.evaluate(cell, d["W"], d["U"], d["x"], b_x=d["b_x"], b_h=d["b_h"], h0=d["h0"], max_iters=5, tol=-1.0,
                     jac_mode=WL.JAC_FULL)
    b = _run(cell, p, 5, -1.0, WL.JAC_FULL, 1500)
    assert torch.equal(a["h"], b["h"]) and a["history"] == b["history"]


def test_one_step_chunks_and_an_empty_sequence():
    cell = WL.CELL_GRU_DIAG
    p = WL.random_problem(cell, 2, 37, 3, 2, seed=17, x_dtype=WL.DT_F32, state_dtype=WL.DT_F32, bias_std=0.2,
                          h0_std=0.3)
    q = _f64(p)
    got = _run(cell, p, 4, 1e-6, WL.JAC_FULL, 1)
    ref = O.sequential(cell, q["W"], q["U"], q["b_x"], q["b_h"], q["x"], q["h0"])
    assert got["status"] == pnr.OK and got["iters"] == 37
    assert np.abs(_np(got["h"]) - ref).max() < 1e-5
    e = WL.random_problem(cell, 2, 0, 3, 2, seed=1, x_dtype=WL.DT_F32, state_dtype=WL.DT_F32)
    r = _run(cell, e, 4, 1e-6, WL.JAC_FULL, 16)
    assert r["status"] == pnr.OK and r["iters"] == 0 and r["h"].numel() == 0


def test_nonfinite_chunk_stops_the_evaluation():
    cell = WL.CELL_GRU_DIAG
    p = WL.random_problem(cell, 1, 3000, 4, 3, seed=19, x_dtype=WL.DT_F32, state_dtype=WL.DT_F32, bias_std=0.2)
    p["x"][0, 1500, 1] = float("nan")
    got = _run(cell, p, 10, 1e-6, WL.JAC_FULL, 1000)
    assert got["status"] == pnr.NONFINITE
    # the first chunk converged on its own; the second reported the NaN at its first residual
    h = got["history"]
    assert h[-1] == float("inf") and got["iters"] == len(h) - 2
