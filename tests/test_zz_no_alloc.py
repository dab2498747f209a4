"""pnr_eval_static: pnr_eval on the library's static device scratch, for callers that cannot
allocate.  Its results must match pnr_eval's (the same kernels on another scratch) to the
parity bar, and its scratch keeps the last call's contents, so every case makes two calls
in a row, the second on a smaller problem, each compared with pnr_eval on the same inputs
and with the fp64 sequential oracle.
"""
import ctypes

import numpy as np
import pytest
import torch

import oracle as O
from nonlinear_rnn_evaluation_amd import pnr
from nonlinear_rnn_evaluation_amd import workloads as WL


def _problem(cell, B, T, D, D_in, dt, seed):
    p = WL.random_problem(cell, B, T, D, D_in, seed=seed, x_dtype=dt, state_dtype=dt, bias_std=0.2, h0_std=0.3)
    return p


def _run_pair(cell, shape, dt, mode, jac_every, tol, seed):
    B, T, D, D_in = shape
    p = _problem(cell, B, T, D, D_in, dt, seed)
    d = {k: (None if v is None else v.to("cuda")) for k, v in p.items()}
    kw = dict(b_x=d["b_x"], b_h=d["b_h"], h0=d["h0"], max_iters=64, tol=tol, jac_mode=mode, jac_every=jac_every)
    print(f"# no-alloc: cell {cell} shape {shape} dtype {dt} mode {mode}", flush=True)
    got = pnr.evaluate(cell, d["W"], d["U"], d["x"], static_scratch=True, **kw)
    ref = pnr.evaluate(cell, d["W"], d["U"], d["x"], **kw)
    torch.cuda.synchronize()
    assert got["status"] == ref["status"] == pnr.OK, (got["status"], ref["status"])
    assert got["iters"] == ref["iters"]
    bar = 1e-9 if dt == WL.DT_F64 else 1e-4
    diff = (got["h"].double() - ref["h"].double()).abs().max().item()
    assert diff <= bar, diff
    q = {k: (None if v is None else WL.as_f64(v)) for k, v in p.items()}
    seq = O.sequential(cell, q["W"], q["U"], q["b_x"], q["b_h"], q["x"], q["h0"])
    err = float(np.abs(got["h"].double().cpu().numpy() - seq).max())
    print(f"#   iters {got['iters']} |static - pnr_eval| {diff:.2e} |static - oracle| {err:.2e}", flush=True)
    assert err <= bar, err
    return got


CASES = [
    # (cell, first shape, second (smaller) shape, dtype, jac_mode, jac_every, tol)
    (WL.CELL_GRU, (8, 4096, 64, 64), (2, 1000, 64, 64), WL.DT_F32, WL.JAC_DIAG, 1, 1e-5),
    (WL.CELL_GRU, (4, 2048, 16, 16), (1, 333, 16, 16), WL.DT_F32, WL.JAC_FULL, 1, 1e-5),
    (WL.CELL_LSTM_DIAG, (2, 3000, 16, 32), (1, 1025, 8, 32), WL.DT_F32, WL.JAC_FULL, 2, 1e-5),
    (WL.CELL_GRU_DIAG, (4, 2048, 64, 48), (3, 700, 24, 48), WL.DT_F32, WL.JAC_FULL, 1, 1e-5),
    (WL.CELL_GRU, (1, 64, 4, 2), (1, 20, 4, 2), WL.DT_F64, WL.JAC_FULL, 1, 1e-10),
]


@pytest.mark.gpu
@pytest.mark.parametrize("case", CASES, ids=[f"cell{c[0]}-D{c[1][2]}-mode{c[4]}-dt{c[3]}" for c in CASES])
def test_static_scratch_matches_pnr_eval_on_two_calls(case):
    cell, big, small, dt, mode, jac_every, tol = case
    try:
        _run_pair(cell, big, dt, mode, jac_every, tol, seed=11)
        _run_pair(cell, small, dt, mode, jac_every, tol, seed=12)
    finally:
        torch.cuda.empty_cache()


def test_static_scratch_rejects_a_problem_larger_than_its_scratch():
    """Checked on the host before any HIP call: runs without a GPU."""
    cell = pnr.make_cell(WL.CELL_LSTM_DIAG, 4096, 4096, 131072, 1, WL.DT_BF16, WL.DT_F32, 2)
    need = pnr.pnr_workspace_bytes(cell, WL.JAC_FULL)
    assert need > pnr.STATIC_SCRATCH_BYTES
    params = pnr.PnrParams(16, 16, None, None)
    rc = pnr.pnr_eval_static(cell, params, 16, None, 16, 8, 1e-4, WL.JAC_FULL)
    assert rc == pnr.E_WORKSPACE
    msg = pnr.pnr_last_error()
    assert str(need) in msg and "static scratch" in msg
    assert pnr.pnr_iters_used() == -1
    # invalid arguments are still reported as such
    rc = pnr.pnr_eval_static(cell, params, 16, None, 16, -1, 1e-4, WL.JAC_FULL)
    assert rc == pnr.E_INVALID
