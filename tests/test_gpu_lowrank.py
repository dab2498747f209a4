"""pnr_eval_lowrank (the dense GRU with a low-rank approximation of its Jacobian) against the
oracle's newton_dense(..., jac_rank=r), through the C ABI.

States and residual history after exactly k updates are compared element by element for
ranks 0 .. D on the MFMA kernel (D = 16, fp32) and the VALU kernel (other D, fp32 and
fp64), on one tile and on several tiles with a ragged tail; rank D must reproduce
pnr_eval's dense Jacobian bit for bit (the same matrix in the same kernel), and the
converged states must be the sequential ones.
"""
import numpy as np
import pytest
import torch

import oracle as O
from nonlinear_rnn_evaluation_amd import pnr
from nonlinear_rnn_evaluation_amd import workloads as WL

pytestmark = pytest.mark.gpu


def _problem(B, T, D, D_in, seed, dt):
    p = WL.random_problem(WL.CELL_GRU, B, T, D, D_in, seed=seed, x_dtype=dt, state_dtype=dt, bias_std=0.2,
                          h0_std=0.3)
    d = {k: (None if v is None else v.to("cuda")) for k, v in p.items()}
    q = {k: (None if v is None else WL.as_f64(v)) for k, v in p.items()}
    return d, q


def _eval(d, **kw):
    return pnr.evaluate(WL.CELL_GRU, d["W"], d["U"], d["x"], b_x=d["b_x"], b_h=d["b_h"], h0=d["h0"], **kw)


CASES = [(16, WL.DT_F32), (8, WL.DT_F32), (24, WL.DT_F32), (4, WL.DT_F64), (8, WL.DT_F64)]


@pytest.mark.parametrize("D,dt", CASES, ids=[f"D{D}-{'f64' if dt == WL.DT_F64 else 'f32'}" for D, dt in CASES])
@pytest.mark.parametrize("T", [37, 700])
def test_lowrank_iterates_match_the_oracle(D, dt, T):
    d, q = _problem(2, T, D, 5, seed=D + T, dt=dt)
    bar = 1e-9 if dt == WL.DT_F64 else 1e-4
    k = 3
    for rank in sorted({0, D // 4, D // 2, D}):
        print(f"# low-rank D={D} T={T} rank={rank}", flush=True)
        got = _eval(d, max_iters=k, tol=-1.0, jac_mode=WL.JAC_FULL, jac_rank=rank)
        ref = O.newton_dense(WL.CELL_GRU, q["W"], q["U"], q["b_x"], q["b_h"], q["x"], q["h0"], k, -1.0,
                             WL.JAC_FULL, solver="loop", jac_rank=rank)
        assert got["status"] == pnr.NOT_CONVERGED and got["iters"] == k
        err = float(np.abs(got["h"].double().cpu().numpy() - ref["states"]).max())
        assert err <= bar, (rank, err)
        assert np.allclose(got["history"], ref["rhos"], rtol=1e-3, atol=bar)


@pytest.mark.parametrize("D,dt", [(16, WL.DT_F32), (8, WL.DT_F32), (8, WL.DT_F64)])
def test_full_rank_is_pnr_eval_bit_for_bit(D, dt):
    d, q = _problem(3, 500, D, 4, seed=9, dt=dt)
    a = _eval(d, max_iters=4, tol=-1.0, jac_mode=WL.JAC_FULL)
    b = _eval(d, max_iters=4, tol=-1.0, jac_mode=WL.JAC_FULL, jac_rank=D)
    assert torch.equal(a["h"], b["h"])
    assert a["history"] == b["history"]


@pytest.mark.parametrize("rank", [0, 2, 8, 16])
def test_lowrank_converges_to_the_sequential_states(rank):
    d, q = _problem(2, 3000, 16, 16, seed=4, dt=WL.DT_F32)
    got = _eval(d, max_iters=64, tol=1e-6, jac_mode=WL.JAC_FULL, jac_rank=rank)
    seq = O.sequential(WL.CELL_GRU, q["W"], q["U"], q["b_x"], q["b_h"], q["x"], q["h0"])
    err = float(np.abs(got["h"].double().cpu().numpy() - seq).max())
    print(f"# rank {rank}: status {got['status']} iters {got['iters']} max-abs {err:.2e}", flush=True)
    assert got["status"] == pnr.OK
    assert err < 1e-4


def test_lowrank_rejects_bad_requests():
    d, q = _problem(1, 10, 8, 2, seed=0, dt=WL.DT_F32)
    with pytest.raises(pnr.PnrError, match="rank must be"):
        _eval(d, max_iters=2, tol=1e-5, jac_mode=WL.JAC_FULL, jac_rank=9)
    p = WL.random_problem(WL.CELL_GRU_DIAG, 1, 10, 8, 2, seed=0, x_dtype=WL.DT_F32, state_dtype=WL.DT_F32)
    dd = {k: (None if v is None else v.to("cuda")) for k, v in p.items()}
    with pytest.raises(pnr.PnrError, match="dense recurrent"):
        pnr.evaluate(WL.CELL_GRU_DIAG, dd["W"], dd["U"], dd["x"], max_iters=2, tol=1e-5, jac_mode=WL.JAC_FULL,
                     jac_rank=2)
