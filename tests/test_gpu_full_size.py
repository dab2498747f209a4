"""Full-size parity: every named workload at its full shape, through the same C ABI call
and launch configuration the benchmark times, against the fp64 sequential oracle.

Dense-GRU workloads are compared on every output.  The damped (quasi-ELK) variant of the
long diagonal GRU is included: it converges to the same trajectory.  For the diagonal-recurrence cells a
set of evenly spaced channels is compared: with elementwise recurrent weights a channel
subset is an exact sub-problem of its own (oracle.restrict_channels), so the oracle
computes those outputs one channel group at a time.  Bar: 1e-4 max-abs for fp32 state,
1e-9 for fp64 state; the returned residual must satisfy the stopping test.
"""
import numpy as np
import pytest
import torch

import oracle as O
from oracle.sequential import output_channel_columns
from nonlinear_rnn_evaluation_amd import pnr
from nonlinear_rnn_evaluation_amd import workloads as WL

pytestmark = pytest.mark.gpu


def _check(name, mode):
    w = WL.get_workload(name)
    p = WL.generate(w)
    d = {k: (None if v is None else v.to("cuda")) for k, v in p.items()}
    print(f"# full-size parity: {name} mode {mode}", flush=True)
    res = pnr.evaluate(w.cell, d["W"], d["U"], d["x"], b_x=d["b_x"], b_h=d["b_h"], h0=d["h0"],
                       max_iters=w.max_iters, tol=w.tol, jac_mode=mode, jac_every=w.jac_every,
                       damping=w.damping)
    assert res["status"] == pnr.OK, (name, res["status"], res["residual"])
    assert 0 < res["iters"] <= w.max_iters
    assert res["residual"] <= w.tol
    assert res["history"][res["iters"]] == res["residual"]
    h = res["h"]
    assert h.shape == (w.B, w.T, WL.state_size(w.cell, w.D))
    W, U, bx, h0 = (WL.as_f64(p[k]) for k in ("W", "U", "b_x", "h0"))
    bh = WL.as_f64(p["b_h"])
    x = p["x"].float().numpy() if p["x"].dtype == torch.bfloat16 else p["x"].numpy()
    if w.cell in (WL.CELL_GRU_DIAG, WL.CELL_LSTM_DIAG):
        ch = np.linspace(0, w.D - 1, 16).round().astype(int)
        Wc, Uc, bxc, bhc, h0c, _ = O.restrict_channels(w.cell, w.D, W, U, bx, bh, h0, ch)
        ref = O.sequential(w.cell, Wc, Uc, bxc, bhc, x, h0c)
        cols = torch.from_numpy(output_channel_columns(w.cell, w.D, ch)).to(h.device)
        got = h[:, :, cols].double().cpu().numpy()
    else:
        ref = O.sequential(w.cell, W, U, bx, bh, x, h0)
        got = h.double().cpu().numpy()
    bar = 1e-9 if w.state_dtype == WL.DT_F64 else 1e-4
    err = np.abs(got - ref).max()
    print(f"#   iters {res['iters']} residual {res['residual']:.3e} max-abs {err:.3e}", flush=True)
    assert err <= bar, (name, mode, err)


CASES = [(name, mode) for name in WL.WORKLOAD_ORDER + ["gru_diag_long_elk"]
         for mode in WL.get_workload(name).jac_modes]


@pytest.mark.parametrize("name,mode", CASES, ids=[f"{n}-{['full', 'diag', 'zero'][m]}" for n, m in CASES])
def test_full_size_workload_matches_sequential_oracle(name, mode):
    try:
        _check(name, mode)
    finally:
        torch.cuda.empty_cache()
