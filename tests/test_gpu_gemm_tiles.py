"""The bf16 projection GEMM's block tiles at ragged sizes, through pnr_eval.

The long products run on 256 x 384 or 256 x 256 block tiles (8 or 16 waves, four LDS
stages, C written through LDS in 16-row rounds); a cost model over the waves of blocks on
the device's CUs picks one.  The named workloads have M = G D a multiple of 256, so these
cases make both M and N = T ragged against both tiles, with biases on the rows:

* D = 1000, T = 40000 (M = 4000, N = 40000): on 256 CUs the model picks 256 x 384
  (1680 blocks, 7 waves, against 2512 blocks, 10 waves, for 256 x 256);
* D = 1000, T = 3000: 256 x 256 (both fill one wave, where the wider tile is slower);
* D = 300, T = 2000 (M = 1200).

A diagonal LSTM with bf16 x and W converges on each; channels are compared over every
step with the fp64 sequential oracle on a channel subset that includes the last channels
(the rows of the last, partial row tile), at the 1e-4 bar of fp32 state.
"""
import numpy as np
import pytest
import torch

import oracle as O
from oracle.sequential import output_channel_columns
from nonlinear_rnn_evaluation_amd import pnr
from nonlinear_rnn_evaluation_amd import workloads as WL

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("D,T", [(1000, 40000), (1000, 3000), (300, 2000)])
def test_ragged_projection_tiles_match_sequential_oracle(D, T):
    cell, D_in = WL.CELL_LSTM_DIAG, 96
    p = WL.random_problem(cell, 1, T, D, D_in, seed=11, x_dtype=WL.DT_BF16, state_dtype=WL.DT_F32, bias_std=0.3)
    d = {k: (None if v is None else v.to("cuda")) for k, v in p.items()}
    print(f"# ragged GEMM tiles: D {D} (M {4 * D}) T {T} K {D_in}", flush=True)
    res = pnr.evaluate(cell, d["W"], d["U"], d["x"], b_x=d["b_x"], b_h=d["b_h"], h0=d["h0"], max_iters=64, tol=1e-5,
                       jac_mode=pnr.JAC_FULL, jac_every=1)
    assert res["status"] == pnr.OK, (res["status"], res["residual"])
    ch = np.unique(np.concatenate([np.linspace(0, D - 1, 24).round().astype(int), np.arange(D - 8, D)]))
    W, U, bx, bh, h0 = (None if p[k] is None else WL.as_f64(p[k]) for k in ("W", "U", "b_x", "b_h", "h0"))
    Wc, Uc, bxc, bhc, h0c, _ = O.restrict_channels(cell, D, W, U, bx, bh, h0, ch)
    ref = O.sequential(cell, Wc, Uc, bxc, bhc, p["x"].float().numpy(), h0c)
    cols = torch.from_numpy(output_channel_columns(cell, D, ch)).to("cuda")
    got = res["h"][:, :, cols].double().cpu().numpy()
    err = np.abs(got - ref).max()
    print(f"#   iters {res['iters']} residual {res['residual']:.2e} max-abs {err:.2e} over {len(ch)} channels",
          flush=True)
    assert err <= 1e-4
