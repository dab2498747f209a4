"""CPU oracle for parallel Newton evaluation of nonlinear RNNs (fp64, numpy).

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import this package: it
is used by ``tests/``, by ``__graft_entry__.smoke()`` and by the ``cpu_baseline`` leg
of ``bench.py``.  It shares no code with the HIP library and calls nothing in it.

What it computes (sources are the five pages on this method):

* ``sequential`` -- the plain definition: states produced one step at a time,
  s_t = f(s_{t-1}, x_t) from s_0 = h0.  The parallel methods reach exactly this fixed
  point ("Parallelizing non-linear sequential models over the sequence length",
  abstract: evaluation is parallelized without compromising output accuracy; the
  recurrence is the unique solution of the system of equations one obtains by
  unfolding it, ParaRNN overview, "Core Idea").
* ``newton_dense`` -- Newton's method on that system, each linear solve done by
  assembling the block lower-bidiagonal matrix densely and calling LAPACK (ParaRNN
  overview, "Technical Implementation / Newton's Iteration": Jacobian per iteration,
  block lower-triangular structure, optional Jacobian reuse; quasi-Newton diagonal
  approximation from "Towards Scalable and Stable Parallelization of Nonlinear RNNs",
  abstract and the scime summary's "Approach").
* ``scan_loop`` / ``scan_doubling`` -- the linear recurrence d_t = A_t d_{t-1} + b_t as
  a sequential loop, and as a recursive-doubling scan of affine maps (scime summary,
  "Builds on: parallel associative scan").
* ``sequential(..., dtype=np.float32)`` -- the same loop in fp32: the conditioning
  floor, i.e. the best agreement any fp32 evaluation can reach on a workload.
* ``lm_step_dense`` / ``lm_step_kalman`` -- the damped (Levenberg-Marquardt) step of
  ELK / quasi-ELK, by its normal equations and as a Kalman filter and smoother
  ("Towards Scalable and Stable Parallelization of Nonlinear RNNs", abstract and the
  summary's "Approach"); ``newton_dense(..., damping=lam)`` iterates it.
* ``bptt`` / ``cell_vjp`` -- gradients through the evaluated sequence: the adjoint run
  backwards in time, step by step (ParaRNN overview, "Newton's Iteration": forward and
  backward substitution; training through the parallel evaluation, "Parallelizing
  non-linear sequential models over the sequence length", abstract).
* ``newton_dense(..., bounded=True)`` -- each Newton iterate projected onto the box every
  reachable state lies in (``state_bounds``): a safeguard of this oracle's readings against
  the divergence of undamped Newton ("Towards Scalable and Stable Parallelization of
  Nonlinear RNNs", summary page, "Problem").
* ``newton_dense(..., jac_rank=r)`` -- the dense GRU with a low-rank approximation of its
  Jacobian (ParaRNN overview, "Newton's Iteration": low-rank approximations among the
  approximate-Newton strategies; ``oracle.lowrank``).
* ``newton_chunked`` -- the sequence evaluated chunk by chunk, each chunk from the
  previous chunk's last state (ParaRNN overview, "Experimental Results": chunking to
  bound the memory of long sequences).

Cell equations are not printed on the pages; the readings used (linear-before-reset
GRU with gates (r, z, n); LSTM with gates (i, f, o, g) and state (c, h); elementwise
recurrent weights for the diagonal-recurrence variants) are pinned by the tests in
``tests/test_oracle_*.py`` against torch's GRUCell/LSTMCell and autograd.
"""
from .cells import (CELL_GRU, CELL_GRU_DIAG, CELL_LSTM_DIAG, JAC_FULL, JAC_DIAG, JAC_ZERO,
                    cell_step, cell_jacobian, approx_jacobian, gates_of, state_size)
from .sequential import project, sequential, restrict_channels
from .newton import (newton_dense, STATUS_OK, STATUS_NOT_CONVERGED, STATUS_NONFINITE, max_abs,
                     state_bounds, project_states)
from .scan import scan_loop, scan_doubling, compose
from .damped import lm_step_dense, lm_step_kalman, damped_step
from .chunked import newton_chunked
from .lowrank import lowrank_matrix, truncated
from .backward import bptt, cell_vjp

__all__ = [
    "CELL_GRU", "CELL_GRU_DIAG", "CELL_LSTM_DIAG", "JAC_FULL", "JAC_DIAG", "JAC_ZERO",
    "cell_step", "cell_jacobian", "approx_jacobian", "gates_of", "state_size",
    "project", "sequential", "restrict_channels",
    "newton_dense", "STATUS_OK", "STATUS_NOT_CONVERGED", "STATUS_NONFINITE", "max_abs",
    "state_bounds", "project_states",
    "scan_loop", "scan_doubling", "compose",
    "lm_step_dense", "lm_step_kalman", "damped_step",
    "newton_chunked", "bptt", "cell_vjp", "lowrank_matrix", "truncated",
]
