"""Parallel-in-time Newton evaluation of nonlinear RNNs on AMD MI355X (gfx950).

The compute path is the HIP library ``libpnr.so`` (C ABI declared in ``include/pnr.h``);
``nonlinear_rnn_evaluation_amd.pnr`` is a thin ctypes binding over it that only
marshals arguments.  ``workloads`` draws the seeded synthetic inputs.
"""
__all__ = ["pnr", "workloads"]
