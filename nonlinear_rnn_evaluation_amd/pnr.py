"""ctypes binding of libpnr (include/pnr.h): argument marshalling only.

Every step of the evaluation runs in the HIP library; this module turns torch tensors
into device pointers and the C structs, passes torch's current stream, and allocates
the output and workspace tensors (PyTorch is used only for device memory and streams).
If ``libpnr.so`` has not been built, loading raises -- there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
import re
from typing import Optional

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libpnr.so")
HEADER = os.path.join(os.path.dirname(HERE), "include", "pnr.h")

CELL_GRU, CELL_GRU_DIAG, CELL_LSTM_DIAG = 0, 1, 2
JAC_FULL, JAC_DIAG, JAC_ZERO = 0, 1, 2
F64, F32, BF16 = 0, 1, 2
OK, NOT_CONVERGED, NONFINITE = 0, 1, 2
E_INVALID, E_UNSUPPORTED, E_WORKSPACE, E_HIP = -1, -2, -3, -4
STATIC_SCRATCH_BYTES = 64 << 20   # PNR_STATIC_SCRATCH_BYTES of include/pnr.h

_DT = {torch.float64: F64, torch.float32: F32, torch.bfloat16: BF16}


class PnrCell(ctypes.Structure):
    _fields_ = [("kind", ctypes.c_int32), ("D", ctypes.c_int32), ("D_in", ctypes.c_int32),
                ("T", ctypes.c_int32), ("B", ctypes.c_int32), ("x_dtype", ctypes.c_int32),
                ("state_dtype", ctypes.c_int32), ("jac_every", ctypes.c_int32),
                ("stream", ctypes.c_void_p), ("workspace", ctypes.c_void_p),
                ("workspace_bytes", ctypes.c_size_t)]


class PnrParams(ctypes.Structure):
    _fields_ = [("W", ctypes.c_void_p), ("U", ctypes.c_void_p), ("b_x", ctypes.c_void_p),
                ("b_h", ctypes.c_void_p)]


class PnrProfile(ctypes.Structure):
    _fields_ = [("total_ms", ctypes.c_double), ("proj_ms", ctypes.c_double), ("newton_ms", ctypes.c_double),
                ("out_ms", ctypes.c_double), ("passes", ctypes.c_int32), ("resid_only", ctypes.c_int32)]


_lib = None


def load() -> ctypes.CDLL:
    """Load libpnr.so from the package directory (raises if it is not built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"libpnr.so not found at {LIB_PATH}; build it with "
                           "`python -m nonlinear_rnn_evaluation_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    P = ctypes.POINTER
    lib.pnr_workspace_bytes.argtypes = [P(PnrCell), ctypes.c_int]
    lib.pnr_workspace_bytes.restype = ctypes.c_size_t
    lib.pnr_eval.argtypes = [P(PnrCell), P(PnrParams), ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                             ctypes.c_int, ctypes.c_double, ctypes.c_int]
    lib.pnr_eval.restype = ctypes.c_int
    lib.pnr_workspace_bytes_damped.argtypes = [P(PnrCell), ctypes.c_int]
    lib.pnr_workspace_bytes_damped.restype = ctypes.c_size_t
    lib.pnr_eval_damped.argtypes = [P(PnrCell), P(PnrParams), ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                    ctypes.c_int, ctypes.c_double, ctypes.c_int, ctypes.c_double]
    lib.pnr_eval_damped.restype = ctypes.c_int
    lib.pnr_workspace_bytes_chunked.argtypes = [P(PnrCell), ctypes.c_int, ctypes.c_double, ctypes.c_int]
    lib.pnr_workspace_bytes_chunked.restype = ctypes.c_size_t
    lib.pnr_eval_chunked.argtypes = [P(PnrCell), P(PnrParams), ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                     ctypes.c_int, ctypes.c_double, ctypes.c_int, ctypes.c_double, ctypes.c_int]
    lib.pnr_eval_chunked.restype = ctypes.c_int
    lib.pnr_workspace_bytes_backward.argtypes = [P(PnrCell)]
    lib.pnr_workspace_bytes_backward.restype = ctypes.c_size_t
    lib.pnr_backward.argtypes = [P(PnrCell), P(PnrParams)] + [ctypes.c_void_p] * 10
    lib.pnr_backward.restype = ctypes.c_int
    lib.pnr_workspace_bytes_lowrank.argtypes = [P(PnrCell), ctypes.c_int]
    lib.pnr_workspace_bytes_lowrank.restype = ctypes.c_size_t
    lib.pnr_eval_lowrank.argtypes = [P(PnrCell), P(PnrParams), ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                     ctypes.c_int, ctypes.c_double, ctypes.c_int]
    lib.pnr_eval_lowrank.restype = ctypes.c_int
    lib.pnr_eval_bounded.argtypes = [P(PnrCell), P(PnrParams), ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                     ctypes.c_int, ctypes.c_double, ctypes.c_int]
    lib.pnr_eval_bounded.restype = ctypes.c_int
    lib.pnr_eval_static.argtypes = [P(PnrCell), P(PnrParams), ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                    ctypes.c_int, ctypes.c_double, ctypes.c_int]
    lib.pnr_eval_static.restype = ctypes.c_int
    lib.pnr_backward_approx.argtypes = [P(PnrCell), P(PnrParams)] + [ctypes.c_void_p] * 10 + [ctypes.c_int]
    lib.pnr_backward_approx.restype = ctypes.c_int
    lib.pnr_eval_adaptive.argtypes = [P(PnrCell), P(PnrParams), ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                      ctypes.c_int, ctypes.c_double, ctypes.c_int, ctypes.c_double]
    lib.pnr_eval_adaptive.restype = ctypes.c_int
    lib.pnr_workspace_bytes_backward_chunked.argtypes = [P(PnrCell), ctypes.c_int]
    lib.pnr_workspace_bytes_backward_chunked.restype = ctypes.c_size_t
    lib.pnr_backward_chunked.argtypes = [P(PnrCell), P(PnrParams)] + [ctypes.c_void_p] * 10 + [ctypes.c_int]
    lib.pnr_backward_chunked.restype = ctypes.c_int
    lib.pnr_iters_used.argtypes = []
    lib.pnr_iters_used.restype = ctypes.c_int
    lib.pnr_last_residual.argtypes = []
    lib.pnr_last_residual.restype = ctypes.c_double
    lib.pnr_last_residual_history.argtypes = [P(ctypes.c_double), ctypes.c_int]
    lib.pnr_last_residual_history.restype = ctypes.c_int
    lib.pnr_last_error.argtypes = []
    lib.pnr_last_error.restype = ctypes.c_char_p
    lib.pnr_scan_workspace_bytes.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int]
    lib.pnr_scan_workspace_bytes.restype = ctypes.c_size_t
    lib.pnr_scan.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p,
                             ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
    lib.pnr_scan.restype = ctypes.c_int
    lib.pnr_profile_enable.argtypes = [ctypes.c_int]
    lib.pnr_profile_enable.restype = ctypes.c_int
    lib.pnr_last_profile.argtypes = [P(PnrProfile)]
    lib.pnr_last_profile.restype = ctypes.c_int
    _lib = lib
    return lib


def header_functions() -> list:
    """Names of the functions declared in include/pnr.h."""
    with open(HEADER) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return re.findall(r"\b(pnr_[a-z_]+)\s*\(", text)


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("libpnr takes device tensors")
    if not t.is_contiguous():
        raise ValueError("libpnr takes contiguous tensors")
    return t.data_ptr()


def _check(t: Optional[torch.Tensor], name: str, dtype: torch.dtype, shape: tuple) -> Optional[torch.Tensor]:
    """The library reads raw memory, so a tensor of another dtype or shape would be
    reinterpreted, not converted: refuse it."""
    if t is None:
        return None
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype} (got {t.dtype})")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)} (got {tuple(t.shape)})")
    return t


def _arg(t: Optional[torch.Tensor], name: str, dtype: torch.dtype, shape: tuple) -> Optional[int]:
    return _ptr(_check(t, name, dtype, shape))


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def make_cell(kind: int, D: int, D_in: int, T: int, B: int, x_dtype: int, state_dtype: int,
              jac_every: int = 1, stream: Optional[int] = None, workspace: Optional[int] = None,
              workspace_bytes: int = 0) -> PnrCell:
    return PnrCell(kind, D, D_in, T, B, x_dtype, state_dtype, jac_every, stream, workspace, workspace_bytes)


# ---- the C entry points under their own names ------------------------------------------
def pnr_workspace_bytes(cell: PnrCell, jac_mode: int) -> int:
    return load().pnr_workspace_bytes(ctypes.byref(cell), jac_mode)


def pnr_eval(cell: PnrCell, params: PnrParams, x: int, h0: Optional[int], h_out: int, max_iters: int,
             tol: float, jac_mode: int) -> int:
    return load().pnr_eval(ctypes.byref(cell), ctypes.byref(params), x, h0, h_out, max_iters, tol, jac_mode)


def pnr_workspace_bytes_lowrank(cell: PnrCell, rank: int) -> int:
    return load().pnr_workspace_bytes_lowrank(ctypes.byref(cell), rank)


def pnr_eval_lowrank(cell: PnrCell, params: PnrParams, x: int, h0: Optional[int], h_out: int, max_iters: int,
                     tol: float, rank: int) -> int:
    return load().pnr_eval_lowrank(ctypes.byref(cell), ctypes.byref(params), x, h0, h_out, max_iters, tol, rank)


def pnr_eval_bounded(cell: PnrCell, params: PnrParams, x: int, h0: Optional[int], h_out: int, max_iters: int,
                     tol: float, jac_mode: int) -> int:
    return load().pnr_eval_bounded(ctypes.byref(cell), ctypes.byref(params), x, h0, h_out, max_iters, tol, jac_mode)


def pnr_eval_static(cell: PnrCell, params: PnrParams, x: int, h0: Optional[int], h_out: int, max_iters: int,
                    tol: float, jac_mode: int) -> int:
    return load().pnr_eval_static(ctypes.byref(cell), ctypes.byref(params), x, h0, h_out, max_iters, tol, jac_mode)


def pnr_eval_adaptive(cell: PnrCell, params: PnrParams, x: int, h0: Optional[int], h_out: int, max_iters: int,
                      tol: float, jac_mode: int, refresh_ratio: float) -> int:
    return load().pnr_eval_adaptive(ctypes.byref(cell), ctypes.byref(params), x, h0, h_out, max_iters, tol,
                                    jac_mode, refresh_ratio)


def pnr_workspace_bytes_damped(cell: PnrCell, jac_mode: int) -> int:
    return load().pnr_workspace_bytes_damped(ctypes.byref(cell), jac_mode)


def pnr_eval_damped(cell: PnrCell, params: PnrParams, x: int, h0: Optional[int], h_out: int, max_iters: int,
                    tol: float, jac_mode: int, damping: float) -> int:
    return load().pnr_eval_damped(ctypes.byref(cell), ctypes.byref(params), x, h0, h_out, max_iters, tol, jac_mode,
                                  damping)


def pnr_workspace_bytes_chunked(cell: PnrCell, jac_mode: int, damping: float, chunk_len: int) -> int:
    return load().pnr_workspace_bytes_chunked(ctypes.byref(cell), jac_mode, damping, chunk_len)


def pnr_eval_chunked(cell: PnrCell, params: PnrParams, x: int, h0: Optional[int], h_out: int, max_iters: int,
                     tol: float, jac_mode: int, damping: float, chunk_len: int) -> int:
    return load().pnr_eval_chunked(ctypes.byref(cell), ctypes.byref(params), x, h0, h_out, max_iters, tol, jac_mode,
                                   damping, chunk_len)


def pnr_workspace_bytes_backward(cell: PnrCell) -> int:
    return load().pnr_workspace_bytes_backward(ctypes.byref(cell))


def pnr_backward(cell: PnrCell, params: PnrParams, x: int, h0: Optional[int], h: int, grad_h: int,
                 grad_x: Optional[int], grad_W: Optional[int], grad_U: Optional[int], grad_b_x: Optional[int],
                 grad_b_h: Optional[int], grad_h0: Optional[int]) -> int:
    return load().pnr_backward(ctypes.byref(cell), ctypes.byref(params), x, h0, h, grad_h, grad_x, grad_W, grad_U,
                               grad_b_x, grad_b_h, grad_h0)


def pnr_backward_approx(cell: PnrCell, params: PnrParams, x: int, h0: Optional[int], h: int, grad_h: int,
                        grad_x: Optional[int], grad_W: Optional[int], grad_U: Optional[int],
                        grad_b_x: Optional[int], grad_b_h: Optional[int], grad_h0: Optional[int],
                        jac_mode: int) -> int:
    return load().pnr_backward_approx(ctypes.byref(cell), ctypes.byref(params), x, h0, h, grad_h, grad_x, grad_W,
                                      grad_U, grad_b_x, grad_b_h, grad_h0, jac_mode)


def pnr_workspace_bytes_backward_chunked(cell: PnrCell, chunk_len: int) -> int:
    return load().pnr_workspace_bytes_backward_chunked(ctypes.byref(cell), chunk_len)


def pnr_backward_chunked(cell: PnrCell, params: PnrParams, x: int, h0: Optional[int], h: int, grad_h: int,
                         grad_x: Optional[int], grad_W: Optional[int], grad_U: Optional[int],
                         grad_b_x: Optional[int], grad_b_h: Optional[int], grad_h0: Optional[int],
                         chunk_len: int) -> int:
    return load().pnr_backward_chunked(ctypes.byref(cell), ctypes.byref(params), x, h0, h, grad_h, grad_x, grad_W,
                                       grad_U, grad_b_x, grad_b_h, grad_h0, chunk_len)


def pnr_iters_used() -> int:
    return load().pnr_iters_used()


def pnr_last_residual() -> float:
    return load().pnr_last_residual()


def pnr_last_residual_history() -> list:
    lib = load()
    n = lib.pnr_last_residual_history(None, 0)
    buf = (ctypes.c_double * max(n, 1))()
    lib.pnr_last_residual_history(buf, n)
    return list(buf[:n])


def pnr_last_error() -> str:
    return load().pnr_last_error().decode()


def pnr_scan_workspace_bytes(kind: int, R: int, T: int, tile_len: int = 0) -> int:
    return load().pnr_scan_workspace_bytes(kind, R, T, tile_len)


def pnr_scan(kind: int, R: int, T: int, A: int, b: int, d: int, tile_len: int, workspace: int,
             workspace_bytes: int, stream: Optional[int]) -> int:
    return load().pnr_scan(kind, R, T, A, b, d, tile_len, workspace, workspace_bytes, stream)


def pnr_profile_enable(on: bool) -> int:
    return load().pnr_profile_enable(1 if on else 0)


def pnr_last_profile() -> Optional[dict]:
    p = PnrProfile()
    if load().pnr_last_profile(ctypes.byref(p)) != 0:
        return None
    return {name: getattr(p, name) for name, _ in PnrProfile._fields_}


# ---- torch-level conveniences (allocation + marshalling) ---------------------------------
class PnrError(RuntimeError):
    pass


def evaluate(kind: int, W: torch.Tensor, U: torch.Tensor, x: torch.Tensor, *, b_x=None, b_h=None,
             h0=None, max_iters: int = 64, tol: float = 1e-5, jac_mode: int = JAC_FULL,
             jac_every: int = 1, h_out: Optional[torch.Tensor] = None,
             workspace: Optional[torch.Tensor] = None, damping: Optional[float] = None,
             chunk_len: Optional[int] = None, refresh_ratio: Optional[float] = None,
             static_scratch: bool = False, bounded: bool = False, jac_rank: Optional[int] = None) -> dict:
    """Run pnr_eval (or pnr_eval_damped when `damping` is given, pnr_eval_chunked when
    `chunk_len` is given, pnr_eval_adaptive when `refresh_ratio` is given, pnr_eval_static
    -- no workspace; the library's static device scratch -- when `static_scratch`,
    pnr_eval_bounded when `bounded`, pnr_eval_lowrank when `jac_rank` is given -- the
    jac_mode argument is then FULL) on device tensors; returns dict(h=[B,T,S], status,
    iters, residual, history)."""
    if refresh_ratio is not None and (damping is not None or chunk_len is not None):
        raise ValueError("refresh_ratio combines with neither damping nor chunk_len")
    if static_scratch and (refresh_ratio is not None or damping is not None or chunk_len is not None
                           or workspace is not None):
        raise ValueError("static_scratch is pnr_eval's variant: no damping, chunking, refresh ratio or workspace")
    if jac_rank is not None and (refresh_ratio is not None or damping is not None or chunk_len is not None
                                 or static_scratch or bounded):
        raise ValueError("jac_rank is pnr_eval's variant: no damping, chunking, refresh ratio, bounds or static scratch")
    if bounded and (refresh_ratio is not None or damping is not None or chunk_len is not None or static_scratch):
        raise ValueError("bounded is pnr_eval's variant: no damping, chunking, refresh ratio or static scratch")
    B, T, D_in = x.shape
    D = U.shape[1]
    S = 2 * D if kind == CELL_LSTM_DIAG else D
    if x.dtype not in _DT or U.dtype not in _DT:
        raise TypeError(f"unsupported dtypes x {x.dtype}, U {U.dtype}")
    xdt, sdt = _DT[x.dtype], _DT[U.dtype]
    G = 4 if kind == CELL_LSTM_DIAG else 3
    sd = U.dtype
    args = dict(W=_check(W, "W", x.dtype, (G * D, D_in)),
                U=_check(U, "U", sd, (G * D, D) if kind == CELL_GRU else (G, D)),
                b_x=_check(b_x, "b_x", sd, (G * D,)), b_h=_check(b_h, "b_h", sd, (G * D,)),
                h0=_check(h0, "h0", sd, (B, S)), x=x)
    if h_out is not None:
        _check(h_out, "h_out", sd, (B, T, S))
    ptrs = {k: _ptr(v) for k, v in args.items()}
    cell = make_cell(kind, D, D_in, T, B, xdt, sdt, jac_every, _stream())
    if static_scratch:
        need = 0
    elif jac_rank is not None:
        need = pnr_workspace_bytes_lowrank(cell, jac_rank)
    elif chunk_len is not None:
        need = pnr_workspace_bytes_chunked(cell, jac_mode, damping or 0.0, chunk_len)
    elif damping is None:
        need = pnr_workspace_bytes(cell, jac_mode)
    else:
        need = pnr_workspace_bytes_damped(cell, jac_mode)
    if need == 0 and not static_scratch:
        raise PnrError(pnr_last_error())
    if not static_scratch:
        if workspace is None or workspace.numel() < need:
            workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
        cell.workspace = workspace.data_ptr()
        cell.workspace_bytes = workspace.numel()
    if h_out is None:
        h_out = torch.empty(B, T, S, dtype=U.dtype, device=x.device)
    out = _arg(h_out, "h_out", sd, (B, T, S))
    params = PnrParams(ptrs["W"], ptrs["U"], ptrs["b_x"], ptrs["b_h"])
    if jac_rank is not None:
        rc = pnr_eval_lowrank(cell, params, ptrs["x"], ptrs["h0"], out, max_iters, tol, jac_rank)
    elif bounded:
        rc = pnr_eval_bounded(cell, params, ptrs["x"], ptrs["h0"], out, max_iters, tol, jac_mode)
    elif static_scratch:
        rc = pnr_eval_static(cell, params, ptrs["x"], ptrs["h0"], out, max_iters, tol, jac_mode)
    elif chunk_len is not None:
        rc = pnr_eval_chunked(cell, params, ptrs["x"], ptrs["h0"], out, max_iters, tol, jac_mode,
                              damping or 0.0, chunk_len)
    elif refresh_ratio is not None:
        rc = pnr_eval_adaptive(cell, params, ptrs["x"], ptrs["h0"], out, max_iters, tol, jac_mode, refresh_ratio)
    elif damping is None:
        rc = pnr_eval(cell, params, ptrs["x"], ptrs["h0"], out, max_iters, tol, jac_mode)
    else:
        rc = pnr_eval_damped(cell, params, ptrs["x"], ptrs["h0"], out, max_iters, tol, jac_mode, damping)
    if rc < 0:
        raise PnrError(f"pnr_eval returned {rc}: {pnr_last_error()}")
    return {"h": h_out, "status": rc, "iters": pnr_iters_used(), "residual": pnr_last_residual(),
            "history": pnr_last_residual_history(), "workspace": workspace}


def backward(kind: int, W: torch.Tensor, U: torch.Tensor, x: torch.Tensor, h: torch.Tensor, grad_h: torch.Tensor,
             *, b_x=None, b_h=None, h0=None, want=("x", "W", "U", "b_x", "b_h", "h0"),
             workspace: Optional[torch.Tensor] = None, chunk_len: int = 0,
             jac_mode: Optional[int] = None) -> dict:
    """Run pnr_backward on device tensors: gradients of L through the recurrence whose
    states are h, given grad_h = dL/dh.  Returns {name: fp32 tensor} for the names in
    `want` (the others are not computed), plus "workspace" and the adjoint solve's
    "status", "iters", "residual" and "history" (dense GRU: refinement iterations;
    diagonal cells: one scan, iters 0).  chunk_len > 0 runs pnr_backward_chunked: the
    sequence is processed in chunks of that many steps, last chunk first, with a
    workspace sized for one chunk.  jac_mode runs pnr_backward_approx: JAC_FULL exact,
    JAC_DIAG the diagonal approximation in the adjoint recursion."""
    if jac_mode is not None and chunk_len:
        raise ValueError("jac_mode applies to the unchunked backward pass")
    B, T, D_in = x.shape
    G, D = (U.shape[0] // U.shape[1], U.shape[1]) if kind == CELL_GRU else (U.shape[0], U.shape[1])
    S = 2 * D if kind == CELL_LSTM_DIAG else D
    if x.dtype not in _DT or U.dtype not in _DT:
        raise TypeError(f"unsupported dtypes x {x.dtype}, U {U.dtype}")
    sd = U.dtype
    args = dict(h=_check(h, "h", sd, (B, T, S)), grad_h=_check(grad_h, "grad_h", sd, (B, T, S)),
                W=_check(W, "W", x.dtype, (G * D, D_in)), b_x=_check(b_x, "b_x", sd, (G * D,)),
                b_h=_check(b_h, "b_h", sd, (G * D,)), h0=_check(h0, "h0", sd, (B, S)), U=U, x=x)
    ptrs = {k: _ptr(v) for k, v in args.items()}
    cell = make_cell(kind, D, D_in, T, B, _DT[x.dtype], _DT[U.dtype], 1, _stream())
    if chunk_len < 0:
        raise ValueError(f"chunk_len must be >= 0 (got {chunk_len})")
    need = pnr_workspace_bytes_backward_chunked(cell, chunk_len) if chunk_len else pnr_workspace_bytes_backward(cell)
    if need == 0:
        raise PnrError(pnr_last_error())
    if workspace is None or workspace.numel() < need:
        workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
    cell.workspace = workspace.data_ptr()
    cell.workspace_bytes = workspace.numel()
    f32 = dict(dtype=torch.float32, device=x.device)
    shapes = {"x": (B, T, D_in), "W": (G * D, D_in), "U": tuple(U.shape), "b_x": (G * D,), "b_h": (G * D,),
              "h0": (B, S)}
    out = {k: torch.empty(shapes[k], **f32) for k in want}
    params = PnrParams(ptrs["W"], ptrs["U"], ptrs["b_x"], ptrs["b_h"])
    grads = [_ptr(out.get(k)) for k in ("x", "W", "U", "b_x", "b_h", "h0")]
    if chunk_len:
        rc = pnr_backward_chunked(cell, params, ptrs["x"], ptrs["h0"], ptrs["h"], ptrs["grad_h"], *grads, chunk_len)
    elif jac_mode is not None:
        rc = pnr_backward_approx(cell, params, ptrs["x"], ptrs["h0"], ptrs["h"], ptrs["grad_h"], *grads, jac_mode)
    else:
        rc = pnr_backward(cell, params, ptrs["x"], ptrs["h0"], ptrs["h"], ptrs["grad_h"], *grads)
    if rc < 0:
        raise PnrError(f"pnr_backward{'_chunked' if chunk_len else ''} returned {rc}: {pnr_last_error()}")
    out.update(workspace=workspace, status=rc, iters=pnr_iters_used(), residual=pnr_last_residual(),
               history=pnr_last_residual_history())
    return out


def scan(kind: int, A: torch.Tensor, b: torch.Tensor, tile_len: int = 0) -> torch.Tensor:
    """Standalone linear scan d_t = A_t d_{t-1} + b_t (kind 1: [R,T]; kind 2: A [R,4,T], b [R,2,T])."""
    R, T = b.shape[0], b.shape[-1]
    shapes = {1: ((R, T), (R, T)), 2: ((R, 4, T), (R, 2, T))}.get(kind)
    if shapes is not None:
        _check(A, "A", torch.float32, shapes[0])
        _check(b, "b", torch.float32, shapes[1])
    d = torch.empty_like(b)
    need = pnr_scan_workspace_bytes(kind, R, T, tile_len)
    ws = torch.empty(max(need, 256), dtype=torch.uint8, device=b.device)
    rc = pnr_scan(kind, R, T, _ptr(A), _ptr(b), _ptr(d), tile_len, ws.data_ptr(), ws.numel(), _stream())
    if rc < 0:
        raise PnrError(f"pnr_scan returned {rc}: {pnr_last_error()}")
    return d
