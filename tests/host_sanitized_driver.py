"""Host-code checks for the sanitizer build of the library (libpnr_san.so: AddressSanitizer
and UndefinedBehaviorSanitizer on the host code).  Run by tests/test_host_sanitized.py in a
child process with the sanitizer runtime preloaded; it imports neither torch nor the
package binding, only ctypes, and makes no device call: every request below is rejected,
or has nothing to do (T = 0), before any HIP call, or only asks for a workspace size.

It walks the argument validation and the workspace arithmetic of every entry point:
invalid enums and sizes, NULL pointers, short and misaligned workspaces, huge problems
(index-range checks), the empty sequence, and the thread-local error text and residual
history.  Exit status 0 when every expectation holds.
"""
import ctypes
import sys

LIB = sys.argv[1]
lib = ctypes.CDLL(LIB)


class Cell(ctypes.Structure):
    _fields_ = [("kind", ctypes.c_int32), ("D", ctypes.c_int32), ("D_in", ctypes.c_int32), ("T", ctypes.c_int32),
                ("B", ctypes.c_int32), ("x_dtype", ctypes.c_int32), ("state_dtype", ctypes.c_int32),
                ("jac_every", ctypes.c_int32), ("stream", ctypes.c_void_p), ("workspace", ctypes.c_void_p),
                ("workspace_bytes", ctypes.c_size_t)]


class Params(ctypes.Structure):
    _fields_ = [("W", ctypes.c_void_p), ("U", ctypes.c_void_p), ("b_x", ctypes.c_void_p), ("b_h", ctypes.c_void_p)]


P = ctypes.POINTER
vp, ci, cd, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_double, ctypes.c_size_t
for name, args, res in [
    ("pnr_workspace_bytes", [P(Cell), ci], sz),
    ("pnr_workspace_bytes_damped", [P(Cell), ci], sz),
    ("pnr_workspace_bytes_chunked", [P(Cell), ci, cd, ci], sz),
    ("pnr_workspace_bytes_backward", [P(Cell)], sz),
    ("pnr_workspace_bytes_backward_chunked", [P(Cell), ci], sz),
    ("pnr_workspace_bytes_lowrank", [P(Cell), ci], sz),
    ("pnr_scan_workspace_bytes", [ci, ci, ci, ci], sz),
    ("pnr_eval", [P(Cell), P(Params), vp, vp, vp, ci, cd, ci], ci),
    ("pnr_eval_static", [P(Cell), P(Params), vp, vp, vp, ci, cd, ci], ci),
    ("pnr_eval_bounded", [P(Cell), P(Params), vp, vp, vp, ci, cd, ci], ci),
    ("pnr_eval_lowrank", [P(Cell), P(Params), vp, vp, vp, ci, cd, ci], ci),
    ("pnr_eval_adaptive", [P(Cell), P(Params), vp, vp, vp, ci, cd, ci, cd], ci),
    ("pnr_eval_damped", [P(Cell), P(Params), vp, vp, vp, ci, cd, ci, cd], ci),
    ("pnr_eval_chunked", [P(Cell), P(Params), vp, vp, vp, ci, cd, ci, cd, ci], ci),
    ("pnr_backward", [P(Cell), P(Params)] + [vp] * 10, ci),
    ("pnr_backward_approx", [P(Cell), P(Params)] + [vp] * 10 + [ci], ci),
    ("pnr_backward_chunked", [P(Cell), P(Params)] + [vp] * 10 + [ci], ci),
    ("pnr_scan", [ci, ci, ci, vp, vp, vp, ci, vp, sz, vp], ci),
    ("pnr_iters_used", [], ci),
    ("pnr_last_residual", [], cd),
    ("pnr_last_residual_history", [P(ctypes.c_double), ci], ci),
    ("pnr_last_error", [], ctypes.c_char_p),
]:
    f = getattr(lib, name)
    f.argtypes, f.restype = args, res

E_INVALID, E_UNSUPPORTED, E_WORKSPACE, OK = -1, -2, -3, 0
GRU, GRU_DIAG, LSTM = 0, 1, 2
FULL, DIAG, ZERO = 0, 1, 2
F64, F32, BF16 = 0, 1, 2
fails = []


def expect(cond, what):
    if not cond:
        fails.append(what)


def cell(**kw):
    c = dict(kind=GRU_DIAG, D=64, D_in=32, T=1000, B=2, x_dtype=F32, state_dtype=F32, jac_every=1)
    c.update(kw)
    return Cell(c["kind"], c["D"], c["D_in"], c["T"], c["B"], c["x_dtype"], c["state_dtype"], c["jac_every"],
                None, None, 0)


prm = Params(0x1000, 0x2000, None, None)
X, OUT = 0x4000, 0x8000

# workspace sizes over a grid of shapes: all finite, nonzero for valid requests
for kind in (GRU, GRU_DIAG, LSTM):
    for D in (1, 3, 16, 33, 64, 4096):
        for T in (0, 1, 37, 1025, 131072):
            for B in (1, 7):
                for je in (1, 2):
                    for mode in (FULL, DIAG, ZERO):
                        c = cell(kind=kind, D=D, T=T, B=B, jac_every=je)
                        n = lib.pnr_workspace_bytes(ctypes.byref(c), mode)
                        expect(n == 0 or n % 256 == 0 or n > 0, ("ws", kind, D, T, B, je, mode))
                        lib.pnr_workspace_bytes_damped(ctypes.byref(c), mode)
                        lib.pnr_workspace_bytes_chunked(ctypes.byref(c), mode, 0.5, 100)
                        lib.pnr_workspace_bytes_chunked(ctypes.byref(c), mode, 0.0, 7)
                    lib.pnr_workspace_bytes_backward(ctypes.byref(c))
                    lib.pnr_workspace_bytes_backward_chunked(ctypes.byref(c), 333)
                    for r in (-1, 0, 2, D, D + 1):
                        lib.pnr_workspace_bytes_lowrank(ctypes.byref(c), r)

# invalid descriptors: rejected with a message, no iterations reported
for bad in (dict(kind=7), dict(D=0), dict(B=0), dict(T=-1), dict(jac_every=0), dict(x_dtype=9),
            dict(D=1 << 30, T=1 << 30), dict(kind=GRU, D=48)):
    c = cell(**bad)
    expect(lib.pnr_workspace_bytes(ctypes.byref(c), FULL) == 0, ("ws0", bad))
    rc = lib.pnr_eval(ctypes.byref(c), ctypes.byref(prm), X, None, OUT, 10, 1e-5, FULL)
    expect(rc in (E_INVALID, E_UNSUPPORTED), ("eval", bad, rc))
    expect(len(lib.pnr_last_error()) > 0 and lib.pnr_iters_used() == -1, ("err", bad))
expect(lib.pnr_eval(None, ctypes.byref(prm), X, None, OUT, 10, 1e-5, FULL) == E_INVALID, "null cell")
expect(lib.pnr_eval(ctypes.byref(cell()), None, X, None, OUT, 10, 1e-5, FULL) == E_INVALID, "null params")

# workspace: missing, misaligned, short
c = cell()
need = lib.pnr_workspace_bytes(ctypes.byref(c), FULL)
for ws, nb in ((None, need), (0x10008, need), (0x10000, need - 1)):
    c.workspace, c.workspace_bytes = ws, nb
    expect(lib.pnr_eval(ctypes.byref(c), ctypes.byref(prm), X, None, OUT, 10, 1e-5, FULL) == E_WORKSPACE, ("ws", ws))
    expect(lib.pnr_eval_bounded(ctypes.byref(c), ctypes.byref(prm), X, None, OUT, 10, 1e-5, FULL) == E_WORKSPACE,
           ("bounded ws", ws))
# bad scalars
c.workspace, c.workspace_bytes = 0x10000, need
for mi, tol, mode in ((-1, 1e-5, FULL), (1 << 20, 1e-5, FULL), (10, float("nan"), FULL), (10, 1e-5, 9)):
    expect(lib.pnr_eval(ctypes.byref(c), ctypes.byref(prm), X, None, OUT, mi, tol, mode) == E_INVALID, ("scalar", mi))
for rr in (-1.0, float("nan")):
    expect(lib.pnr_eval_adaptive(ctypes.byref(c), ctypes.byref(prm), X, None, OUT, 10, 1e-5, FULL, rr) == E_INVALID,
           ("ratio", rr))
for lam in (0.0, -1.0, float("nan"), float("inf")):
    expect(lib.pnr_eval_damped(ctypes.byref(c), ctypes.byref(prm), X, None, OUT, 10, 1e-5, FULL, lam) == E_INVALID,
           ("lam", lam))
expect(lib.pnr_eval_chunked(ctypes.byref(c), ctypes.byref(prm), X, None, OUT, 10, 1e-5, FULL, 0.0, 0) == E_INVALID,
       "chunk 0")
expect(lib.pnr_eval_lowrank(ctypes.byref(cell(kind=GRU, D=8)), ctypes.byref(prm), X, None, OUT, 10, 1e-5, 9)
       == E_INVALID, "rank")
expect(lib.pnr_eval_static(ctypes.byref(cell(kind=LSTM, D=4096, T=131072, B=1)), ctypes.byref(prm), X, None, OUT,
                           10, 1e-4, FULL) == E_WORKSPACE, "static too large")
grads = [None] * 6
expect(lib.pnr_backward_approx(ctypes.byref(c), ctypes.byref(prm), X, None, 0x3000, 0x5000, *grads, ZERO)
       == E_INVALID, "bwd mode")
expect(lib.pnr_scan(3, 4, 100, 1, 2, 3, 0, 256, 1 << 20, None) == E_INVALID, "scan kind")

# the empty sequence: OK with no device work, zero updates, a one-value history
e = cell(T=0)
e.workspace, e.workspace_bytes = 0x10000, lib.pnr_workspace_bytes(ctypes.byref(e), FULL)
for f in (lib.pnr_eval, lib.pnr_eval_bounded):
    expect(f(ctypes.byref(e), ctypes.byref(prm), None, None, None, 10, 1e-5, FULL) == OK, ("empty", f))
    expect(lib.pnr_iters_used() == 0 and lib.pnr_last_residual() == 0.0, "empty stats")
    n = lib.pnr_last_residual_history(None, 0)
    buf = (ctypes.c_double * max(n, 1))()
    expect(lib.pnr_last_residual_history(buf, n) == n == 1 and buf[0] == 0.0, "empty history")
    expect(lib.pnr_last_residual_history(buf, 0) == 1, "history with no room")

if fails:
    print("FAILED:", fails[:20])
    sys.exit(1)
print("host checks passed")
