/*
 * pnr.h -- C ABI of libpnr: parallel-in-time Newton evaluation of a nonlinear RNN
 * on one AMD MI355X (gfx950).
 *
 * The operation.  Given inputs x_1..x_T, an initial state s_0 = h0 and a cell f, the
 * library returns the states s_t = f(s_{t-1}, x_t), t = 1..T.  Instead of stepping
 * through time it unfolds the recurrence into one system of nonlinear equations, one
 * per step (ParaRNN overview page, "Core Idea"; DEER poses the states as the solution
 * of a fixed-point problem: "Towards Scalable and Stable Parallelization of Nonlinear
 * RNNs", abstract) and solves it with Newton iterations (ParaRNN overview, "Newton's
 * Iteration").  One iteration k:
 *   r_t   = f(s_{t-1}^(k), x_t) - s_t^(k)                       residual, every t at once
 *   J_t   = df/ds evaluated at s_{t-1}                          Jacobian (mode below)
 *   rho_k = max_{b,t,i} |r|   (NaN counts as +inf)              two-level reduction
 *           stop if rho_k <= tol or rho_k is not finite          (ParaRNN overview, "Parallel Reduction")
 *   d_t   = J_t d_{t-1} + r_t, d_0 = 0                          block lower-bidiagonal solve,
 *                                                                done as a parallel scan of
 *                                                                affine maps
 *   s^(k+1) = s^(k) + d
 * The converged states equal sequential evaluation ("Parallelizing non-linear
 * sequential models over the sequence length", abstract).  The initial guess is
 * s^(0) = 0.  The Newton loop runs on the device: no host synchronisation happens
 * between iterations; the call synchronises once at its end.
 *
 * Cells (the pages print no equations; these are the readings implemented):
 *   PNR_CELL_GRU        GRU, dense recurrent matrix U [3D, D], gate blocks (r, z, n),
 *                       "linear before reset": n = tanh(gx_n + r*(U_n h + b_hn)),
 *                       h' = (1-z) n + z h.  State size S = D.
 *   PNR_CELL_GRU_DIAG   the same GRU with elementwise recurrent weights u [3, D]
 *                       (diagonal recurrence, as in ParaRNN's GRU adaptation).  S = D.
 *   PNR_CELL_LSTM_DIAG  LSTM with elementwise recurrent weights u [4, D], gate blocks
 *                       (i, f, o, g); state (c, h), S = 2D, c first.
 *
 * Jacobian modes (jac_mode):
 *   PNR_JAC_FULL  exact Jacobian in the cell's own structure: dense D x D (GRU),
 *                 diagonal (GRU_DIAG), one 2x2 block per channel (LSTM_DIAG).
 *   PNR_JAC_DIAG  its diagonal: quasi-Newton ("quasi-DEER"; "Towards Scalable and
 *                 Stable Parallelization of Nonlinear RNNs", abstract).
 *   PNR_JAC_ZERO  no Jacobian: a fixed-point (Picard) sweep.  Test mode.
 * pnr_cell.jac_every = e >= 1 recomputes the Jacobian only on iterations k with
 * k % e == 0 and reuses it otherwise (ParaRNN overview, "Newton's Iteration": the
 * Jacobian recomputed only every few steps); the residual is always fresh.
 *
 * Memory and layout.  Every tensor argument is a DEVICE pointer, row-major, owned by
 * the caller and not retained after the call returns (x and h_out may be NULL when
 * T = 0):
 *   x      [B, T, D_in]            x_dtype
 *   h0     [B, S]                  state_dtype (may be NULL: zeros)
 *   h_out  [B, T, S]               state_dtype; h_out[b, t] = s_{t+1}; h0 excluded
 *   W      [G*D, D_in]             x_dtype     (G = 3 for GRU cells, 4 for LSTM)
 *   U      GRU: [3D, D]; GRU_DIAG: [3, D]; LSTM_DIAG: [4, D]     state_dtype
 *   b_x    [G*D] (NULL = 0)        state_dtype; added to W x
 *   b_h    [G*D] (NULL = 0)        state_dtype; added to the recurrent term (for
 *                                  the GRU candidate gate it sits inside r*(...))
 * The library allocates no device memory: all scratch comes from pnr_cell.workspace,
 * at least pnr_workspace_bytes() bytes, 256-byte aligned.  Work is enqueued on
 * pnr_cell.stream (a hipStream_t; NULL = the default stream).
 *
 * Supported combinations (others return PNR_E_UNSUPPORTED):
 *   GRU:        (x, state) in {(f64, f64), (f32, f32), (bf16, f32)}; D <= 32 with
 *               PNR_JAC_FULL, D <= 64 (fp32 state) or 32 (fp64 state) otherwise
 *   GRU_DIAG,
 *   LSTM_DIAG:  (x, state) in {(f32, f32), (bf16, f32)}
 *
 * Launches.  Each Newton loop is one persistent kernel whose workgroups wait on one
 * another, sized to the device's resident capacity and launched with
 * hipLaunchCooperativeKernel, which guarantees that they are all resident at once, also
 * next to other work on the device; calls with distinct workspaces may therefore run on
 * different streams at the same time.  Every device-side wait is bounded: one that runs
 * out is reported as PNR_E_HIP, never a hang.  Setting PNR_COOPERATIVE=0 in the
 * environment (read once per process) selects ordinary launches, slightly cheaper, for
 * callers that run nothing else on the device while a call is in flight.
 *
 * Errors.  Functions never abort and never print.  Negative return codes mean no
 * result was produced; the text of the last error of the calling thread is
 * available from pnr_last_error().  Argument validation happens before any HIP call.
 */
#ifndef PNR_H
#define PNR_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum pnr_cell_kind { PNR_CELL_GRU = 0, PNR_CELL_GRU_DIAG = 1, PNR_CELL_LSTM_DIAG = 2 };
enum pnr_jac_mode { PNR_JAC_FULL = 0, PNR_JAC_DIAG = 1, PNR_JAC_ZERO = 2 };
enum pnr_dtype { PNR_F64 = 0, PNR_F32 = 1, PNR_BF16 = 2 };
enum pnr_status {
  PNR_OK = 0,             /* converged: rho <= tol                                   */
  PNR_NOT_CONVERGED = 1,  /* max_iters updates applied, rho > tol; h_out = last iterate */
  PNR_NONFINITE = 2,      /* a residual was NaN/Inf; h_out = the iterate that made it   */
  PNR_E_INVALID = -1,     /* bad pointer, size, enum or combination                   */
  PNR_E_UNSUPPORTED = -2, /* valid request outside the supported set above            */
  PNR_E_WORKSPACE = -3,   /* workspace NULL, misaligned or smaller than required      */
  PNR_E_HIP = -4          /* a HIP runtime call failed                                */
};

/* Problem description.  All sizes must be >= 1 (T may be 0: nothing to do). */
typedef struct pnr_cell {
  int32_t kind;          /* pnr_cell_kind                                   */
  int32_t D;             /* channels (hidden size)                          */
  int32_t D_in;          /* input features                                  */
  int32_t T;             /* sequence length                                 */
  int32_t B;             /* batch                                           */
  int32_t x_dtype;       /* pnr_dtype of x and W                            */
  int32_t state_dtype;   /* pnr_dtype of h0, h_out, U, b_x, b_h             */
  int32_t jac_every;     /* >= 1                                            */
  void* stream;          /* hipStream_t, NULL = default stream              */
  void* workspace;       /* device scratch, >= pnr_workspace_bytes(...)     */
  size_t workspace_bytes;
} pnr_cell;

typedef struct pnr_params {
  const void* W;    /* [G*D, D_in]        x_dtype                       */
  const void* U;    /* see the cell list   state_dtype                   */
  const void* b_x;  /* [G*D] or NULL       state_dtype                   */
  const void* b_h;  /* [G*D] or NULL       state_dtype                   */
} pnr_params;

/*
 * Scratch bytes pnr_eval needs for this problem and Jacobian mode (0 on invalid
 * input; the reason is in pnr_last_error()).  Pure host arithmetic; no HIP call.
 * The Jacobian itself is never stored: it is rebuilt inside the iteration kernel from
 * the stored states (and, for the dense GRU, from U), so the dense mode needs no
 * O(T D^2) buffer and both Jacobian modes use O(T D) workspace.
 */
size_t pnr_workspace_bytes(const pnr_cell* cell, int jac_mode);

/*
 * Evaluate the RNN by parallel Newton iterations (see the top of this file).
 *   max_iters  >= 0: at most this many Newton updates; 0 returns the initial guess.
 *   tol        stop when rho_k <= tol; tol < 0 never stops early (exactly max_iters
 *              updates are applied).
 * Returns a pnr_status.  On PNR_OK / PNR_NOT_CONVERGED / PNR_NONFINITE, h_out holds
 * the iterate s^(k) whose residual rho_k was checked last, and the call has
 * synchronised the stream.  Thread-safe for distinct workspaces.
 */
int pnr_eval(const pnr_cell* cell, const pnr_params* params, const void* x, const void* h0,
             void* h_out, int max_iters, double tol, int jac_mode);

/*
 * pnr_eval with an adaptive Jacobian refresh, for the diagonal-recurrence cells
 * (PNR_CELL_GRU_DIAG, PNR_CELL_LSTM_DIAG).  The ParaRNN overview ("Newton's Iteration")
 * names recomputing the Jacobian only every few steps among its approximate-Newton
 * strategies; here the residual decides when, by a rule of this library's own: iteration
 * k takes a new Jacobian (at its current iterate) when
 *     k == 0,  or  k - (last refresh) >= cell->jac_every,
 *     or  k >= 2 and rho_{k-1} > refresh_ratio * rho_{k-2},
 * i.e. also when the update before last shrank the max-norm residual by less than the
 * ratio.  The rule looks one update back because the fused pass that evaluates the
 * residual rho_k also takes the Jacobian, before rho_k is known.  refresh_ratio = +inf
 * is pnr_eval's fixed schedule; refresh_ratio = 0 refreshes at every k >= 2.  Arguments,
 * workspace (pnr_workspace_bytes) and results as pnr_eval.  refresh_ratio must be >= 0
 * (PNR_E_INVALID otherwise, NaN included); the dense-U GRU returns PNR_E_UNSUPPORTED.
 */
int pnr_eval_adaptive(const pnr_cell* cell, const pnr_params* params, const void* x, const void* h0,
                      void* h_out, int max_iters, double tol, int jac_mode, double refresh_ratio);

/*
 * pnr_eval without allocation, for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).  Same
 * arguments, iteration, results and errors as pnr_eval, except that pnr_cell.workspace
 * and workspace_bytes are ignored: the scratch (control words, residual partials,
 * look-back slots, gate pre-activations and iterates) lives in a static device array of
 * PNR_STATIC_SCRATCH_BYTES, one per device, held from the library's first use on that
 * device until the process ends.  A problem whose pnr_workspace_bytes() exceeds that
 * size returns PNR_E_WORKSPACE before any device work (e.g. B=8, T=4096, D=64 fits; the
 * long diagonal workloads do not).  The call makes no hipMalloc/hipFree and no other
 * allocating call; it clears what must start at zero with a kernel on the caller's
 * stream.  Every call on one device shares that device's array: calls that overlap on
 * one device (other threads, other streams) race and must be serialised by the caller.
 * Measurement mode (pnr_profile_enable) does not apply to this entry point.
 */
#define PNR_STATIC_SCRATCH_BYTES ((size_t)64 << 20)
int pnr_eval_static(const pnr_cell* cell, const pnr_params* params, const void* x, const void* h0,
                    void* h_out, int max_iters, double tol, int jac_mode);

/*
 * pnr_eval with a bounded iteration, for the diagonal-recurrence cells (PNR_CELL_GRU_DIAG,
 * PNR_CELL_LSTM_DIAG).  Undamped Newton can diverge ("Towards Scalable and Stable
 * Parallelization of Nonlinear RNNs", summary page, "Problem"): from the zero guess the
 * linearised recurrence of a stiff cell can be so expansive that the step overflows.
 * Here each new iterate is projected onto the box every reachable state lies in -- a
 * safeguard of this library's own, not the pages' damping -- and a component the step
 * made NaN keeps its current value:
 *     GRU_DIAG:   |h_t| <= max(1, |h0|)      (h' is a convex combination of tanh(.) and h)
 *     LSTM_DIAG:  |h_t| <= 1,  |c_t| <= |c0| + t      (t = 1..T)
 * The true states lie inside the box, so the projection never moves them: every property
 * of pnr_eval's iteration that rests on them holds (after k updates the first k states
 * are exact; the fixed point is the sequential trajectory), and iterates that stay inside
 * are pnr_eval's, bit for bit.  Arguments, workspace (pnr_workspace_bytes), jac_mode,
 * jac_every and results as pnr_eval; the dense-U GRU returns PNR_E_UNSUPPORTED.
 */
int pnr_eval_bounded(const pnr_cell* cell, const pnr_params* params, const void* x, const void* h0,
                     void* h_out, int max_iters, double tol, int jac_mode);

/*
 * pnr_eval with a low-rank approximation of the Jacobian, for the GRU with a dense
 * recurrent matrix (PNR_CELL_GRU; D <= 32, the sizes its dense Jacobian supports).  The
 * ParaRNN overview page ("Technical Implementation / Newton's Iteration") names low-rank
 * approximations among the approximate-Newton strategies, with no form; this library's
 * reading keeps the exact Jacobian's structure
 *     J_t = diag(z) + diag(al) U_z + diag(be) U_r + diag(ga) U_n
 * and replaces, in the Jacobian only, each gate block U_g by its best rank-`rank`
 * approximation (truncated singular value decomposition; computed on the device, once
 * per call, from the Gram matrix U_g^T U_g by the cyclic Jacobi eigenvalue method), with
 * U_g's own diagonal restored so that the Jacobian's diagonal stays exact.  The gates and
 * residuals still use U.  rank = D is pnr_eval's dense Jacobian (Newton); rank = 0 its
 * diagonal (quasi-Newton).  rank must be in [0, D] (PNR_E_INVALID).  Other arguments and
 * results as pnr_eval with jac_mode = PNR_JAC_FULL (cell->jac_every honoured).
 * Workspace: pnr_workspace_bytes_lowrank() bytes (pnr_workspace_bytes(cell, FULL) plus the
 * approximated factors, 3 D^2 state elements); 0 = invalid or unsupported request.
 */
size_t pnr_workspace_bytes_lowrank(const pnr_cell* cell, int rank);
int pnr_eval_lowrank(const pnr_cell* cell, const pnr_params* params, const void* x, const void* h0,
                     void* h_out, int max_iters, double tol, int rank);

/* Newton updates applied by the calling thread's last pnr_eval (-1 if it failed before). */
int pnr_iters_used(void);

/* rho of the state returned by the calling thread's last pnr_eval (NaN if none). */
double pnr_last_residual(void);

/*
 * Copies the residual history rho_0..rho_iters of the last pnr_eval (at most max_n
 * values) into host memory `out`; returns how many values that history has.
 */
int pnr_last_residual_history(double* out, int max_n);

/* Text of the calling thread's last error ("" if none).  Valid until the next call. */
const char* pnr_last_error(void);

/*
 * Damped Newton evaluation: ELK / quasi-ELK ("Towards Scalable and Stable
 * Parallelization of Nonlinear RNNs", abstract; summary page, "Approach": a
 * Levenberg-Marquardt trust region whose linear-Gaussian MAP solve is a Kalman filter
 * and smoother; with the diagonal Jacobian, quasi-ELK; "Limitations": the trust-region
 * strength is a hyperparameter).  Same iteration, stopping test and results as
 * pnr_eval, except that the update d minimises
 *     sum_t |d_t - J_t d_{t-1} - r_t|^2 + damping * sum_t |d_t|^2      (d_0 = 0)
 * instead of solving d_t = J_t d_{t-1} + r_t (damping -> 0 gives pnr_eval's step).  With
 * a diagonal J_t this splits into one scalar problem per state component, solved by a
 * Kalman filter (forward scan) and RTS smoother (backward scan).  The step is always
 * taken (fixed damping, no adaptive trust region).
 * Supported, with jac_every = 1 and (x, state) as for pnr_eval:
 *   PNR_CELL_GRU_DIAG, jac_mode PNR_JAC_FULL or PNR_JAC_DIAG (its exact Jacobian is
 *     diagonal, so both are ELK);
 *   PNR_CELL_LSTM_DIAG, jac_mode PNR_JAC_DIAG (quasi-ELK: the diagonal of the 2x2 block,
 *     dc'/dc and dh'/dh, per channel; h_out holds (c, h) as for pnr_eval);
 *   PNR_CELL_GRU (dense U), fp32 state, D <= 64, jac_mode PNR_JAC_DIAG (quasi-ELK: the
 *     diagonal of the dense Jacobian).  Each iteration is a host-driven sequence of
 *     launches (the recurrent GEMM, the cell, one 4-byte read-back of max |r|, the filter
 *     and smoother scans).
 * Others return PNR_E_UNSUPPORTED.  damping must be finite and > 0 (else PNR_E_INVALID).
 * Workspace: pnr_workspace_bytes_damped() bytes (the smoother's per-step gain and
 * offset take 8 bytes per state element more than pnr_eval).
 */
size_t pnr_workspace_bytes_damped(const pnr_cell* cell, int jac_mode);
int pnr_eval_damped(const pnr_cell* cell, const pnr_params* params, const void* x, const void* h0,
                    void* h_out, int max_iters, double tol, int jac_mode, double damping);

/*
 * Chunked evaluation (ParaRNN overview page, "Experimental Results", on long sequences:
 * the memory that stored hidden states take during the Newton iteration is kept in check
 * by chunking, together with gradient checkpointing).  The sequence is cut into consecutive
 * chunks of chunk_len steps (the last may be shorter).  Chunk c is evaluated exactly as
 * pnr_eval (damping == 0) or pnr_eval_damped (damping > 0) evaluates a sequence of its
 * length, with the same max_iters, tol and jac_mode per chunk, and with initial state
 * h0 for the first chunk and, for the others, the returned state at the previous chunk's
 * last step (h_out[b, t0 - 1]).  At convergence the result is the sequential one within
 * the tolerance, as for pnr_eval; the workspace covers one chunk instead of the whole
 * sequence (plus, for B > 1 with more than one chunk, contiguous staging of the chunk's
 * x, boundary state and output, copied on the stream).
 * Arguments and layouts as for pnr_eval / pnr_eval_damped; chunk_len >= 1; damping
 * finite and >= 0.  Results: the worst status over chunks (NONFINITE > NOT_CONVERGED >
 * OK; after a NONFINITE chunk the later chunks are not evaluated and their h_out
 * entries are left as they were); pnr_iters_used() = the sum of the chunks' iterations;
 * pnr_last_residual() = the largest final rho; pnr_last_residual_history() = the chunks'
 * histories one after another; in measurement mode (pnr_profile_enable) the profile
 * record holds sums over the chunks (resid_only: the number of chunks whose last pass
 * only evaluated the residual).  Synchronises the stream before returning.
 * pnr_workspace_bytes_chunked returns 0 for an invalid or unsupported request.
 */
size_t pnr_workspace_bytes_chunked(const pnr_cell* cell, int jac_mode, double damping, int chunk_len);
int pnr_eval_chunked(const pnr_cell* cell, const pnr_params* params, const void* x, const void* h0,
                     void* h_out, int max_iters, double tol, int jac_mode, double damping, int chunk_len);

/*
 * Backward pass: gradients through an evaluated sequence, for training through the
 * parallel evaluation ("Parallelizing non-linear sequential models over the sequence
 * length", abstract; ParaRNN overview, "Newton's Iteration": the block lower-triangular
 * system is solved by backward as well as forward substitution).  Given the states h
 * (e.g. pnr_eval's h_out at convergence) and g = dL/dh, the explicit loss gradient at
 * every state, it computes the gradients of L through the recurrence
 * s_t = f(s_{t-1}, x_t), s_0 = h0, taking h as its solution:
 *     lam_t = g_t + J_{t+1}^T lam_{t+1}   (lam_T = g_T; J exact, not approximated)
 * is run backwards in time as a scan, and each step's lam_t is sent back through the
 * cell's gates to the pre-activations, the recurrent weights and biases, the inputs
 * (through W) and h0.
 * Supported: PNR_CELL_GRU_DIAG and PNR_CELL_LSTM_DIAG (the adjoint is one scan: status
 * PNR_OK, pnr_iters_used() = 0), and PNR_CELL_GRU with D <= 64, whose dense Jacobians
 * couple the channels: there the adjoint system is solved by quasi-Newton refinement
 * ("Towards Scalable and Stable Parallelization of Nonlinear RNNs", abstract: the
 * diagonal approximation, here as the preconditioner of a diagonal scan, with the dense
 * J^T lam of each residual on MFMA) from lam = 0 until max |residual| <= 2e-5 max |g|,
 * checked after every group of 4 iterations, at most 256.  Status PNR_OK,
 * PNR_NOT_CONVERGED (gradients of the last iterate) or PNR_NONFINITE;
 * pnr_iters_used() = refinement updates applied (up to 3 past the passing check),
 * pnr_last_residual_history() = the residuals up to the passing one.  x in {f32, bf16}, state f32; the
 * cell's jac_every is ignored.  Device pointers, caller-owned; each gradient output may
 * be NULL (not computed); all gradients are fp32 and overwritten (not accumulated):
 *   h, grad_h  [B, T, S]   fp32, inputs (S = D, or 2D for the LSTM's (c, h))
 *   grad_x     [B, T, D_in]     grad_W    [G*D, D_in]     grad_U   as U ([3D, D] or [G, D])
 *   grad_b_x   [G*D]            grad_b_h  [G*D]           grad_h0  [B, S]
 * x, h0, params as for pnr_eval (h0 may be NULL: zeros).  Workspace:
 * pnr_workspace_bytes_backward() bytes (0 = invalid or unsupported request).  For the
 * diagonal cells the work is enqueued on cell->stream and the call returns without
 * waiting for it; the dense GRU's refinement reads its residual back every iteration
 * and the call returns with the work still enqueued for the final gradients.  In
 * measurement mode the profile record holds: proj_ms the recomputed gate
 * pre-activations, newton_ms the adjoint (scan kernel, or the refinement loop with its
 * read-backs), out_ms the reductions and gradient GEMMs.
 */
size_t pnr_workspace_bytes_backward(const pnr_cell* cell);
int pnr_backward(const pnr_cell* cell, const pnr_params* params, const void* x, const void* h0,
                 const void* h, const void* grad_h, void* grad_x, void* grad_W, void* grad_U,
                 void* grad_b_x, void* grad_b_h, void* grad_h0);

/*
 * pnr_backward with a choice of Jacobian in the adjoint recursion.  jac_mode PNR_JAC_FULL is
 * pnr_backward (the exact gradients).  PNR_JAC_DIAG is the diagonal approximation in the
 * backward pass ("Towards Scalable and Stable Parallelization of Nonlinear RNNs", summary
 * page, "Measured effects": diagonal Jacobian approximations "including in the backward
 * pass"): the adjoint carries diag(J_{t+1}) lam_{t+1} instead of J_{t+1}^T lam_{t+1}
 * (grad_h0 = diag(J_1) lam_1 likewise), while every step still sends its lam_t back
 * through the cell's gates exactly; the gradients are those approximate adjoints' (exact
 * for PNR_CELL_GRU_DIAG, whose Jacobian is diagonal).  For the dense GRU it is one
 * diagonal scan instead of the refinement: pnr_iters_used() = 1, pnr_last_residual() = 0.
 * Other jac_mode values return PNR_E_INVALID.  Arguments, workspace
 * (pnr_workspace_bytes_backward) and results otherwise as pnr_backward.
 */
int pnr_backward_approx(const pnr_cell* cell, const pnr_params* params, const void* x, const void* h0,
                        const void* h, const void* grad_h, void* grad_x, void* grad_W, void* grad_U,
                        void* grad_b_x, void* grad_b_h, void* grad_h0, int jac_mode);

/*
 * Backward pass over chunks, the gradient-checkpointing half of chunked evaluation
 * (ParaRNN overview page, "Experimental Results": chunking together with gradient
 * checkpointing keeps the memory of long sequences in check).  The sequence is cut into
 * consecutive chunks of chunk_len steps (the last may be shorter), as pnr_eval_chunked
 * cuts it, and the chunks are processed last to first, each by pnr_backward on the
 * chunk's steps, with initial state h0 for the first chunk and h[b, t0 - 1] for the
 * others.  The adjoint crossing a boundary, J^T lam of the later chunk's first step
 * (that chunk's grad_h0), is added to grad_h at the earlier chunk's last step, so that
 * the result is pnr_backward's on the whole sequence up to rounding (and, for the dense
 * GRU, up to each chunk's refinement tolerance).  Weight and bias gradients are summed
 * over chunks; grad_x and the first chunk's grad_h0 are written per chunk.  Arguments,
 * layouts and NULL outputs as for pnr_backward; chunk_len >= 1.  Workspace:
 * pnr_workspace_bytes_backward_chunked() bytes (0 = invalid or unsupported request): one
 * chunk's pnr_backward workspace, the chunk's grad_h, two B x S boundary adjoints, one
 * set of weight-gradient partials and, for B > 1 with more than one chunk, contiguous
 * staging of the chunk's x, h and grad_x.  Results: the worst status over chunks
 * (NONFINITE > NOT_CONVERGED > OK; every chunk is processed); pnr_iters_used() = the
 * sum of the chunks' refinement iterations; pnr_last_residual() = the largest;
 * pnr_last_residual_history() = the chunks' histories, last chunk first; the profile
 * record holds sums over chunks.  Synchronises the stream before returning.
 */
size_t pnr_workspace_bytes_backward_chunked(const pnr_cell* cell, int chunk_len);
int pnr_backward_chunked(const pnr_cell* cell, const pnr_params* params, const void* x,
                         const void* h0, const void* h, const void* grad_h, void* grad_x,
                         void* grad_W, void* grad_U, void* grad_b_x, void* grad_b_h,
                         void* grad_h0, int chunk_len);

/*
 * Standalone linear solve used inside every Newton iteration, exposed for testing
 * the scan on its own: d_t = A_t d_{t-1} + b_t, d_0 = 0 along t, for R independent
 * rows (ParaRNN overview, "Newton's Iteration": forward substitution on the block
 * lower-triangular system).  fp32, device pointers:
 *   kind 1 (diagonal):  A, b, d are [R, T]
 *   kind 2 (2x2 block): A is [R, 4, T] (a00, a01, a10, a11 planes), b and d [R, 2, T]
 * tile_len (0 = library default) sets the per-block tile along T; smaller tiles mean
 * more blocks linked by the decoupled look-back.  workspace as for pnr_eval, size
 * from pnr_scan_workspace_bytes.  Synchronises the stream before returning.
 */
size_t pnr_scan_workspace_bytes(int kind, int R, int T, int tile_len);
int pnr_scan(int kind, int R, int T, const float* A, const float* b, float* d, int tile_len,
             void* workspace, size_t workspace_bytes, void* stream);

/*
 * Per-phase timing of the calling thread's pnr_eval calls, for measurement only.  When
 * enabled (pnr_profile_enable(1)), pnr_eval records a HIP event before and after each
 * of its kernel launches on the caller's stream and, after its final synchronisation,
 * fills the record below (milliseconds of GPU time between those events).  The whole
 * Newton loop is one launch; `passes` counts the fused passes it ran (one per
 * residual evaluated: iters + 1).  Disabled by default; enabling it adds one event pair
 * per launch.  pnr_last_profile returns 0, or -1 if no profiled call completed.
 */
typedef struct pnr_profile {
  double total_ms;       /* first launch to last launch of the call                    */
  double proj_ms;        /* input projection                                            */
  double newton_ms;      /* the persistent Newton-loop kernel                           */
  double out_ms;         /* conversion of the returned iterate to h_out                 */
  int32_t passes;        /* fused passes of the Newton kernel (iters + 1)               */
  int32_t resid_only;    /* 1 if the last pass only evaluated the residual (max_iters)  */
} pnr_profile;

int pnr_profile_enable(int on);
int pnr_last_profile(pnr_profile* out);

#ifdef __cplusplus
}
#endif

#endif /* PNR_H */
