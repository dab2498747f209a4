// Internal launch interface between the host driver and the HIP kernels of libpnr.
#pragma once

#include "common.h"

namespace pnr {

// Upper bound on the grid of any persistent iteration kernel (sizes the partials array).
constexpr int kMaxGrid = 16384;
// rows of padding after the gate-input region: the longest dense tile, so a tile's rows
// past the end of the sequence can be read (and masked) without a bounds branch
constexpr int kGxPadRows = 128;

// Resident blocks of `fn` per CU with `lds` bytes of dynamic LDS (raising the kernel's
// LDS limit first when needed), 0 when it cannot run.  Cached per (kernel, LDS size):
// the runtime queries cost tens of microseconds per call.
// `threads`: the kernel's block size (most persistent kernels use PNR_BLOCK).
int cached_occupancy(const void* fn, size_t lds, int threads = PNR_BLOCK);
// launch of a grid sized to the resident capacity (cooperative, or ordinary when
// PNR_COOPERATIVE=0), with blocks of `threads` threads
hipError_t launch_persistent(const void* fn, int grid, size_t lds, void** args, hipStream_t st,
                             int threads = PNR_BLOCK);

// ---------------------------------------------------------------------------------
// Decision taken by the block that merges the residual partials of iteration k (the
// "final block" of the two-level reduction): record rho_k and stop when it is within
// tol, not finite, or when k is the residual-only pass after max_iters updates.
//
// Every field of the control block is written with agent-scope (coherent) stores: the
// merging block differs from pass to pass and may sit on another XCD, and plain stores
// of one address from several XCDs' L2 caches reach memory in no defined order.
// refresh_ratio >= 0: also decide the adaptive Jacobian refresh of pass k+1, which takes
// a new Jacobian when the current one has jac_every updates of age or when this update
// contracted the residual by less than the ratio (rho_k > ratio * rho_{k-1}, k >= 1;
// c->rho still holds rho_{k-1} here).  Pass 0 always takes one; c->jac_pass records the
// last pass that did.
__device__ inline void finish_iteration(Ctrl* c, double* hist, double rho, int k, int cur_buf,
                                        int max_iters, double tol, double refresh_ratio = -1.0,
                                        int jac_every = 1) {
  hist[k] = rho;
  if (refresh_ratio >= 0.0) {
    const double prev = __hip_atomic_load(&c->rho, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const int last = __hip_atomic_load(&c->jac_pass, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const bool next = (k + 1 - last >= jac_every) || (k >= 1 && rho > refresh_ratio * prev);
    __hip_atomic_store(&c->refresh, next ? 1 : 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (next) __hip_atomic_store(&c->jac_pass, k + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __hip_atomic_store(&c->rho, rho, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  int done = 0, status = PNR_NOT_CONVERGED;
  if (!(rho < __builtin_inf())) {
    done = 1; status = PNR_NONFINITE;
  } else if (rho <= tol) {
    done = 1; status = PNR_OK;
  } else if (k >= max_iters) {
    done = 1; status = PNR_NOT_CONVERGED;
  }
  if (done) {
    __hip_atomic_store(&c->status, status, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(&c->iters, k, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(&c->result_buf, cur_buf, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    // every block reads `done` right after the barrier: publish it coherently
    __hip_atomic_store(&c->done, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// ---------------------------------------------------------------------------------
struct DiagLoopArgs {
  const float* gx;     // [B][G][D][T]
  const float* u;      // [G][D]
  const float* bh;     // [G*D] or nullptr
  const float* h0;     // [B][S] or nullptr
  float* H[3];         // state buffers [B][S][T]
  int nbuf;            // 2, or 3 when the Jacobian is reused
  uint64_t* slots;     // look-back slots, n_tiles * slot words
  uint32_t* partials;  // per-block residual maxima
  Ctrl* ctrl;
  double* rho_hist;
  int B, D, T;
  int tiles_per_row;
  int n_tiles;         // B * D * tiles_per_row
  int n_rows;          // B * D
  int walk;            // 1: one block walks a whole row with a carry; 0: tiles + look-back
  int max_iters, jac_every, jac_mode;
  double tol;
  double refresh_ratio;   // >= 0: adaptive Jacobian refresh (jac_every = largest age); < 0: fixed schedule
  int bounded;            // 1: each new iterate projected onto the reachable-state box
};

// Damped (quasi-ELK) Newton loop for GRU_DIAG and LSTM_DIAG (G gates, S = D or 2D state
// components per batch element): one block walks a whole row (channel) per pass, a
// forward (filter) and a backward (smoother) sweep over its tiles.
struct ElkArgs {
  const float* gx;     // [B][G][D][T]
  const float* u;      // [G][D]
  const float* bh;     // [G*D] or nullptr
  const float* h0;     // [B][S] or nullptr
  float* H[2];         // state buffers [B][S][T]
  float* Gs;           // smoother gain per step [B][S][T]
  float* Es;           // smoother offset per step, in new-iterate space [B][S][T]
  uint32_t* partials;  // per-block residual maxima
  Ctrl* ctrl;
  double* rho_hist;
  int B, D, T;
  int tiles_per_row;
  int n_rows;          // B * D
  int max_iters, jac_mode;
  double tol;
  float lam;           // damping (> 0)
};
int elk_items_per_thread();
hipError_t launch_elk_diag(int cell, const ElkArgs& a, int num_cu, hipStream_t st);
// ELK proper for LSTM_DIAG: the exact 2x2 Jacobian block per channel; Gs holds the 2x2
// smoother gain as [B][4][D][T] and Es the offset as [B][2][D][T]
hipError_t launch_elk2_lstm(const ElkArgs& a, int num_cu, hipStream_t st);

// Backward pass of the diagonal-recurrence cells (GRU_DIAG, LSTM_DIAG): the adjoint
// scan run backwards in time with the per-step gate gradients; one block walks a row.
struct BwdArgs {
  const float* gx;     // [B][G][D][T] pre-activations from the input projection
  const float* u;      // [G][D]
  const float* bh;     // [G*D] or nullptr
  const float* h0;     // [B][S] or nullptr
  const float* hT;     // states [B][S][T]
  const float* gT;     // dL/ds [B][S][T]
  void* dgx;           // out: dL/d(pre-activation) [G*D][B*T], fp32 or (dgx_bf16) bf16
  float* part;         // out: per batch element sums [B][3][G][D] (dU, db_h, db_x)
  float* dh0;          // out: dL/dh0 [B][S] or nullptr
  int B, D, T;
  int tiles_per_row;
  int n_rows;          // B * D
  int dgx_bf16;
  int jdiag;           // 1: the adjoint carries diag(J) mu (the diagonal approximation), not J^T mu
};
int adjoint_items_per_thread();
hipError_t launch_adjoint_diag(int cell, const BwdArgs& a, int num_cu, hipStream_t st);

// Backward pass of the dense GRU (dense_bwd.hip): the adjoint solved by quasi-Newton
// refinement (diagonal scan + one GEMM per iteration).  Layouts [B][T][D] / [B][T][3D].
hipError_t launch_gru_shift_states(const float* h, const float* h0, float* hprev, int B, int T, int D,
                                   hipStream_t st);
// F: six [B*T][D] planes (z, diag J, f_z, f_n, r, f_r)
hipError_t launch_gru_bwd_factors(const float* gx, const float* gh, const float* hprev, const float* U, float* F,
                                  size_t n, int D, hipStream_t st);
hipError_t launch_gru_bwd_gates(const float* F, const float* lam, float* dgh, float* dgx, size_t n, int D,
                                hipStream_t st);
// One refinement step of the dense adjoint in the [B][T][D] layout (D <= 64): residual
// (max |R| into rmax), the diagonal scan over chunks of 64 steps, lam_new = lam + delta,
// and dgh of lam_new.  agg: B * chunks * D float2, carry: B * chunks * D floats.
hipError_t launch_gru_bwd_refine(const float* F, const float* lam, const float* v, const float* g, float* lam_new,
                                 float* dgh, float2* agg, float* carry, uint32_t* rmax, int B, int T, int D,
                                 hipStream_t st);
int gru_bwd_chunks(int T);
// The dense GRU's adjoint refinement as one persistent loop (D <= 64): lam[0], v[0] and
// bnd start at zero; on return ctrl and hist hold the decision as for the Newton loops,
// and lam[ctrl->result_buf] is the adjoint whose residual passed.
struct BwdLoopArgs {
  const float* F;      // gate factors [6][B*T*D]: z, d, f_z, f_n, r, f_r
  const float* g;      // dL/dh [B][T][D]
  const float* U;      // [3D][D]
  float* lam[2];       // adjoint iterates [B][T][D]; lam[0] zero at launch
  float* v[2];         // U^T dgh(lam) [B][T][D]; v[0] zero at launch
  float* agg;          // chunk maps (P, Q) [B][D][nch][2]
  float* carry;        // delta at the first step after each chunk [B][nch][D]
  float* bnd;          // per chunk, lam of the iterate at the step after it [B][nch][D]; zero at launch
  uint32_t* rmax;      // max |R| of each iteration as ordered bits [max_iters + 1]; zero at launch
  Ctrl* ctrl;          // zero at launch
  double* hist;        // [max_iters + 1]
  int B, T, D, nch, max_iters;
  double tol_rel;      // stop when rho_k <= tol_rel * rho_0
};
hipError_t launch_gru_bwd_loop(const BwdLoopArgs& a, int num_cu, hipStream_t st);
hipError_t launch_gru_bwd_dh0(const float* F, const float* lam, const float* v, float* dh0, int B, int T, int D,
                              hipStream_t st);
// C [M][N] = A [M][K] B[N][K]^T (fp32) for a long K and small M x N: K cut into at most
// max_slices slices summed from `part` (max_slices * M * N floats).
constexpr int kSplitKSlices = 64;
hipError_t launch_gemm_split_k(const float* A, int lda, const float* Bm, int ldb, float* C, int M, int N, int K,
                               float* part, int max_slices, hipStream_t st);
// out[r] = sum over the cols of row r of M [rows][cols], in 32 column segments per row
// (partials in `part`: 32 * rows floats) summed in a fixed order
hipError_t launch_row_sum(const float* M, int rows, size_t cols, float* out, float* part, hipStream_t st);

// Damped (quasi-ELK) loop of the dense GRU (dense_elk.hip), [B][T][D] layout, D <= 64: one
// persistent, co-resident grid runs every iteration and records the decision in ctrl.
int elk_dense_chunks(int T);
struct ElkLoopArgs {
  const float* gx;     // x W^T + b_x [B][T][3D]
  const float* U;      // [3D][D]
  const float* bh;     // [3D] or nullptr
  const float* h0;     // [B][D] or nullptr
  float* H[2];         // iterates [B][T][D]; H[0] holds the zero guess at launch
  float* R;            // residual of the iterate [B][T][D]
  float* J;            // quasi Jacobian of the iterate [B][T][D]
  float* G;            // smoother gain [B][T][D]
  float* E;            // smoother offset [B][T][D]
  float* agg;          // filter chunk maps [B][D][nch][8]
  float* carry;        // filter state (u, n) entering each chunk [B][nch][2][D]
  float* agg2;         // smoother chunk maps (P, Q) [B][D][nch][2]
  float* carry2;       // smoothed state at the step after each chunk [B][nch][D]
  float* head;         // (J, R, h) at each chunk's first step [B][nch][3][D]
  float* tailge;       // (G, e) at each chunk's last step [B][nch][2][D]
  float* hb;           // state before each chunk's first step [B][nch][D]; zero at launch
  uint32_t* rmax;      // max |R| of each iteration as ordered bits [max_iters + 1]; zero at launch
  Ctrl* ctrl;          // zero at launch
  double* hist;        // [max_iters + 1]
  int B, T, D, nch, max_iters;
  float lam;           // damping
  double tol;          // stop when rho_k <= tol
};
hipError_t launch_gru_elk_loop(const ElkLoopArgs& a, int num_cu, hipStream_t st);
// out [n] = H[ctrl->result_buf] (the loop's decision, read on the device)
hipError_t launch_elk_dense_output(const float* H0, const float* H1, const Ctrl* ctrl, float* out, size_t n,
                                   hipStream_t st);

int diag_items_per_thread(int cell);
int diag_slot_words(int cell);
int diag_grid_capacity(int cell, int num_cu);
hipError_t launch_diag_newton(int cell, const DiagLoopArgs& a, int grid, hipStream_t st);

// ---------------------------------------------------------------------------------
template <typename Tt>
struct DenseLoopArgs {
  const Tt* gx;        // [B][T][3D]
  // When x is set, the loop kernel computes gx itself (writing gx_out == gx) from
  // x [B][T][D_in], W [3D][D_in] and bx [3D] (or nullptr) before its first pass.
  const Tt* x;
  const Tt* W;
  const Tt* bx;
  Tt* gx_out;
  int D_in;
  const Tt* U;         // [3D][D]
  const Tt* Uj;        // the Jacobian's matrix factors [3D][D] (low-rank approximation); nullptr: U
  const Tt* bh;        // [3D] or nullptr
  const Tt* h0;        // [B][D] or nullptr
  Tt* H[4];            // state buffers [B][T][D] (dense_state_buffers of them)
  Tt* out;             // resident mode only: the caller's h_out, written by the loop kernel
  int nbuf;
  uint64_t* slots;
  uint64_t* partials;  // kPartialWords
  Ctrl* ctrl;
  double* rho_hist;
  int B, D, T;
  int L;               // steps per tile
  int tiles_per_row;
  int n_tiles;
  int max_iters, jac_every, jac_mode;
  double tol;
};

// U^ [3D][D] of the low-rank Jacobian: every gate block of U truncated to rank r (its r
// leading singular directions), its diagonal reset to U's own (D <= 32; r >= D copies U).
template <typename Tt>
hipError_t launch_lowrank_matrix(const Tt* U, Tt* Uh, int D, int rank, hipStream_t st);

// Tile length, look-back slot words per tile and number of [B][T][D] state buffers for
// the dense GRU path.
int dense_state_buffers(int D, int full, int is_f64, int reuse);
int dense_tile_len(int D, int full, int is_f64);
int dense_slot_words(int D, int full, int is_f64);
size_t dense_lds_bytes(int D, int full, int is_f64, int reuse, int lowrank = 0);
int dense_supported(int D, int full, int is_f64);
hipError_t launch_dense_newton_f32(const DenseLoopArgs<float>& a, int full, int num_cu, hipStream_t st);
// MFMA kernels (fp32; diagonal Jacobian with D in {16, 32, 64}, dense Jacobian with D = 16)
int dense_mfma_supported(int D, int full, int is_f64);
int dense_mfma_tile_len();
int dense_mfma_slot_words(int D, int full);
hipError_t launch_dense_mfma(const DenseLoopArgs<float>& a, int full, int num_cu, hipStream_t st);
// Tile length of the resident variant when every tile can own a co-resident block (and
// the variant applies), else 0.  The caller then sets DenseLoopArgs::L and ::out (the
// loop kernel writes h_out itself) and skips the output kernel.
int dense_mfma_resident_tile(int D, int full, int B, int T, int reuse, int num_cu);
hipError_t launch_dense_newton_f64(const DenseLoopArgs<double>& a, int full, int num_cu, hipStream_t st);

// ---------------------------------------------------------------------------------
// Input projection C[z][i][j] = sum_k A[z][i][k] * Bm[z][j][k] + bias, both operands
// K-contiguous; bias indexed by i (bias_on_i) or j.  C row-major with leading dim ldc.
struct GemmArgs {
  const void* A; const void* Bm; const void* bias; void* C;
  int M, N, K;
  long long sA, sB, sC;   // batch strides in elements (0 = shared)
  int lda, ldb, ldc;
  int batch;
  int bias_on_i;
};
hipError_t launch_gemm(int in_dtype, int out_dtype, const GemmArgs& g, hipStream_t st);

// ---------------------------------------------------------------------------------
// Misc: control/slot initialisation and the output layout conversion.
// Per-block residual words: three per block (one per pass modulo 3) for the barrier-free
// loops, which tag each word with its pass.
constexpr size_t kPartialWords = 3 * (size_t)kMaxGrid;
// [Z][R][C] -> [Z][C][R]; in and out each PNR_F32 or PNR_BF16 (round to nearest even).
hipError_t launch_transpose(const void* in, int in_dtype, void* out, int out_dtype, int Z, int R, int C,
                            hipStream_t st);
// p[0..n) = 0 (a kernel, so that the call can sit in a captured graph).
hipError_t launch_fill_zero(float* p, size_t n, hipStream_t st);
// out_q[j] = sum_b part[b][q][j], q = 0..2, j < n (null outputs are skipped).
hipError_t launch_sum_over_batch(const float* part, int B, int n, float* o0, float* o1, float* o2, hipStream_t st);
hipError_t launch_init(Ctrl* ctrl, uint64_t* slots, size_t slot_words, uint64_t* partials, size_t partial_words,
                       hipStream_t st);
// diag layout [B][S][T] -> h_out [B][T][S] (or zeros when the result is the zero guess)
hipError_t launch_diag_output(const float* const* bufs, const Ctrl* ctrl, float* h_out, int B, int S,
                              int T, hipStream_t st);
template <typename Tt>
hipError_t launch_dense_output(const Tt* const* bufs /* 4 */, const Ctrl* ctrl, Tt* h_out, size_t n,
                               hipStream_t st);

// Standalone scan (testing entry point)
hipError_t launch_scan(int kind, int R, int T, const float* A, const float* b, float* d, int tile_len,
                       uint64_t* slots, Ctrl* ctrl, int num_cu, hipStream_t st);
int scan_default_tile(int kind);
int scan_slot_words(int kind);

}  // namespace pnr
