// Host side of the C ABI declared in include/pnr.h.
//
// pnr_eval validates its arguments without touching HIP, carves the caller's workspace,
// then enqueues on the caller's stream:
//   init -> input projection (a GEMM, or inside the loop kernel for the quasi-Newton
//   dense GRU) -> one persistent launch running every Newton iteration -> output layout
//   conversion (unless the loop kernel wrote h_out) -> one control read-back.
// The loop decides on the device when to stop, so the host never waits between
// iterations (ParaRNN overview page, "Technical Implementation": Newton iterations with
// a residual check).
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <mutex>
#include <string>
#include <vector>

#include "common.h"
#include "kernels.h"

using namespace pnr;

namespace {

// Residual history of the calling thread's last call.  A single solve (max_iters <
// PNR_MAX_ITERS) fits the fixed part, so recording it touches no heap; only the chunked
// calls, which concatenate one history per chunk, may spill into the heap-backed tail.
class History {
 public:
  void clear() {
    n_ = 0;
    tail_.clear();
  }
  size_t size() const { return n_ + tail_.size(); }
  double operator[](size_t i) const { return i < n_ ? head_[i] : tail_[i - n_]; }
  void push_back(double v) {
    if (n_ < kHead && tail_.empty())
      head_[n_++] = v;
    else
      tail_.push_back(v);
  }
  void assign(const double* b, const double* e) {
    clear();
    for (; b != e; ++b) push_back(*b);
  }
  void assign(size_t n, double v) {
    clear();
    for (size_t i = 0; i < n; ++i) push_back(v);
  }

 private:
  static constexpr size_t kHead = PNR_MAX_ITERS + 1;
  double head_[kHead];
  size_t n_ = 0;
  std::vector<double> tail_;
};

struct LastCall {
  int iters = -1;
  double residual = NAN;
  History hist;
  char err[512] = {0};
  void reset() {
    iters = -1;
    residual = NAN;
    hist.clear();
    err[0] = 0;
  }
};
thread_local LastCall g_last;

int fail(int code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last.err, sizeof g_last.err, fmt, ap);
  va_end(ap);
  return code;
}

size_t align_up(size_t v, size_t a = 256) { return (v + a - 1) / a * a; }
size_t dsize(int dt) { return dt == PNR_F64 ? 8 : (dt == PNR_F32 ? 4 : 2); }

bool is_diag_cell(int kind) { return kind == PNR_CELL_GRU_DIAG || kind == PNR_CELL_LSTM_DIAG; }
int gates(int kind) { return kind == PNR_CELL_LSTM_DIAG ? 4 : 3; }
int states(int kind, int D) { return kind == PNR_CELL_LSTM_DIAG ? 2 * D : D; }

struct Layout {
  size_t ctrl = 0, hist = 0, partials = 0, slots = 0, gx = 0, h[4] = {0, 0, 0, 0}, total = 0;
  size_t slot_words = 0;
  int nbuf = 2, tiles_per_row = 0, n_tiles = 0, L = 0;
  bool dense_full = false;
};

// Validate the request; returns 0 or a negative status with the reason recorded.
int validate(const pnr_cell* c, int jac_mode) {
  if (!c) return fail(PNR_E_INVALID, "cell descriptor is NULL");
  if (c->kind < PNR_CELL_GRU || c->kind > PNR_CELL_LSTM_DIAG) return fail(PNR_E_INVALID, "unknown cell kind %d", c->kind);
  if (jac_mode < PNR_JAC_FULL || jac_mode > PNR_JAC_ZERO) return fail(PNR_E_INVALID, "unknown jac_mode %d", jac_mode);
  if (c->D < 1 || c->D_in < 1 || c->B < 1 || c->T < 0)
    return fail(PNR_E_INVALID, "sizes must satisfy D, D_in, B >= 1 and T >= 0 (got D=%d D_in=%d B=%d T=%d)", c->D,
                c->D_in, c->B, c->T);
  if (c->jac_every < 1) return fail(PNR_E_INVALID, "jac_every must be >= 1 (got %d)", c->jac_every);
  for (int dt : {c->x_dtype, c->state_dtype})
    if (dt < PNR_F64 || dt > PNR_BF16) return fail(PNR_E_INVALID, "unknown dtype %d", dt);
  const int xd = c->x_dtype, sd = c->state_dtype;
  if (c->kind == PNR_CELL_GRU) {
    const bool ok = (xd == PNR_F64 && sd == PNR_F64) || (xd == PNR_F32 && sd == PNR_F32) ||
                    (xd == PNR_BF16 && sd == PNR_F32);
    if (!ok) return fail(PNR_E_UNSUPPORTED, "GRU supports (x, state) dtypes (f64,f64), (f32,f32), (bf16,f32)");
    const int full = jac_mode == PNR_JAC_FULL;
    if (!dense_supported(c->D, full, sd == PNR_F64))
      return fail(PNR_E_UNSUPPORTED, "GRU with D=%d is not supported in this mode (%s, %s)", c->D,
                  full ? "dense Jacobian: D <= 32" : "diagonal Jacobian: D <= 64 (fp32) / 32 (fp64)",
                  sd == PNR_F64 ? "fp64" : "fp32");
  } else {
    const bool ok = (xd == PNR_F32 || xd == PNR_BF16) && sd == PNR_F32;
    if (!ok) return fail(PNR_E_UNSUPPORTED, "diagonal-recurrence cells support x in {f32, bf16} with f32 state");
  }
  const double elems = (double)c->B * c->T * states(c->kind, c->D);
  if (elems * gates(c->kind) > 9.0e18 || (double)c->T * 4 > 2.0e9)
    return fail(PNR_E_INVALID, "problem too large for this library's index range");
  return 0;
}

Layout make_layout(const pnr_cell* c, int jac_mode) {
  Layout l;
  const int G = gates(c->kind), S = states(c->kind, c->D);
  const size_t B = c->B, T = c->T, D = c->D;
  const size_t es = dsize(c->state_dtype);
  l.nbuf = c->jac_every > 1 ? 3 : 2;
  if (c->kind == PNR_CELL_GRU)
    l.nbuf = dense_state_buffers(c->D, jac_mode == PNR_JAC_FULL, c->state_dtype == PNR_F64, c->jac_every > 1);
  size_t off = 0;
  l.ctrl = off; off = align_up(off + sizeof(Ctrl));
  l.hist = off; off = align_up(off + sizeof(double) * (PNR_MAX_ITERS + 1));
  l.partials = off; off = align_up(off + sizeof(uint64_t) * kPartialWords);
  if (is_diag_cell(c->kind)) {
    const int tile = PNR_BLOCK * diag_items_per_thread(c->kind);
    l.tiles_per_row = (int)((T + tile - 1) / tile);
    l.n_tiles = (int)(B * D * l.tiles_per_row);
    l.slot_words = (size_t)l.n_tiles * diag_slot_words(c->kind);
  } else {
    l.dense_full = jac_mode == PNR_JAC_FULL;
    l.L = dense_tile_len(c->D, l.dense_full, c->state_dtype == PNR_F64);
    l.tiles_per_row = (int)((T + l.L - 1) / l.L);
    l.n_tiles = (int)(B * l.tiles_per_row);
    l.slot_words = (size_t)l.n_tiles * dense_slot_words(c->D, l.dense_full, c->state_dtype == PNR_F64);
  }
  l.slots = off; off = align_up(off + sizeof(uint64_t) * (l.slot_words ? l.slot_words : 1));
  // gx, plus kGxPadRows rows that the dense kernels may read (and mask) past the end
  l.gx = off; off = align_up(off + es * (B * T + (size_t)kGxPadRows) * (size_t)G * D);
  for (int i = 0; i < l.nbuf; ++i) { l.h[i] = off; off = align_up(off + es * B * T * (size_t)S); }
  l.total = off;
  return l;
}

// ---- optional per-launch timing (measurement mode) ----
struct Prof {
  bool on = false;
  bool valid = false;
  std::vector<hipEvent_t> pool;
  size_t used = 0;
  pnr_profile last{};
  hipEvent_t next() {
    if (used == pool.size()) {
      hipEvent_t e;
      if (hipEventCreate(&e) != hipSuccess) return nullptr;
      pool.push_back(e);
    }
    return pool[used++];
  }
};
thread_local Prof g_prof;

// Event pair around one launch group; no-op when profiling is off.
struct Mark {
  hipEvent_t a = nullptr, b = nullptr;
};
Mark mark_begin(hipStream_t st) {
  Mark m;
  if (!g_prof.on) return m;
  m.a = g_prof.next();
  if (m.a) (void)hipEventRecord(m.a, st);
  return m;
}
void mark_end(Mark& m, hipStream_t st) {
  if (!g_prof.on || !m.a) return;
  m.b = g_prof.next();
  if (m.b) (void)hipEventRecord(m.b, st);
}
double mark_ms(const Mark& m) {
  float ms = 0.f;
  if (!m.a || !m.b || hipEventElapsedTime(&ms, m.a, m.b) != hipSuccess) return 0.0;
  return ms;
}

// Row walk (no look-back) when the rows alone fill the resident grid evenly enough;
// PNR_DIAG_WALK=0/1 forces either organisation (used by the tests to cover both).
int walk_mode(int rows, int capacity) {
  const char* e = getenv("PNR_DIAG_WALK");
  if (e && (e[0] == '0' || e[0] == '1')) return e[0] == '1';
  return rows >= capacity && (rows % capacity == 0 || rows >= 4 * capacity);
}

struct DevInfo { int dev = -1; int num_cu = 0; };
thread_local DevInfo g_dev;

int device_info(int* num_cu) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return fail(PNR_E_HIP, "hipGetDevice failed");
  if (g_dev.dev != dev) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 1)
      return fail(PNR_E_HIP, "cannot query the compute-unit count");
    g_dev.dev = dev;
    g_dev.num_cu = n;
  }
  *num_cu = g_dev.num_cu;
  return 0;
}

#define PNR_HIP(call)                                                                     \
  do {                                                                                    \
    hipError_t e_ = (call);                                                               \
    if (e_ != hipSuccess) return fail(PNR_E_HIP, "%s failed: %s", #call, hipGetErrorString(e_)); \
  } while (0)

// The one device -> host crossing of a call: the control block and the residual
// history (adjacent in the workspace) in one copy into thread-local host storage (plain
// pageable memory of fixed size: the library holds no pinned host allocation, so nothing
// is left to release at exit), one stream synchronisation; then the call's results and,
// in measurement mode, its per-phase timing.  Returns the call's status.
// The history follows the control block after at most 255 bytes of alignment.
constexpr size_t kReadBackMax = sizeof(Ctrl) + 256 + sizeof(double) * (PNR_MAX_ITERS + 1);
int finish_call(size_t ctrl_off, size_t hist_off, char* ws, int max_iters, hipStream_t st, const Mark& m_first,
                const Mark& m_proj, const Mark& m_newton, const Mark& m_out) {
  alignas(64) static thread_local char rb[kReadBackMax];
  const size_t rb_bytes = (hist_off - ctrl_off) + sizeof(double) * (max_iters + 1);
  if (rb_bytes > kReadBackMax) return fail(PNR_E_INVALID, "control read-back of %zu bytes exceeds %zu", rb_bytes,
                                           kReadBackMax);
  PNR_HIP(hipMemcpyAsync(rb, ws + ctrl_off, rb_bytes, hipMemcpyDeviceToHost, st));
  PNR_HIP(hipStreamSynchronize(st));
  Ctrl hc;
  memcpy(&hc, rb, sizeof(Ctrl));
  const double* hh = reinterpret_cast<const double*>(rb + (hist_off - ctrl_off));
  if (hc.fault)
    return fail(PNR_E_HIP, "device loop gave up waiting (%s); results are not valid",
                hc.fault == 1 ? "look-back" : "grid barrier");
  if (!hc.done || hc.iters < 0) return fail(PNR_E_HIP, "device loop did not record a decision");
  g_last.iters = hc.iters;
  g_last.residual = hc.rho;
  g_last.hist.assign(hh, hh + hc.iters + 1);
  if (g_prof.on) {
    pnr_profile p{};
    p.total_ms = mark_ms(m_first);
    p.proj_ms = mark_ms(m_proj);
    p.newton_ms = mark_ms(m_newton);
    p.out_ms = mark_ms(m_out);
    p.passes = hc.iters + 1;
    p.resid_only = hc.iters == max_iters;
    g_prof.last = p;
    g_prof.valid = true;
  }
  return hc.status;
}

}  // namespace

extern "C" {

size_t pnr_workspace_bytes(const pnr_cell* cell, int jac_mode) {
  if (validate(cell, jac_mode) != 0) return 0;
  return make_layout(cell, jac_mode).total;
}

const char* pnr_last_error(void) { return g_last.err; }

int pnr_profile_enable(int on) {
  g_prof.on = on != 0;
  return 0;
}
int pnr_last_profile(pnr_profile* out) {
  if (!g_prof.valid || !out) return -1;
  *out = g_prof.last;
  return 0;
}
int pnr_iters_used(void) { return g_last.iters; }
double pnr_last_residual(void) { return g_last.residual; }
int pnr_last_residual_history(double* out, int max_n) {
  const int n = (int)g_last.hist.size();
  if (out)
    for (int i = 0; i < n && i < max_n; ++i) out[i] = g_last.hist[i];
  return n;
}

namespace {
// Argument checks shared by pnr_eval and its variants (no HIP call).
int check_eval_args(const pnr_cell* cell, const pnr_params* params, const void* x, const void* h_out,
                    int max_iters, double tol, int jac_mode) {
  int rc = validate(cell, jac_mode);
  if (rc) return rc;
  if (!params) return fail(PNR_E_INVALID, "params is NULL");
  if (!params->W || !params->U || (cell->T > 0 && (!x || !h_out)))
    return fail(PNR_E_INVALID, "W, U and (for T > 0) x and h_out must be non-NULL");
  if (max_iters < 0 || max_iters >= PNR_MAX_ITERS)
    return fail(PNR_E_INVALID, "max_iters must be in [0, %d)", PNR_MAX_ITERS);
  if (isnan(tol)) return fail(PNR_E_INVALID, "tol is NaN");
  return 0;
}

// The evaluation proper, on the scratch memory `ws` (at least make_layout(...).total bytes,
// 256-byte aligned; checked by the callers).
int eval_impl(const pnr_cell* cell, const pnr_params* params, const void* x, const void* h0, void* h_out,
              int max_iters, double tol, int jac_mode, double refresh_ratio, int bounded, int jac_rank, char* ws) {
  int rc = 0;
  const Layout l = make_layout(cell, jac_mode);
  // low-rank Jacobian (dense GRU): its matrix factors follow the layout
  void* Uh = jac_rank >= 0 ? ws + l.total : nullptr;
  if (cell->T == 0) {
    g_last.iters = 0;
    g_last.residual = 0.0;
    g_last.hist.assign(1, 0.0);
    return PNR_OK;
  }

  int num_cu = 0;
  if ((rc = device_info(&num_cu))) return rc;
  hipStream_t st = reinterpret_cast<hipStream_t>(cell->stream);
  Ctrl* ctrl = reinterpret_cast<Ctrl*>(ws + l.ctrl);
  double* hist = reinterpret_cast<double*>(ws + l.hist);
  uint64_t* slots = reinterpret_cast<uint64_t*>(ws + l.slots);
  void* gx = ws + l.gx;
  void* H[4] = {ws + l.h[0], ws + l.h[1], l.nbuf > 2 ? ws + l.h[2] : nullptr, l.nbuf > 3 ? ws + l.h[3] : nullptr};

  const int kind = cell->kind, D = cell->D, T = cell->T, B = cell->B, Din = cell->D_in;
  const int G = gates(kind), S = states(kind, D);

  Mark m_first = mark_begin(st);
  PNR_HIP(launch_init(ctrl, slots, l.slot_words, reinterpret_cast<uint64_t*>(ws + l.partials), kPartialWords, st));

  // ---- input projection ----
  GemmArgs g{};
  if (is_diag_cell(kind)) {
    // gx[b][m][t] = sum_k W[m][k] x[b][t][k] + b_x[m]
    g = GemmArgs{params->W, x, params->b_x, gx, G * D, T, Din, 0, (long long)T * Din, (long long)G * D * T,
                 Din, Din, T, B, 1};
  } else {
    // gx[(b,t)][m] = sum_k x[(b,t)][k] W[m][k] + b_x[m]
    g = GemmArgs{x, params->W, params->b_x, gx, B * T, G * D, Din, 0, 0, 0, Din, Din, G * D, 1, 0};
  }
  // The quasi-Newton dense GRU kernel (fp32 inputs) computes its tiles' projection itself,
  // saving a launch and a round trip of gx through the queue.
  const bool fused_proj = kind == PNR_CELL_GRU && cell->x_dtype == PNR_F32 && cell->state_dtype == PNR_F32 &&
                          !l.dense_full && dense_mfma_supported(D, 0, 0);
  Mark m_proj = mark_begin(st);
  if (!fused_proj) PNR_HIP(launch_gemm(cell->x_dtype, cell->state_dtype, g, st));
  mark_end(m_proj, st);

  // ---- the Newton loop: one persistent launch; the device decides when to stop ----
  bool out_written = false;
  Mark m_newton = mark_begin(st);
  if (is_diag_cell(kind)) {
    DiagLoopArgs a{};
    a.gx = static_cast<const float*>(gx);
    a.u = static_cast<const float*>(params->U);
    a.bh = static_cast<const float*>(params->b_h);
    a.h0 = static_cast<const float*>(h0);
    for (int i = 0; i < 3; ++i) a.H[i] = static_cast<float*>(H[i]);
    a.nbuf = l.nbuf;
    a.slots = slots;
    a.partials = reinterpret_cast<uint32_t*>(ws + l.partials);
    a.ctrl = ctrl;
    a.rho_hist = hist;
    a.B = B; a.D = D; a.T = T;
    a.tiles_per_row = l.tiles_per_row;
    a.n_tiles = l.n_tiles;
    a.n_rows = B * D;
    a.max_iters = max_iters; a.jac_every = cell->jac_every; a.jac_mode = jac_mode;
    a.tol = tol;
    a.refresh_ratio = refresh_ratio;
    a.bounded = bounded;
    const int cap = diag_grid_capacity(kind, num_cu);
    // A block walks whole rows (no look-back) when there are enough rows to fill the
    // grid; otherwise rows are cut into tiles linked by the decoupled look-back.
    a.walk = walk_mode(a.n_rows, cap);
    const int items = a.walk ? a.n_rows : a.n_tiles;
    int grid = items < cap ? items : cap;
    // a walking grid takes the largest divisor of the row count above half the capacity,
    // so that every block walks the same number of rows
    if (a.walk && items > cap)
      for (int g = cap; 2 * g > cap; --g)
        if (items % g == 0) {
          grid = g;
          break;
        }
    PNR_HIP(launch_diag_newton(kind, a, grid, st));
  } else if (cell->state_dtype == PNR_F32) {
    DenseLoopArgs<float> a{};
    a.gx = static_cast<const float*>(gx);
    a.U = static_cast<const float*>(params->U);
    if (Uh) {
      PNR_HIP(launch_lowrank_matrix<float>(a.U, static_cast<float*>(Uh), D, jac_rank, st));
      a.Uj = static_cast<const float*>(Uh);
    }
    a.bh = static_cast<const float*>(params->b_h);
    a.h0 = static_cast<const float*>(h0);
    for (int i = 0; i < 4; ++i) a.H[i] = static_cast<float*>(H[i]);
    a.nbuf = l.nbuf;
    a.slots = slots; a.partials = reinterpret_cast<uint64_t*>(ws + l.partials);
    a.ctrl = ctrl; a.rho_hist = hist;
    a.B = B; a.D = D; a.T = T; a.L = l.L;
    a.tiles_per_row = l.tiles_per_row; a.n_tiles = l.n_tiles;
    a.max_iters = max_iters; a.jac_every = cell->jac_every; a.jac_mode = jac_mode; a.tol = tol;
    if (fused_proj) {
      a.x = static_cast<const float*>(x);
      a.W = static_cast<const float*>(params->W);
      a.bx = static_cast<const float*>(params->b_x);
      a.gx_out = static_cast<float*>(gx);
      a.D_in = Din;
    }
    // resident variant: the loop kernel writes the returned iterate to h_out itself.  Its
    // tiles are at least as long as the layout's, so the slot region suffices.
    const int rtl = dense_mfma_resident_tile(D, l.dense_full, B, T, cell->jac_every > 1, num_cu);
    if (rtl > 0) {
      a.L = rtl;
      a.tiles_per_row = (T + rtl - 1) / rtl;
      a.n_tiles = B * a.tiles_per_row;
      a.out = static_cast<float*>(h_out);
      out_written = true;
    }
    PNR_HIP(launch_dense_newton_f32(a, l.dense_full, num_cu, st));
  } else {
    DenseLoopArgs<double> a{};
    a.gx = static_cast<const double*>(gx);
    a.U = static_cast<const double*>(params->U);
    if (Uh) {
      PNR_HIP(launch_lowrank_matrix<double>(a.U, static_cast<double*>(Uh), D, jac_rank, st));
      a.Uj = static_cast<const double*>(Uh);
    }
    a.bh = static_cast<const double*>(params->b_h);
    a.h0 = static_cast<const double*>(h0);
    for (int i = 0; i < 4; ++i) a.H[i] = static_cast<double*>(H[i]);
    a.nbuf = l.nbuf;
    a.slots = slots; a.partials = reinterpret_cast<uint64_t*>(ws + l.partials);
    a.ctrl = ctrl; a.rho_hist = hist;
    a.B = B; a.D = D; a.T = T; a.L = l.L;
    a.tiles_per_row = l.tiles_per_row; a.n_tiles = l.n_tiles;
    a.max_iters = max_iters; a.jac_every = cell->jac_every; a.jac_mode = jac_mode; a.tol = tol;
    PNR_HIP(launch_dense_newton_f64(a, l.dense_full, num_cu, st));
  }
  mark_end(m_newton, st);

  // ---- returned iterate -> caller layout ----
  Mark m_out = mark_begin(st);
  if (is_diag_cell(kind)) {
    const float* bufs[3] = {static_cast<const float*>(H[0]), static_cast<const float*>(H[1]),
                            static_cast<const float*>(H[2])};
    PNR_HIP(launch_diag_output(bufs, ctrl, static_cast<float*>(h_out), B, S, T, st));
  } else if (out_written) {
    // nothing to do
  } else if (cell->state_dtype == PNR_F32) {
    const float* bufs[4] = {static_cast<const float*>(H[0]), static_cast<const float*>(H[1]),
                            static_cast<const float*>(H[2]), static_cast<const float*>(H[3])};
    PNR_HIP(launch_dense_output<float>(bufs, ctrl, static_cast<float*>(h_out), (size_t)B * T * S, st));
  } else {
    const double* bufs[4] = {static_cast<const double*>(H[0]), static_cast<const double*>(H[1]),
                             static_cast<const double*>(H[2]), static_cast<const double*>(H[3])};
    PNR_HIP(launch_dense_output<double>(bufs, ctrl, static_cast<double*>(h_out), (size_t)B * T * S, st));
  }

  mark_end(m_out, st);
  mark_end(m_first, st);

  return finish_call(l.ctrl, l.hist, ws, max_iters, st, m_first, m_proj, m_newton, m_out);
}
}  // namespace

namespace {
// pnr_eval / pnr_eval_adaptive on the caller's workspace.
int eval_workspace(const pnr_cell* cell, const pnr_params* params, const void* x, const void* h0, void* h_out,
                   int max_iters, double tol, int jac_mode, double refresh_ratio, int bounded) {
  int rc = check_eval_args(cell, params, x, h_out, max_iters, tol, jac_mode);
  if (rc) return rc;
  const size_t need = make_layout(cell, jac_mode).total;
  if (!cell->workspace) return fail(PNR_E_WORKSPACE, "workspace is NULL (%zu bytes required)", need);
  if ((uintptr_t)cell->workspace % 256) return fail(PNR_E_WORKSPACE, "workspace must be 256-byte aligned");
  if (cell->workspace_bytes < need)
    return fail(PNR_E_WORKSPACE, "workspace has %zu bytes, %zu required", cell->workspace_bytes, need);
  return eval_impl(cell, params, x, h0, h_out, max_iters, tol, jac_mode, refresh_ratio, bounded, -1,
                   static_cast<char*>(cell->workspace));
}
}  // namespace

int pnr_eval(const pnr_cell* cell, const pnr_params* params, const void* x, const void* h0, void* h_out,
             int max_iters, double tol, int jac_mode) {
  g_last.reset();
  g_prof.valid = false;
  g_prof.used = 0;
  return eval_workspace(cell, params, x, h0, h_out, max_iters, tol, jac_mode, -1.0, 0);
}

namespace {
int validate_lowrank(const pnr_cell* c, int rank) {
  int rc = validate(c, PNR_JAC_FULL);
  if (rc) return rc;
  if (c->kind != PNR_CELL_GRU)
    return fail(PNR_E_UNSUPPORTED, "the low-rank Jacobian is defined for the GRU with a dense recurrent matrix");
  if (rank < 0 || rank > c->D) return fail(PNR_E_INVALID, "rank must be in [0, D] (got %d, D = %d)", rank, c->D);
  return 0;
}
size_t lowrank_total(const pnr_cell* c) {
  return make_layout(c, PNR_JAC_FULL).total + align_up((size_t)3 * c->D * c->D * dsize(c->state_dtype));
}
}  // namespace

size_t pnr_workspace_bytes_lowrank(const pnr_cell* cell, int rank) {
  if (validate_lowrank(cell, rank) != 0) return 0;
  return lowrank_total(cell);
}

int pnr_eval_lowrank(const pnr_cell* cell, const pnr_params* params, const void* x, const void* h0, void* h_out,
                     int max_iters, double tol, int rank) {
  g_last.reset();
  g_prof.valid = false;
  g_prof.used = 0;
  int rc = validate_lowrank(cell, rank);
  if (rc) return rc;
  if ((rc = check_eval_args(cell, params, x, h_out, max_iters, tol, PNR_JAC_FULL))) return rc;
  const size_t need = lowrank_total(cell);
  if (!cell->workspace) return fail(PNR_E_WORKSPACE, "workspace is NULL (%zu bytes required)", need);
  if ((uintptr_t)cell->workspace % 256) return fail(PNR_E_WORKSPACE, "workspace must be 256-byte aligned");
  if (cell->workspace_bytes < need)
    return fail(PNR_E_WORKSPACE, "workspace has %zu bytes, %zu required", cell->workspace_bytes, need);
  return eval_impl(cell, params, x, h0, h_out, max_iters, tol, PNR_JAC_FULL, -1.0, 0, rank,
                   static_cast<char*>(cell->workspace));
}

int pnr_eval_bounded(const pnr_cell* cell, const pnr_params* params, const void* x, const void* h0, void* h_out,
                     int max_iters, double tol, int jac_mode) {
  g_last.reset();
  g_prof.valid = false;
  g_prof.used = 0;
  if (cell && cell->kind == PNR_CELL_GRU)
    return fail(PNR_E_UNSUPPORTED, "the bounded iteration is implemented for the diagonal-recurrence cells");
  return eval_workspace(cell, params, x, h0, h_out, max_iters, tol, jac_mode, -1.0, 1);
}

int pnr_eval_adaptive(const pnr_cell* cell, const pnr_params* params, const void* x, const void* h0, void* h_out,
                      int max_iters, double tol, int jac_mode, double refresh_ratio) {
  g_last.reset();
  g_prof.valid = false;
  g_prof.used = 0;
  if (!(refresh_ratio >= 0.0)) return fail(PNR_E_INVALID, "refresh_ratio must be >= 0 (got %g)", refresh_ratio);
  if (cell && cell->kind == PNR_CELL_GRU)
    return fail(PNR_E_UNSUPPORTED, "the adaptive Jacobian refresh is implemented for the diagonal-recurrence cells");
  return eval_workspace(cell, params, x, h0, h_out, max_iters, tol, jac_mode, refresh_ratio, 0);
}

// ---- evaluation without allocation: pnr_eval on a static device scratch ----
// Callers that cannot allocate (code under graph capture, tight serving loops) use this
// array instead of a workspace.  Each device the library runs on holds its own copy for
// the life of the process.  Host code never passes the array's name to a kernel: its
// device address is looked up once per device with hipGetSymbolAddress and kept below.
static __device__ __align__(256) unsigned char scratch[PNR_STATIC_SCRATCH_BYTES];

namespace {
constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mu;
char* g_scratch_ptr[kMaxScratchDevices];   // per device; guarded by g_scratch_mu

// Device address of `scratch` on the current device (looked up on the first call there).
int static_scratch(char** out) {
  int dev = 0;
  PNR_HIP(hipGetDevice(&dev));
  if (dev < 0 || dev >= kMaxScratchDevices)
    return fail(PNR_E_UNSUPPORTED, "device %d is beyond the %d devices pnr_eval_static tracks", dev,
                kMaxScratchDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    PNR_HIP(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)));
    if (!p || (uintptr_t)p % 256) return fail(PNR_E_HIP, "hipGetSymbolAddress gave an unusable scratch address");
    g_scratch_ptr[dev] = static_cast<char*>(p);
  }
  *out = g_scratch_ptr[dev];
  return 0;
}
}  // namespace

int pnr_eval_static(const pnr_cell* cell, const pnr_params* params, const void* x, const void* h0, void* h_out,
                    int max_iters, double tol, int jac_mode) {
  g_last.reset();
  g_prof.valid = false;
  g_prof.used = 0;
  int rc = check_eval_args(cell, params, x, h_out, max_iters, tol, jac_mode);
  if (rc) return rc;
  const size_t need = make_layout(cell, jac_mode).total;
  if (need > PNR_STATIC_SCRATCH_BYTES)
    return fail(PNR_E_WORKSPACE,
                "this problem needs %zu bytes of scratch; pnr_eval_static's static scratch holds %zu "
                "(use pnr_eval with a workspace)",
                need, (size_t)PNR_STATIC_SCRATCH_BYTES);
  char* ws = nullptr;
  if (cell->T > 0 && (rc = static_scratch(&ws))) return rc;
  // measurement mode would create HIP events: it does not apply to this entry point
  const bool prof = g_prof.on;
  g_prof.on = false;
  rc = eval_impl(cell, params, x, h0, h_out, max_iters, tol, jac_mode, -1.0, 0, -1, ws);
  g_prof.on = prof;
  return rc;
}

// ---- damped (quasi-ELK) evaluation ----
namespace {
int validate_damped(const pnr_cell* c, int jac_mode) {
  int rc = validate(c, jac_mode);
  if (rc) return rc;
  if (!(c->kind == PNR_CELL_GRU_DIAG && (jac_mode == PNR_JAC_FULL || jac_mode == PNR_JAC_DIAG)) &&
      !(c->kind == PNR_CELL_LSTM_DIAG && (jac_mode == PNR_JAC_FULL || jac_mode == PNR_JAC_DIAG)) &&
      !(c->kind == PNR_CELL_GRU && jac_mode == PNR_JAC_DIAG && c->state_dtype == PNR_F32))
    return fail(PNR_E_UNSUPPORTED,
                "the damped step is implemented for GRU_DIAG and LSTM_DIAG (full or diagonal Jacobian) and the fp32 "
                "GRU (diagonal Jacobian)");
  if (c->jac_every != 1) return fail(PNR_E_UNSUPPORTED, "the damped step needs jac_every = 1");
  return 0;
}
// The dense GRU's damped loop (host-driven, [B][T][D] / [B][T][3D] fp32 arrays).
struct DenseElkLayout {
  size_t gx = 0, h[2] = {0, 0}, R = 0, J = 0, G = 0, E = 0, agg = 0, carry = 0, agg2 = 0, carry2 = 0, head = 0,
         tailge = 0, hb = 0, rmax = 0, ctrl = 0, hist = 0, total = 0;
};
DenseElkLayout make_dense_elk_layout(const pnr_cell* c) {
  DenseElkLayout l;
  const size_t BT = (size_t)c->B * c->T, D = c->D, f = sizeof(float);
  const size_t ch = (size_t)c->B * elk_dense_chunks(c->T) * D;
  size_t off = 0;
  l.gx = off; off = align_up(off + f * BT * 3 * D);
  for (int i = 0; i < 2; ++i) { l.h[i] = off; off = align_up(off + f * BT * D); }
  l.R = off; off = align_up(off + f * BT * D);
  l.J = off; off = align_up(off + f * BT * D);
  l.G = off; off = align_up(off + f * BT * D);
  l.E = off; off = align_up(off + f * BT * D);
  l.agg = off; off = align_up(off + f * 8 * ch);
  l.carry = off; off = align_up(off + f * 2 * ch);
  l.agg2 = off; off = align_up(off + f * 2 * ch);
  l.carry2 = off; off = align_up(off + f * ch);
  l.head = off; off = align_up(off + f * 3 * ch);
  l.tailge = off; off = align_up(off + f * 2 * ch);
  l.hb = off; off = align_up(off + f * ch);
  l.rmax = off; off = align_up(off + sizeof(uint32_t) * (PNR_MAX_ITERS + 1));
  // the control block and the residual history, adjacent: one read-back
  l.ctrl = off; off = align_up(off + sizeof(Ctrl));
  l.hist = off; off = align_up(off + sizeof(double) * (PNR_MAX_ITERS + 1));
  l.total = off;
  return l;
}
// pnr_eval's layout, plus two per-step planes of the smoother (gain, offset) per state component
size_t damped_planes_offset(const Layout& l) { return l.total; }
// the smoother's per-step gain and offset: one plane each per state component, or for the
// LSTM's full 2x2 block (ELK proper) four gain planes and two offset planes per channel
size_t damped_total(const pnr_cell* c, const Layout& l, int jac_mode) {
  const size_t per = c->kind == PNR_CELL_LSTM_DIAG && jac_mode == PNR_JAC_FULL ? 3 : 2;
  return align_up(l.total + per * sizeof(float) * (size_t)c->B * c->T * states(c->kind, c->D));
}
}  // namespace

size_t pnr_workspace_bytes_damped(const pnr_cell* cell, int jac_mode) {
  if (validate_damped(cell, jac_mode) != 0) return 0;
  if (cell->kind == PNR_CELL_GRU) return make_dense_elk_layout(cell).total;
  return damped_total(cell, make_layout(cell, jac_mode), jac_mode);
}

namespace {
// quasi-ELK for the dense GRU: the input projection, then the whole loop in one persistent
// launch (the returned iterate is the one whose residual was checked), the returned
// iterate copied out on the device, and one read-back of the decision and the history.
int eval_damped_dense(const pnr_cell* cell, const pnr_params* params, const void* x, const void* h0, void* h_out,
                      int max_iters, double tol, float lam) {
  const DenseElkLayout l = make_dense_elk_layout(cell);
  const int D = cell->D, T = cell->T, B = cell->B, Din = cell->D_in, GD = 3 * D;
  const size_t BT = (size_t)B * T, n = BT * D;
  const int nch = elk_dense_chunks(T);
  int num_cu = 0, rc = 0;
  if ((rc = device_info(&num_cu))) return rc;
  hipStream_t st = reinterpret_cast<hipStream_t>(cell->stream);
  char* ws = static_cast<char*>(cell->workspace);
  auto fp = [&](size_t off) { return reinterpret_cast<float*>(ws + off); };
  Mark m_first = mark_begin(st);
  Mark m_proj = mark_begin(st);
  GemmArgs gp{x, params->W, params->b_x, fp(l.gx), (int)BT, GD, Din, 0, 0, 0, Din, Din, GD, 1, 0};
  PNR_HIP(launch_gemm(cell->x_dtype, PNR_F32, gp, st));
  mark_end(m_proj, st);
  Mark m_loop = mark_begin(st);
  PNR_HIP(launch_fill_zero(fp(l.h[0]), n, st));                     // the zero guess, stored
  PNR_HIP(launch_fill_zero(fp(l.hb), (size_t)B * nch * D, st));     // ... and its chunk halos
  PNR_HIP(launch_fill_zero(fp(l.rmax), (size_t)max_iters + 1, st));
  Ctrl* ctrl = reinterpret_cast<Ctrl*>(ws + l.ctrl);
  PNR_HIP(launch_init(ctrl, nullptr, 0, nullptr, 0, st));
  ElkLoopArgs a{};
  a.gx = fp(l.gx);
  a.U = static_cast<const float*>(params->U);
  a.bh = static_cast<const float*>(params->b_h);
  a.h0 = static_cast<const float*>(h0);
  a.H[0] = fp(l.h[0]);
  a.H[1] = fp(l.h[1]);
  a.R = fp(l.R); a.J = fp(l.J); a.G = fp(l.G); a.E = fp(l.E);
  a.agg = fp(l.agg); a.carry = fp(l.carry); a.agg2 = fp(l.agg2); a.carry2 = fp(l.carry2);
  a.head = fp(l.head); a.tailge = fp(l.tailge); a.hb = fp(l.hb);
  a.rmax = reinterpret_cast<uint32_t*>(ws + l.rmax);
  a.ctrl = ctrl;
  a.hist = reinterpret_cast<double*>(ws + l.hist);
  a.B = B; a.T = T; a.D = D; a.nch = nch; a.max_iters = max_iters;
  a.lam = lam;
  a.tol = tol;
  PNR_HIP(launch_gru_elk_loop(a, num_cu, st));
  mark_end(m_loop, st);
  Mark m_out = mark_begin(st);
  PNR_HIP(launch_elk_dense_output(a.H[0], a.H[1], ctrl, static_cast<float*>(h_out), n, st));
  mark_end(m_out, st);
  mark_end(m_first, st);
  return finish_call(l.ctrl, l.hist, ws, max_iters, st, m_first, m_proj, m_loop, m_out);
}
}  // namespace

int pnr_eval_damped(const pnr_cell* cell, const pnr_params* params, const void* x, const void* h0, void* h_out,
                    int max_iters, double tol, int jac_mode, double damping) {
  g_last.reset();
  g_prof.valid = false;
  g_prof.used = 0;
  int rc = validate_damped(cell, jac_mode);
  if (rc) return rc;
  if (!params) return fail(PNR_E_INVALID, "params is NULL");
  if (!params->W || !params->U || (cell->T > 0 && (!x || !h_out)))
    return fail(PNR_E_INVALID, "W, U and (for T > 0) x and h_out must be non-NULL");
  if (max_iters < 0 || max_iters >= PNR_MAX_ITERS)
    return fail(PNR_E_INVALID, "max_iters must be in [0, %d)", PNR_MAX_ITERS);
  if (isnan(tol)) return fail(PNR_E_INVALID, "tol is NaN");
  if (!(damping > 0.0) || !(damping < 1e30)) return fail(PNR_E_INVALID, "damping must be finite and > 0");
  const Layout l = make_layout(cell, jac_mode);
  const size_t need = cell->kind == PNR_CELL_GRU ? make_dense_elk_layout(cell).total : damped_total(cell, l, jac_mode);
  if (!cell->workspace) return fail(PNR_E_WORKSPACE, "workspace is NULL (%zu bytes required)", need);
  if ((uintptr_t)cell->workspace % 256) return fail(PNR_E_WORKSPACE, "workspace must be 256-byte aligned");
  if (cell->workspace_bytes < need)
    return fail(PNR_E_WORKSPACE, "workspace has %zu bytes, %zu required", cell->workspace_bytes, need);
  if (cell->T == 0) {
    g_last.iters = 0;
    g_last.residual = 0.0;
    g_last.hist.assign(1, 0.0);
    return PNR_OK;
  }
  if (cell->kind == PNR_CELL_GRU) return eval_damped_dense(cell, params, x, h0, h_out, max_iters, tol, (float)damping);
  int num_cu = 0;
  if ((rc = device_info(&num_cu))) return rc;
  hipStream_t st = reinterpret_cast<hipStream_t>(cell->stream);
  char* ws = static_cast<char*>(cell->workspace);
  Ctrl* ctrl = reinterpret_cast<Ctrl*>(ws + l.ctrl);
  double* hist = reinterpret_cast<double*>(ws + l.hist);
  const int D = cell->D, T = cell->T, B = cell->B, Din = cell->D_in;
  const int G = gates(cell->kind), S = states(cell->kind, D);
  const size_t plane = (size_t)B * T * S;
  float* planes = reinterpret_cast<float*>(ws + damped_planes_offset(l));

  Mark m_first = mark_begin(st);
  PNR_HIP(launch_init(ctrl, reinterpret_cast<uint64_t*>(ws + l.slots), l.slot_words,
                      reinterpret_cast<uint64_t*>(ws + l.partials), kPartialWords, st));
  // gx[b][m][t] = sum_k W[m][k] x[b][t][k] + b_x[m]
  GemmArgs g{params->W, x, params->b_x, ws + l.gx, G * D, T, Din, 0, (long long)T * Din, (long long)G * D * T,
             Din, Din, T, B, 1};
  Mark m_proj = mark_begin(st);
  PNR_HIP(launch_gemm(cell->x_dtype, cell->state_dtype, g, st));
  mark_end(m_proj, st);

  ElkArgs a{};
  a.gx = reinterpret_cast<const float*>(ws + l.gx);
  a.u = static_cast<const float*>(params->U);
  a.bh = static_cast<const float*>(params->b_h);
  a.h0 = static_cast<const float*>(h0);
  a.H[0] = reinterpret_cast<float*>(ws + l.h[0]);
  a.H[1] = reinterpret_cast<float*>(ws + l.h[1]);
  const bool elk2 = cell->kind == PNR_CELL_LSTM_DIAG && jac_mode == PNR_JAC_FULL;
  a.Gs = planes;
  a.Es = planes + (elk2 ? 2 : 1) * plane;
  a.partials = reinterpret_cast<uint32_t*>(ws + l.partials);
  a.ctrl = ctrl;
  a.rho_hist = hist;
  a.B = B; a.D = D; a.T = T;
  a.tiles_per_row = (T + PNR_BLOCK * elk_items_per_thread() - 1) / (PNR_BLOCK * elk_items_per_thread());
  a.n_rows = B * D;
  a.max_iters = max_iters; a.jac_mode = jac_mode; a.tol = tol;
  a.lam = (float)damping;
  Mark m_newton = mark_begin(st);
  if (elk2)
    PNR_HIP(launch_elk2_lstm(a, num_cu, st));
  else
    PNR_HIP(launch_elk_diag(cell->kind, a, num_cu, st));
  mark_end(m_newton, st);

  Mark m_out = mark_begin(st);
  const float* bufs[3] = {a.H[0], a.H[1], nullptr};
  PNR_HIP(launch_diag_output(bufs, ctrl, static_cast<float*>(h_out), B, S, T, st));
  mark_end(m_out, st);
  mark_end(m_first, st);
  return finish_call(l.ctrl, l.hist, ws, max_iters, st, m_first, m_proj, m_newton, m_out);
}

// ---- chunked evaluation ----
namespace {
// The per-chunk problem, its workspace, and (for B > 1 with several chunks) contiguous
// staging for the chunk's inputs, boundary state and output behind it.
struct ChunkPlan {
  int L = 0;              // chunk length (steps)
  bool staged = false;
  pnr_cell sub{};         // the problem of one chunk (T = L)
  size_t sub_bytes = 0, x_off = 0, h0_off = 0, out_off = 0, total = 0;
};
int plan_chunks(const pnr_cell* c, int jac_mode, double damping, int chunk_len, ChunkPlan& p) {
  if (!c) return fail(PNR_E_INVALID, "cell descriptor is NULL");
  if (chunk_len < 1) return fail(PNR_E_INVALID, "chunk_len must be >= 1 (got %d)", chunk_len);
  if (!(damping >= 0.0) || !(damping < 1e30)) return fail(PNR_E_INVALID, "damping must be finite and >= 0");
  if (c->T < 0) return fail(PNR_E_INVALID, "T must be >= 0 (got %d)", c->T);
  p.L = c->T < chunk_len ? c->T : chunk_len;
  p.sub = *c;
  p.sub.T = p.L;
  const int rc = damping > 0 ? validate_damped(&p.sub, jac_mode) : validate(&p.sub, jac_mode);
  if (rc) return rc;
  const Layout l = make_layout(&p.sub, jac_mode);
  p.sub_bytes = damping <= 0 ? l.total
                : (p.sub.kind == PNR_CELL_GRU ? make_dense_elk_layout(&p.sub).total
                                                : damped_total(&p.sub, l, jac_mode));
  p.staged = c->B > 1 && c->T > p.L;
  size_t off = align_up(p.sub_bytes);
  if (p.staged) {
    const size_t B = c->B, L = p.L, S = states(c->kind, c->D);
    p.x_off = off; off = align_up(off + B * L * c->D_in * dsize(c->x_dtype));
    p.h0_off = off; off = align_up(off + B * S * dsize(c->state_dtype));
    p.out_off = off; off = align_up(off + B * L * S * dsize(c->state_dtype));
  }
  p.total = off;
  return 0;
}
int status_rank(int s) { return s == PNR_NONFINITE ? 2 : (s == PNR_NOT_CONVERGED ? 1 : 0); }
}  // namespace

size_t pnr_workspace_bytes_chunked(const pnr_cell* cell, int jac_mode, double damping, int chunk_len) {
  ChunkPlan p;
  if (plan_chunks(cell, jac_mode, damping, chunk_len, p) != 0) return 0;
  return p.total;
}

int pnr_eval_chunked(const pnr_cell* cell, const pnr_params* params, const void* x, const void* h0, void* h_out,
                     int max_iters, double tol, int jac_mode, double damping, int chunk_len) {
  g_last.reset();
  g_prof.valid = false;
  ChunkPlan p;
  int rc = plan_chunks(cell, jac_mode, damping, chunk_len, p);
  if (rc) return rc;
  if (!params) return fail(PNR_E_INVALID, "params is NULL");
  if (!params->W || !params->U || (cell->T > 0 && (!x || !h_out)))
    return fail(PNR_E_INVALID, "W, U and (for T > 0) x and h_out must be non-NULL");
  if (!cell->workspace) return fail(PNR_E_WORKSPACE, "workspace is NULL (%zu bytes required)", p.total);
  if ((uintptr_t)cell->workspace % 256) return fail(PNR_E_WORKSPACE, "workspace must be 256-byte aligned");
  if (cell->workspace_bytes < p.total)
    return fail(PNR_E_WORKSPACE, "workspace has %zu bytes, %zu required", cell->workspace_bytes, p.total);
  if (cell->T == 0) {
    g_last.iters = 0;
    g_last.residual = 0.0;
    g_last.hist.assign(1, 0.0);
    return PNR_OK;
  }
  hipStream_t st = reinterpret_cast<hipStream_t>(cell->stream);
  char* ws = static_cast<char*>(cell->workspace);
  const size_t B = cell->B, T = cell->T, Din = cell->D_in, S = states(cell->kind, cell->D);
  const size_t xes = dsize(cell->x_dtype), ses = dsize(cell->state_dtype);
  const char* xb = static_cast<const char*>(x);
  char* ob = static_cast<char*>(h_out);
  int iters = 0, status = PNR_OK;
  double residual = 0.0;
  std::vector<double> hist;
  pnr_profile acc{};
  bool prof_ok = g_prof.on;
  for (size_t t0 = 0; t0 < T; t0 += p.L) {
    const size_t Lc = T - t0 < (size_t)p.L ? T - t0 : (size_t)p.L;
    pnr_cell sub = p.sub;
    sub.T = (int)Lc;
    sub.workspace = ws;
    sub.workspace_bytes = p.sub_bytes;
    const void* xc = xb + t0 * Din * xes;
    const void* h0c = t0 == 0 ? h0 : static_cast<const void*>(ob + (t0 - 1) * S * ses);   // the carried-in state
    void* oc = ob + t0 * S * ses;
    if (p.staged) {
      PNR_HIP(hipMemcpy2DAsync(ws + p.x_off, Lc * Din * xes, xc, T * Din * xes, Lc * Din * xes, B,
                               hipMemcpyDeviceToDevice, st));
      if (t0 > 0) {
        PNR_HIP(hipMemcpy2DAsync(ws + p.h0_off, S * ses, h0c, T * S * ses, S * ses, B, hipMemcpyDeviceToDevice, st));
        h0c = ws + p.h0_off;
      }
      xc = ws + p.x_off;
      oc = ws + p.out_off;
    }
    rc = damping > 0 ? pnr_eval_damped(&sub, params, xc, h0c, oc, max_iters, tol, jac_mode, damping)
                     : pnr_eval(&sub, params, xc, h0c, oc, max_iters, tol, jac_mode);
    if (rc < 0) return rc;   // g_last.err holds the chunk's error
    if (p.staged)
      PNR_HIP(hipMemcpy2DAsync(ob + t0 * S * ses, T * S * ses, oc, Lc * S * ses, Lc * S * ses, B,
                               hipMemcpyDeviceToDevice, st));
    if (prof_ok && g_prof.valid) {
      const pnr_profile& c = g_prof.last;
      acc.total_ms += c.total_ms; acc.proj_ms += c.proj_ms; acc.newton_ms += c.newton_ms; acc.out_ms += c.out_ms;
      acc.passes += c.passes; acc.resid_only += c.resid_only;
    } else {
      prof_ok = false;
    }
    iters += g_last.iters;
    if (!(g_last.residual <= residual)) residual = g_last.residual;   // max, NaN wins
    for (size_t i = 0; i < g_last.hist.size(); ++i) hist.push_back(g_last.hist[i]);
    if (status_rank(rc) > status_rank(status)) status = rc;
    if (rc == PNR_NONFINITE) break;   // later chunks would start from a non-finite state
  }
  PNR_HIP(hipStreamSynchronize(st));
  g_last.iters = iters;
  g_last.residual = residual;
  g_last.hist.assign(hist.data(), hist.data() + hist.size());
  g_prof.valid = prof_ok;
  if (prof_ok) g_prof.last = acc;
  return status;
}

// ---- backward pass (diagonal-recurrence cells) ----
namespace {
struct BwdLayout {
  size_t gx = 0, states = 0, dgx = 0, wt = 0, part = 0, total = 0;
};
int validate_backward(const pnr_cell* c) {
  if (!c) return fail(PNR_E_INVALID, "cell descriptor is NULL");
  pnr_cell v = *c;
  v.jac_every = 1;
  // the dense GRU's limits are those of its diagonal-Jacobian forward kernels
  int rc = validate(&v, c->kind == PNR_CELL_GRU ? PNR_JAC_DIAG : PNR_JAC_FULL);
  if (rc) return rc;
  if (c->state_dtype != PNR_F32)
    return fail(PNR_E_UNSUPPORTED, "the backward pass is implemented for fp32 state");
  if ((double)c->B * c->T > 2.0e9 || (double)gates(c->kind) * c->D * c->D_in > 2.0e9)
    return fail(PNR_E_INVALID, "problem too large for this library's index range");
  return 0;
}
constexpr int kBwdMaxIters = 256;      // refinement iterations of the dense adjoint
constexpr double kBwdTolRel = 2e-5;    // stop when max |R| <= kBwdTolRel * max |g|

// Dense GRU: every array [B*T][.] row-major, fp32.
struct DenseBwdLayout {
  size_t gx = 0, gh = 0, hprev = 0, F = 0, lam = 0, dgh = 0, v = 0, scan3 = 0, ut = 0, xt = 0, wt = 0, rmax = 0,
         part = 0, v2 = 0, bnd = 0, ctrl = 0, hist = 0, partials = 0, total = 0;
};
DenseBwdLayout make_dense_bwd_layout(const pnr_cell* c) {
  DenseBwdLayout l;
  const size_t BT = (size_t)c->B * c->T, D = c->D, GD = 3 * D, Din = c->D_in, f = sizeof(float);
  size_t off = 0;
  l.gx = off; off = align_up(off + f * BT * GD);       // gx, then dL/dgx
  l.gh = off; off = align_up(off + f * BT * GD);       // U h + b_h, then dL/dgh transposed
  l.hprev = off; off = align_up(off + f * BT * D);
  l.F = off; off = align_up(off + f * 6 * BT * D);
  l.lam = off; off = align_up(off + f * BT * D);
  l.dgh = off; off = align_up(off + f * BT * GD);
  l.v = off; off = align_up(off + f * BT * D);         // U^T dgh, then h_prev transposed
  // the second adjoint buffer and the chunk scan's aggregates and carries; afterwards
  // dL/dgx transposed (3 B*T*D floats)
  const size_t chunks = (size_t)c->B * gru_bwd_chunks(c->T) * D;
  l.scan3 = off; off = align_up(off + f * std::max(3 * BT * D, BT * D + 3 * chunks + 1));
  l.ut = off; off = align_up(off + f * D * GD);
  l.xt = off; off = align_up(off + f * BT * Din);
  l.wt = off; off = align_up(off + f * Din * GD);
  l.rmax = off; off = align_up(off + sizeof(uint32_t) * (kBwdMaxIters + 1));
  l.part = off; off = align_up(off + f * kSplitKSlices * GD * (D > Din ? D : Din));   // split-K partials
  // the on-device refinement loop: the second v buffer, each chunk's boundary lam, the
  // control block with the residual history right after it (one read-back), and the
  // per-iteration residual maxima
  l.v2 = off; off = align_up(off + f * BT * D);
  l.bnd = off; off = align_up(off + f * chunks);
  l.ctrl = off; off = align_up(off + sizeof(Ctrl));
  l.hist = off; off = align_up(off + sizeof(double) * (kBwdMaxIters + 1));
  l.partials = off; off = align_up(off + sizeof(uint32_t) * (kBwdMaxIters + 1));
  l.total = off;
  return l;
}

BwdLayout make_bwd_layout(const pnr_cell* c) {
  BwdLayout l;
  if (c->kind == PNR_CELL_GRU) {
    l.total = make_dense_bwd_layout(c).total;
    return l;
  }
  const size_t B = c->B, T = c->T, D = c->D, Din = c->D_in, G = gates(c->kind), S = states(c->kind, c->D);
  const size_t ge = dsize(c->x_dtype);   // the gradient GEMMs' operand type: that of x
  size_t off = 0;
  l.gx = off; off = align_up(off + B * T * G * D * sizeof(float));   // gx, then dL/dgx transposed
  const size_t st = 2 * B * T * S * sizeof(float), xt = B * T * Din * ge;
  l.states = off; off = align_up(off + (st > xt ? st : xt));          // h, dL/dh; then x transposed
  l.dgx = off; off = align_up(off + B * T * G * D * ge);
  l.wt = off; off = align_up(off + ge * G * D * Din);
  l.part = off; off = align_up(off + sizeof(float) * B * 3 * G * D);
  l.total = off;
  return l;
}
}  // namespace

namespace {
int backward_dense(const pnr_cell* cell, const pnr_params* params, const void* x, const void* h0, const void* h,
                   const void* grad_h, void* grad_x, void* grad_W, void* grad_U, void* grad_b_x, void* grad_b_h,
                   void* grad_h0, bool jdiag) {
  const DenseBwdLayout l = make_dense_bwd_layout(cell);
  const int D = cell->D, T = cell->T, B = cell->B, Din = cell->D_in, GD = 3 * D;
  const size_t BT = (size_t)B * T, n = BT * D;
  hipStream_t st = reinterpret_cast<hipStream_t>(cell->stream);
  int num_cu = 0, rc;
  if ((rc = device_info(&num_cu))) return rc;
  char* ws = static_cast<char*>(cell->workspace);
  auto fp = [&](size_t off) { return reinterpret_cast<float*>(ws + off); };
  float *gx = fp(l.gx), *gh = fp(l.gh), *hprev = fp(l.hprev), *F = fp(l.F), *lam = fp(l.lam), *dgh = fp(l.dgh),
        *v = fp(l.v), *UT = fp(l.ut);
  float* lam2 = fp(l.scan3);   // the other adjoint buffer
  const size_t chunks = (size_t)B * gru_bwd_chunks(T) * D;
  float2* agg = reinterpret_cast<float2*>(lam2 + ((n + 1) & ~(size_t)1));
  float* carry = reinterpret_cast<float*>(agg + chunks);
  uint32_t* rmax = reinterpret_cast<uint32_t*>(ws + l.rmax);
  const float* U = static_cast<const float*>(params->U);

  Mark m_first = mark_begin(st);
  Mark m_proj = mark_begin(st);
  // the forward's gate pre-activations: gx = x W^T + b_x, gh = h_{t-1} U^T + b_h
  GemmArgs gp{x, params->W, params->b_x, gx, (int)BT, GD, Din, 0, 0, 0, Din, Din, GD, 1, 0};
  PNR_HIP(launch_gemm(cell->x_dtype, PNR_F32, gp, st));
  PNR_HIP(launch_gru_shift_states(static_cast<const float*>(h), static_cast<const float*>(h0), hprev, B, T, D, st));
  GemmArgs gq{hprev, U, params->b_h, gh, (int)BT, GD, D, 0, 0, 0, D, D, GD, 1, 0};
  PNR_HIP(launch_gemm(PNR_F32, PNR_F32, gq, st));
  PNR_HIP(launch_gru_bwd_factors(gx, gh, hprev, U, F, n, D, st));
  PNR_HIP(launch_transpose(U, PNR_F32, UT, PNR_F32, 1, GD, D, st));
  mark_end(m_proj, st);

  // ---- adjoint: quasi-Newton refinement from lam = 0 ----
  Mark m_adj = mark_begin(st);
  PNR_HIP(launch_fill_zero(lam, n, st));
  int status = PNR_NOT_CONVERGED, updates = 0;
  double rho = 0.0;
  std::vector<double> hist;
  const GemmArgs gv{dgh, UT, nullptr, v, (int)BT, D, GD, 0, 0, 0, GD, GD, D, 1, 0};
  if (jdiag) {
    // the diagonal approximation: the first update from lam = 0 is the diagonal system's
    // exact solution (R(0) = g, one diagonal scan); nothing to refine or read back
    PNR_HIP(launch_fill_zero(reinterpret_cast<float*>(rmax), 1, st));
    PNR_HIP(launch_fill_zero(dgh, BT * GD, st));   // dgh(0): v = U^T dgh = 0
    PNR_HIP(launch_gemm(PNR_F32, PNR_F32, gv, st));
    PNR_HIP(launch_gru_bwd_refine(F, lam, v, static_cast<const float*>(grad_h), lam2, dgh, agg, carry, rmax, B, T, D,
                                  st));
    std::swap(lam, lam2);
    updates = 1;
    status = PNR_OK;
    hist.push_back(0.0);
  } else {
    // the whole refinement on the device: one persistent loop decides when to stop (the
    // adjoint returned is the one whose residual passed) and is read back once
    PNR_HIP(launch_fill_zero(v, n, st));   // v_0 = U^T dgh(0) = 0
    PNR_HIP(launch_fill_zero(fp(l.bnd), chunks, st));
    PNR_HIP(launch_fill_zero(fp(l.partials), kBwdMaxIters + 1, st));
    Ctrl* ctrl = reinterpret_cast<Ctrl*>(ws + l.ctrl);
    PNR_HIP(launch_init(ctrl, nullptr, 0, nullptr, 0, st));
    BwdLoopArgs la{};
    la.F = F;
    la.g = static_cast<const float*>(grad_h);
    la.U = U;
    la.lam[0] = lam; la.lam[1] = lam2;
    la.v[0] = v; la.v[1] = fp(l.v2);
    la.agg = reinterpret_cast<float*>(agg);   // the same chunks x 2 floats, in the loop's [B][D][nch] order
    la.carry = carry;
    la.bnd = fp(l.bnd);
    la.rmax = reinterpret_cast<uint32_t*>(ws + l.partials);
    la.ctrl = ctrl;
    la.hist = reinterpret_cast<double*>(ws + l.hist);
    la.B = B; la.T = T; la.D = D; la.nch = gru_bwd_chunks(T);
    la.max_iters = kBwdMaxIters;
    la.tol_rel = kBwdTolRel;
    PNR_HIP(launch_gru_bwd_loop(la, num_cu, st));
    constexpr size_t kRb = sizeof(double) * (kBwdMaxIters + 1);
    alignas(64) static thread_local char rb[sizeof(Ctrl) + 256 + kRb];
    const size_t rb_bytes = (l.hist - l.ctrl) + kRb;
    if (rb_bytes > sizeof(rb)) return fail(PNR_E_INVALID, "control read-back of %zu bytes exceeds %zu", rb_bytes,
                                           sizeof(rb));
    PNR_HIP(hipMemcpyAsync(rb, ws + l.ctrl, rb_bytes, hipMemcpyDeviceToHost, st));
    PNR_HIP(hipStreamSynchronize(st));
    Ctrl hc;
    memcpy(&hc, rb, sizeof(Ctrl));
    if (hc.fault)
      return fail(PNR_E_HIP, "device loop gave up waiting (grid barrier); results are not valid");
    if (!hc.done || hc.iters < 0) return fail(PNR_E_HIP, "device loop did not record a decision");
    const double* hh = reinterpret_cast<const double*>(rb + (l.hist - l.ctrl));
    hist.assign(hh, hh + hc.iters + 1);
    status = hc.status;
    updates = hc.iters;
    rho = hc.rho;
    if (hc.result_buf == 1) std::swap(lam, lam2);   // `lam` is the returned adjoint
  }
  mark_end(m_adj, st);

  // ---- gradients from the adjoint ----
  Mark m_grads = mark_begin(st);
  float* dgx = gx;   // gx is no longer needed
  PNR_HIP(launch_gru_bwd_gates(F, lam, dgh, dgx, n, D, st));
  if (grad_h0) {
    PNR_HIP(launch_gemm(PNR_F32, PNR_F32, gv, st));
    // exact: dh0 = J_1^T lam_1 = z lam + U^T dgh; diagonal approximation: diag(J_1) lam_1
    PNR_HIP(launch_gru_bwd_dh0(jdiag ? F + n : F, lam, jdiag ? nullptr : v, static_cast<float*>(grad_h0), B, T, D,
                               st));
  }
  float* dghT = gh;           // [3D][B*T]
  float* dgxT = fp(l.scan3);  // [3D][B*T]; the adjoint (possibly here) is not read after dh0
  if (grad_U || grad_b_h) PNR_HIP(launch_transpose(dgh, PNR_F32, dghT, PNR_F32, 1, (int)BT, GD, st));
  if (grad_W || grad_b_x) PNR_HIP(launch_transpose(dgx, PNR_F32, dgxT, PNR_F32, 1, (int)BT, GD, st));
  PNR_HIP(launch_row_sum(dghT, grad_b_h ? GD : 0, BT, static_cast<float*>(grad_b_h), fp(l.part), st));
  PNR_HIP(launch_row_sum(dgxT, grad_b_x ? GD : 0, BT, static_cast<float*>(grad_b_x), fp(l.part), st));
  if (grad_U) {
    // dU[m][j] = sum_{b,t} dgh[(b,t)][m] h_{t-1}[(b,t)][j]
    float* hprevT = v;
    PNR_HIP(launch_transpose(hprev, PNR_F32, hprevT, PNR_F32, 1, (int)BT, D, st));
    PNR_HIP(launch_gemm_split_k(dghT, (int)BT, hprevT, (int)BT, static_cast<float*>(grad_U), GD, D, (int)BT,
                                fp(l.part), kSplitKSlices, st));
  }
  if (grad_W) {
    float* xT = fp(l.xt);
    PNR_HIP(launch_transpose(x, cell->x_dtype, xT, PNR_F32, 1, (int)BT, Din, st));
    PNR_HIP(launch_gemm_split_k(dgxT, (int)BT, xT, (int)BT, static_cast<float*>(grad_W), GD, Din, (int)BT,
                                fp(l.part), kSplitKSlices, st));
  }
  if (grad_x) {
    float* WT = fp(l.wt);
    PNR_HIP(launch_transpose(params->W, cell->x_dtype, WT, PNR_F32, 1, GD, Din, st));
    GemmArgs gxg{dgx, WT, nullptr, grad_x, (int)BT, Din, GD, 0, 0, 0, GD, GD, Din, 1, 0};
    PNR_HIP(launch_gemm(PNR_F32, PNR_F32, gxg, st));
  }
  mark_end(m_grads, st);
  mark_end(m_first, st);
  g_last.iters = updates;
  g_last.residual = rho;
  g_last.hist.assign(hist.data(), hist.data() + hist.size());
  if (g_prof.on) {
    PNR_HIP(hipStreamSynchronize(st));
    pnr_profile p{};
    p.total_ms = mark_ms(m_first);
    p.proj_ms = mark_ms(m_proj);
    p.newton_ms = mark_ms(m_adj);
    p.out_ms = mark_ms(m_grads);
    p.passes = updates + 1;
    g_prof.last = p;
    g_prof.valid = true;
  }
  return status;
}
}  // namespace

size_t pnr_workspace_bytes_backward(const pnr_cell* cell) {
  if (validate_backward(cell) != 0) return 0;
  return make_bwd_layout(cell).total;
}

namespace {
int backward_impl(const pnr_cell* cell, const pnr_params* params, const void* x, const void* h0, const void* h,
                  const void* grad_h, void* grad_x, void* grad_W, void* grad_U, void* grad_b_x, void* grad_b_h,
                  void* grad_h0, bool jdiag) {
  g_last.reset();
  g_prof.valid = false;
  g_prof.used = 0;
  int rc = validate_backward(cell);
  if (rc) return rc;
  if (!params) return fail(PNR_E_INVALID, "params is NULL");
  if (!params->W || !params->U || (cell->T > 0 && (!x || !h || !grad_h)))
    return fail(PNR_E_INVALID, "W, U and (for T > 0) x, h and grad_h must be non-NULL");
  const BwdLayout l = make_bwd_layout(cell);
  if (!cell->workspace) return fail(PNR_E_WORKSPACE, "workspace is NULL (%zu bytes required)", l.total);
  if ((uintptr_t)cell->workspace % 256) return fail(PNR_E_WORKSPACE, "workspace must be 256-byte aligned");
  if (cell->workspace_bytes < l.total)
    return fail(PNR_E_WORKSPACE, "workspace has %zu bytes, %zu required", cell->workspace_bytes, l.total);
  const int kind = cell->kind, D = cell->D, T = cell->T, B = cell->B, Din = cell->D_in;
  const int G = gates(kind), S = states(kind, D);
  hipStream_t st = reinterpret_cast<hipStream_t>(cell->stream);
  if (T == 0) {   // no steps: every gradient but dL/dh0 (= 0) is an empty sum
    PNR_HIP(launch_fill_zero(static_cast<float*>(grad_W), (size_t)G * D * Din, st));
    PNR_HIP(launch_fill_zero(static_cast<float*>(grad_U), (size_t)G * D * (kind == PNR_CELL_GRU ? D : 1), st));
    PNR_HIP(launch_fill_zero(static_cast<float*>(grad_b_x), (size_t)G * D, st));
    PNR_HIP(launch_fill_zero(static_cast<float*>(grad_b_h), (size_t)G * D, st));
    PNR_HIP(launch_fill_zero(static_cast<float*>(grad_h0), (size_t)B * S, st));
    g_last.iters = 0;
    g_last.residual = 0.0;
    g_last.hist.assign(1, 0.0);
    return PNR_OK;
  }
  if (kind == PNR_CELL_GRU)
    return backward_dense(cell, params, x, h0, h, grad_h, grad_x, grad_W, grad_U, grad_b_x, grad_b_h, grad_h0, jdiag);
  int num_cu = 0;
  if ((rc = device_info(&num_cu))) return rc;
  char* ws = static_cast<char*>(cell->workspace);
  float* gx = reinterpret_cast<float*>(ws + l.gx);
  float* hT = reinterpret_cast<float*>(ws + l.states);
  float* gT = hT + (size_t)B * T * S;
  void* dgx = ws + l.dgx;
  const int ge = cell->x_dtype;   // PNR_F32 or PNR_BF16: the gradient GEMMs run in the input's type
  float* part = reinterpret_cast<float*>(ws + l.part);
  const size_t BT = (size_t)B * T;

  Mark m_first = mark_begin(st);
  // the forward's input projection, recomputed: gx[b][m][t] = sum_k W[m][k] x[b][t][k] + b_x[m]
  GemmArgs g{params->W, x, params->b_x, gx, G * D, T, Din, 0, (long long)T * Din, (long long)G * D * T,
             Din, Din, T, B, 1};
  Mark m_proj = mark_begin(st);
  PNR_HIP(launch_gemm(cell->x_dtype, PNR_F32, g, st));
  mark_end(m_proj, st);
  PNR_HIP(launch_transpose(h, PNR_F32, hT, PNR_F32, B, T, S, st));
  PNR_HIP(launch_transpose(grad_h, PNR_F32, gT, PNR_F32, B, T, S, st));

  BwdArgs a{};
  a.jdiag = jdiag ? 1 : 0;
  a.gx = gx;
  a.u = static_cast<const float*>(params->U);
  a.bh = static_cast<const float*>(params->b_h);
  a.h0 = static_cast<const float*>(h0);
  a.hT = hT;
  a.gT = gT;
  a.dgx = dgx;
  a.part = part;
  a.dh0 = static_cast<float*>(grad_h0);
  a.B = B; a.D = D; a.T = T;
  a.tiles_per_row = (T + PNR_BLOCK * adjoint_items_per_thread() - 1) / (PNR_BLOCK * adjoint_items_per_thread());
  a.n_rows = B * D;
  a.dgx_bf16 = ge == PNR_BF16;
  Mark m_adj = mark_begin(st);
  PNR_HIP(launch_adjoint_diag(kind, a, num_cu, st));
  mark_end(m_adj, st);

  Mark m_grads = mark_begin(st);
  PNR_HIP(launch_sum_over_batch(part, B, G * D, static_cast<float*>(grad_U), static_cast<float*>(grad_b_h),
                                static_cast<float*>(grad_b_x), st));
  if (grad_W) {
    // dW[m][k] = sum_{b,t} dgx[m][(b,t)] x[(b,t)][k]: x transposed to [k][(b,t)]
    void* xT = hT;   // the transposed states are no longer needed
    PNR_HIP(launch_transpose(x, cell->x_dtype, xT, ge, 1, (int)BT, Din, st));
    GemmArgs gw{dgx, xT, nullptr, grad_W, G * D, Din, (int)BT, 0, 0, 0, (int)BT, (int)BT, Din, 1, 0};
    PNR_HIP(launch_gemm(ge, PNR_F32, gw, st));
  }
  if (grad_x) {
    // dx[(b,t)][k] = sum_m dgx[m][(b,t)] W[m][k]: dgx transposed to [(b,t)][m], W to [k][m]
    void* dgxT = gx;   // gx is no longer needed
    void* WT = ws + l.wt;
    PNR_HIP(launch_transpose(dgx, ge, dgxT, ge, 1, G * D, (int)BT, st));
    PNR_HIP(launch_transpose(params->W, cell->x_dtype, WT, ge, 1, G * D, Din, st));
    GemmArgs gxg{dgxT, WT, nullptr, grad_x, (int)BT, Din, G * D, 0, 0, 0, G * D, G * D, Din, 1, 0};
    PNR_HIP(launch_gemm(ge, PNR_F32, gxg, st));
  }
  mark_end(m_grads, st);
  mark_end(m_first, st);
  g_last.iters = 0;   // the adjoint is one scan
  g_last.residual = 0.0;
  g_last.hist.assign(1, 0.0);
  if (g_prof.on) {
    PNR_HIP(hipStreamSynchronize(st));
    pnr_profile p{};
    p.total_ms = mark_ms(m_first);
    p.proj_ms = mark_ms(m_proj);
    p.newton_ms = mark_ms(m_adj);
    p.out_ms = mark_ms(m_grads);
    p.passes = 1;
    g_prof.last = p;
    g_prof.valid = true;
  }
  return PNR_OK;
}
}  // namespace

int pnr_backward(const pnr_cell* cell, const pnr_params* params, const void* x, const void* h0, const void* h,
                 const void* grad_h, void* grad_x, void* grad_W, void* grad_U, void* grad_b_x, void* grad_b_h,
                 void* grad_h0) {
  return backward_impl(cell, params, x, h0, h, grad_h, grad_x, grad_W, grad_U, grad_b_x, grad_b_h, grad_h0, false);
}

int pnr_backward_approx(const pnr_cell* cell, const pnr_params* params, const void* x, const void* h0, const void* h,
                        const void* grad_h, void* grad_x, void* grad_W, void* grad_U, void* grad_b_x, void* grad_b_h,
                        void* grad_h0, int jac_mode) {
  if (jac_mode != PNR_JAC_FULL && jac_mode != PNR_JAC_DIAG) {
    g_last.reset();
    g_prof.valid = false;
    return fail(PNR_E_INVALID, "jac_mode must be PNR_JAC_FULL (exact) or PNR_JAC_DIAG (got %d)", jac_mode);
  }
  return backward_impl(cell, params, x, h0, h, grad_h, grad_x, grad_W, grad_U, grad_b_x, grad_b_h, grad_h0,
                       jac_mode == PNR_JAC_DIAG);
}

// ---- backward pass over chunks (gradient checkpointing) ----
namespace {
__global__ void __launch_bounds__(256) axpy_kernel(float* __restrict__ y, const float* __restrict__ x, size_t n) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
    y[i] += x[i];
}
// g[b][L-1][s] += mu[b][s]: the adjoint arriving from the later chunk joins the loss
// gradient of the chunk's last step
__global__ void __launch_bounds__(256) add_last_row_kernel(float* __restrict__ g, const float* __restrict__ mu, int B,
                                                           int L, int S) {
  const int e = blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= B * S) return;
  const int b = e / S, c = e - b * S;
  g[((size_t)b * L + (L - 1)) * S + c] += mu[e];
}
hipError_t launch_axpy(float* y, const float* x, size_t n, hipStream_t st) {
  if (!y || n == 0) return hipSuccess;
  size_t blocks = (n + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(axpy_kernel, dim3((unsigned)blocks), dim3(256), 0, st, y, x, n);
  return hipGetLastError();
}

struct BwdChunkPlan {
  int L = 0;
  bool staged = false;   // B > 1 with several chunks: x, h, dx of a chunk go through staging
  pnr_cell sub{};
  size_t sub_bytes = 0, x_off = 0, h_off = 0, g_off = 0, dx_off = 0, h0_off = 0, gw_off = 0, gu_off = 0,
         gbx_off = 0, gbh_off = 0, mu_off[2] = {0, 0}, total = 0;
};
int plan_bwd_chunks(const pnr_cell* c, int chunk_len, BwdChunkPlan& p) {
  if (!c) return fail(PNR_E_INVALID, "cell descriptor is NULL");
  if (chunk_len < 1) return fail(PNR_E_INVALID, "chunk_len must be >= 1 (got %d)", chunk_len);
  if (c->T < 0) return fail(PNR_E_INVALID, "T must be >= 0 (got %d)", c->T);
  p.L = c->T < chunk_len ? c->T : chunk_len;
  p.sub = *c;
  p.sub.T = p.L;
  const int rc = validate_backward(&p.sub);
  if (rc) return rc;
  p.sub_bytes = make_bwd_layout(&p.sub).total;
  p.staged = c->B > 1 && c->T > p.L;
  const size_t B = c->B, L = p.L, D = c->D, Din = c->D_in, G = gates(c->kind), S = states(c->kind, c->D);
  const size_t f = sizeof(float), u_elems = c->kind == PNR_CELL_GRU ? G * D * D : G * D;
  size_t off = align_up(p.sub_bytes);
  p.g_off = off; off = align_up(off + f * B * L * S);
  if (p.staged) {
    p.x_off = off; off = align_up(off + dsize(c->x_dtype) * B * L * Din);
    p.h_off = off; off = align_up(off + f * B * L * S);
    p.dx_off = off; off = align_up(off + f * B * L * Din);
  }
  p.h0_off = off; off = align_up(off + f * B * S);
  p.gw_off = off; off = align_up(off + f * G * D * Din);
  p.gu_off = off; off = align_up(off + f * u_elems);
  p.gbx_off = off; off = align_up(off + f * G * D);
  p.gbh_off = off; off = align_up(off + f * G * D);
  for (int i = 0; i < 2; ++i) { p.mu_off[i] = off; off = align_up(off + f * B * S); }
  p.total = off;
  return 0;
}
}  // namespace

size_t pnr_workspace_bytes_backward_chunked(const pnr_cell* cell, int chunk_len) {
  BwdChunkPlan p;
  if (plan_bwd_chunks(cell, chunk_len, p) != 0) return 0;
  return p.total;
}

int pnr_backward_chunked(const pnr_cell* cell, const pnr_params* params, const void* x, const void* h0, const void* h,
                         const void* grad_h, void* grad_x, void* grad_W, void* grad_U, void* grad_b_x,
                         void* grad_b_h, void* grad_h0, int chunk_len) {
  g_last.reset();
  g_prof.valid = false;
  BwdChunkPlan p;
  int rc = plan_bwd_chunks(cell, chunk_len, p);
  if (rc) return rc;
  if (!params) return fail(PNR_E_INVALID, "params is NULL");
  if (!params->W || !params->U || (cell->T > 0 && (!x || !h || !grad_h)))
    return fail(PNR_E_INVALID, "W, U and (for T > 0) x, h and grad_h must be non-NULL");
  if (!cell->workspace) return fail(PNR_E_WORKSPACE, "workspace is NULL (%zu bytes required)", p.total);
  if ((uintptr_t)cell->workspace % 256) return fail(PNR_E_WORKSPACE, "workspace must be 256-byte aligned");
  if (cell->workspace_bytes < p.total)
    return fail(PNR_E_WORKSPACE, "workspace has %zu bytes, %zu required", cell->workspace_bytes, p.total);
  if (cell->T == 0) {
    pnr_cell sub = p.sub;
    sub.workspace_bytes = p.sub_bytes;
    return pnr_backward(&sub, params, x, h0, h, grad_h, grad_x, grad_W, grad_U, grad_b_x, grad_b_h, grad_h0);
  }
  hipStream_t st = reinterpret_cast<hipStream_t>(cell->stream);
  char* ws = static_cast<char*>(cell->workspace);
  auto fp = [&](size_t off) { return reinterpret_cast<float*>(ws + off); };
  const size_t B = cell->B, T = cell->T, D = cell->D, Din = cell->D_in, G = gates(cell->kind);
  const size_t S = states(cell->kind, cell->D), xes = dsize(cell->x_dtype), f = sizeof(float);
  const size_t u_elems = cell->kind == PNR_CELL_GRU ? G * D * D : G * D;
  const char* xb = static_cast<const char*>(x);
  const char* hb = static_cast<const char*>(h);
  const char* gb = static_cast<const char*>(grad_h);
  const int nck = (int)((T + p.L - 1) / p.L);
  int status = PNR_OK, iters = 0, mu = 0;
  double residual = 0.0;
  std::vector<double> hist;
  pnr_profile acc{};
  bool prof_ok = g_prof.on;
  for (int c = nck - 1; c >= 0; --c) {
    const size_t t0 = (size_t)c * p.L, Lc = std::min((size_t)p.L, T - t0);
    pnr_cell sub = p.sub;
    sub.T = (int)Lc;
    sub.workspace = ws;
    sub.workspace_bytes = p.sub_bytes;
    // the chunk's loss gradient, with the adjoint from the later chunk at its last step
    float* gc = fp(p.g_off);
    PNR_HIP(hipMemcpy2DAsync(gc, Lc * S * f, gb + t0 * S * f, T * S * f, Lc * S * f, B, hipMemcpyDeviceToDevice, st));
    if (c < nck - 1)
      hipLaunchKernelGGL(add_last_row_kernel, dim3((unsigned)((B * S + 255) / 256)), dim3(256), 0, st, gc,
                         fp(p.mu_off[mu ^ 1]), (int)B, (int)Lc, (int)S);
    const void* xc = xb + t0 * Din * xes;
    const void* hc = hb + t0 * S * f;
    void* dxc = grad_x ? static_cast<char*>(grad_x) + t0 * Din * f : nullptr;
    if (p.staged) {
      PNR_HIP(hipMemcpy2DAsync(ws + p.x_off, Lc * Din * xes, xc, T * Din * xes, Lc * Din * xes, B,
                               hipMemcpyDeviceToDevice, st));
      PNR_HIP(hipMemcpy2DAsync(ws + p.h_off, Lc * S * f, hc, T * S * f, Lc * S * f, B, hipMemcpyDeviceToDevice, st));
      xc = ws + p.x_off;
      hc = ws + p.h_off;
      if (dxc) dxc = ws + p.dx_off;
    }
    // the state before the chunk: h0, or the last state of the earlier chunk
    const void* h0c = h0;
    if (t0 > 0) {
      PNR_HIP(hipMemcpy2DAsync(ws + p.h0_off, S * f, hb + (t0 - 1) * S * f, T * S * f, S * f, B,
                               hipMemcpyDeviceToDevice, st));
      h0c = ws + p.h0_off;
    }
    // the first chunk processed writes the weight gradients, the others are added to them
    const bool first = c == nck - 1;
    float* gW = grad_W ? (first ? static_cast<float*>(grad_W) : fp(p.gw_off)) : nullptr;
    float* gU = grad_U ? (first ? static_cast<float*>(grad_U) : fp(p.gu_off)) : nullptr;
    float* gbx = grad_b_x ? (first ? static_cast<float*>(grad_b_x) : fp(p.gbx_off)) : nullptr;
    float* gbh = grad_b_h ? (first ? static_cast<float*>(grad_b_h) : fp(p.gbh_off)) : nullptr;
    // dL/d(state before the chunk): the next chunk's carry, or dL/dh0 for the first chunk
    float* dmu = c > 0 ? fp(p.mu_off[mu]) : static_cast<float*>(grad_h0);
    rc = pnr_backward(&sub, params, xc, h0c, hc, gc, dxc, gW, gU, gbx, gbh, dmu);
    if (rc < 0) return rc;   // g_last.err holds the chunk's error
    if (status_rank(rc) > status_rank(status)) status = rc;
    if (prof_ok && g_prof.valid) {
      const pnr_profile& q = g_prof.last;
      acc.total_ms += q.total_ms; acc.proj_ms += q.proj_ms; acc.newton_ms += q.newton_ms; acc.out_ms += q.out_ms;
      acc.passes += q.passes;
    } else {
      prof_ok = false;
    }
    iters += g_last.iters;
    if (!(g_last.residual <= residual)) residual = g_last.residual;
    for (size_t i = 0; i < g_last.hist.size(); ++i) hist.push_back(g_last.hist[i]);
    if (p.staged && grad_x)
      PNR_HIP(hipMemcpy2DAsync(static_cast<char*>(grad_x) + t0 * Din * f, T * Din * f, dxc, Lc * Din * f,
                               Lc * Din * f, B, hipMemcpyDeviceToDevice, st));
    if (!first) {
      PNR_HIP(launch_axpy(static_cast<float*>(grad_W), gW, G * D * Din, st));
      PNR_HIP(launch_axpy(static_cast<float*>(grad_U), gU, u_elems, st));
      PNR_HIP(launch_axpy(static_cast<float*>(grad_b_x), gbx, G * D, st));
      PNR_HIP(launch_axpy(static_cast<float*>(grad_b_h), gbh, G * D, st));
    }
    mu ^= 1;
  }
  PNR_HIP(hipStreamSynchronize(st));
  g_last.iters = iters;
  g_last.residual = residual;
  g_last.hist.assign(hist.data(), hist.data() + hist.size());
  g_prof.valid = prof_ok;
  if (prof_ok) g_prof.last = acc;
  return status;
}

size_t pnr_scan_workspace_bytes(int kind, int R, int T, int tile_len) {
  if ((kind != 1 && kind != 2) || R < 0 || T < 0) {
    fail(PNR_E_INVALID, "bad scan arguments");
    return 0;
  }
  if (tile_len == 0) tile_len = scan_default_tile(kind);
  const size_t tiles = (size_t)R * ((T + tile_len - 1) / (tile_len > 0 ? tile_len : 1));
  return align_up(sizeof(Ctrl)) + align_up(sizeof(uint64_t) * (tiles * scan_slot_words(kind) + 1));
}

int pnr_scan(int kind, int R, int T, const float* A, const float* b, float* d, int tile_len, void* workspace,
             size_t workspace_bytes, void* stream) {
  g_last.reset();
  if (kind != 1 && kind != 2) return fail(PNR_E_INVALID, "scan kind must be 1 (diagonal) or 2 (2x2)");
  if (R < 0 || T < 0) return fail(PNR_E_INVALID, "R and T must be >= 0");
  if (tile_len == 0) tile_len = scan_default_tile(kind);
  if (tile_len != PNR_BLOCK && tile_len != 2 * PNR_BLOCK && tile_len != 4 * PNR_BLOCK && tile_len != 8 * PNR_BLOCK)
    return fail(PNR_E_INVALID, "tile_len must be 0, 256, 512, 1024 or 2048");
  if (R == 0 || T == 0) return PNR_OK;
  if (!A || !b || !d) return fail(PNR_E_INVALID, "A, b and d must be non-NULL");
  const size_t need = pnr_scan_workspace_bytes(kind, R, T, tile_len);
  if (!workspace || (uintptr_t)workspace % 256 || workspace_bytes < need)
    return fail(PNR_E_WORKSPACE, "workspace must be 256-byte aligned and hold %zu bytes", need);
  int num_cu = 0, rc;
  if ((rc = device_info(&num_cu))) return rc;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  Ctrl* ctrl = reinterpret_cast<Ctrl*>(workspace);
  uint64_t* slots = reinterpret_cast<uint64_t*>(static_cast<char*>(workspace) + align_up(sizeof(Ctrl)));
  const size_t tiles = (size_t)R * ((T + tile_len - 1) / tile_len);
  PNR_HIP(launch_init(ctrl, slots, tiles * scan_slot_words(kind), nullptr, 0, st));
  PNR_HIP(launch_scan(kind, R, T, A, b, d, tile_len, slots, ctrl, num_cu, st));
  PNR_HIP(hipStreamSynchronize(st));
  return PNR_OK;
}

}  // extern "C"
