// The Newton loop for the diagonal-recurrence cells (GRU_DIAG, LSTM_DIAG), one fused
// pass per iteration: cell + Jacobian + residual (every step at once), residual max
// (wave -> LDS -> block partial -> the last block at the grid barrier), and the linear
// solve d_t = J_t d_{t-1} + r_t as a scan of affine maps (thread-serial -> wave DPP ->
// LDS -> carry along a row, or a decoupled look-back across tiles), followed by the
// update s <- s + d.  All iterations run inside one persistent, co-resident grid.
//
// Method: ParaRNN overview page, "Technical Implementation" (Newton's Iteration: a
// Jacobian per iteration, block lower-triangular system, Jacobian reuse; Parallel
// Reduction: block-local reduction, results to global memory, a final block merges);
// quasi-DEER diagonal Jacobian from "Towards Scalable and Stable Parallelization of
// Nonlinear RNNs" (abstract).  With elementwise recurrent weights the exact Jacobian
// of GRU_DIAG is diagonal and that of LSTM_DIAG is one 2x2 block per channel ((c, h)
// of the same channel), so every channel is an independent row.
//
// Layout (time-contiguous rows): gx [B][G][D][T], states [B][S][T] with S = D (GRU) or
// 2D (LSTM: c rows 0..D-1, h rows D..2D-1).  A row (b, d) is cut into tiles of
// PNR_BLOCK*N steps; each thread owns N consecutive steps, loaded as float4s.
//
// The Jacobian is never stored.  A reused (stale) Jacobian is rebuilt from the state
// it was taken at (Hjac), which costs one extra state read instead of a Jacobian
// write + read.
#include "common.h"
#include "diag_cell.h"
#include "kernels.h"

namespace pnr {

// slot I/O for the two element kinds
__device__ __forceinline__ void put_agg(uint64_t* s, uint32_t ep, const Aff1& e) {
  slot_put(s, ep, e.a); slot_put(s + 1, ep, e.b);
}
__device__ __forceinline__ bool get_agg(const uint64_t* s, uint32_t ep, Aff1& e) {
  bool ok = slot_get(s, ep, e.a);
  ok &= slot_get(s + 1, ep, e.b);
  return ok;
}
__device__ __forceinline__ void put_agg(uint64_t* s, uint32_t ep, const Aff2& e) {
  slot_put(s, ep, e.a00); slot_put(s + 1, ep, e.a01); slot_put(s + 2, ep, e.a10);
  slot_put(s + 3, ep, e.a11); slot_put(s + 4, ep, e.b0); slot_put(s + 5, ep, e.b1);
}
__device__ __forceinline__ bool get_agg(const uint64_t* s, uint32_t ep, Aff2& e) {
  bool ok = slot_get(s, ep, e.a00);
  ok &= slot_get(s + 1, ep, e.a01);
  ok &= slot_get(s + 2, ep, e.a10);
  ok &= slot_get(s + 3, ep, e.a11);
  ok &= slot_get(s + 4, ep, e.b0);
  ok &= slot_get(s + 5, ep, e.b1);
  return ok;
}
__device__ __forceinline__ void put_pre(uint64_t* s, uint32_t ep, float d) { slot_put(s, ep, d); }
__device__ __forceinline__ bool get_pre(const uint64_t* s, uint32_t ep, float& d) { return slot_get(s, ep, d); }
__device__ __forceinline__ void put_pre(uint64_t* s, uint32_t ep, float2 d) {
  slot_put(s, ep, d.x); slot_put(s + 1, ep, d.y);
}
__device__ __forceinline__ bool get_pre(const uint64_t* s, uint32_t ep, float2& d) {
  bool ok = slot_get(s, ep, d.x);
  ok &= slot_get(s + 1, ep, d.y);
  return ok;
}

// Decoupled look-back over a window of 64 predecessors, run by one whole wave: lane w
// inspects tile (tile-1-w).  The nearest predecessor that has published its inclusive
// prefix, with every tile after it having published its aggregate, resolves the
// increment entering this tile: d_in = agg_{tile-1} o ... o agg_{p+1} (prefix_p).  If no
// prefix is visible in the window yet, the wave waits and reads the window again; tiles
// publish prefixes in order from the start of each row, so a resolved prefix moves up
// to 64 tiles per round trip.  Returns d_in in every lane.  The wait is bounded.
template <class CellT>
__device__ typename DeltaOf<typename CellT::E>::T lookback_window(uint64_t* slots, int tile, int seg,
                                                                uint32_t ep, const typename CellT::E& tot,
                                                                Ctrl* ctrl) {
  using E = typename CellT::E;
  using Dl = typename DeltaOf<E>::T;
  constexpr int AW = CellT::AGG_WORDS, SW = CellT::AGG_WORDS + CellT::PRE_WORDS;
  const int lane = (int)lane_id();
  uint64_t* mine = slots + (size_t)tile * SW;
  const E idn = identity_of<E>();
  if (seg == 0) {
    if (lane == 0) put_pre(mine + AW, ep, apply(tot, DeltaOf<E>::zero()));
    return DeltaOf<E>::zero();
  }
  if (lane == 0) put_agg(mine, ep, tot);
  uint32_t spins = 0;
  while (true) {
    const bool valid = lane < seg;
    int st = 0;
    E e = idn;
    Dl pre = DeltaOf<E>::zero();
    if (valid) {
      // both reads are issued before either is tested
      const uint64_t* s = slots + (size_t)(tile - 1 - lane) * SW;
      const bool has_pre = get_pre(s + AW, ep, pre);
      const bool has_agg = get_agg(s, ep, e);
      st = has_pre ? 2 : (has_agg ? 1 : 0);
    }
    const uint64_t pm = __ballot(st == 2);
    const uint64_t bad = __ballot(valid && st == 0);
    if (pm) {
      const int p = __ffsll((long long)pm) - 1;
      const uint64_t before = p == 0 ? 0ull : ((1ull << p) - 1ull);
      if ((bad & before) == 0) {
        // lane 0 ends with e_0 o ... o e_{p-1}; lanes at or past p hold nothing and are never
        // composed in (no identity products: see select_aff)
        E x = lane < p ? e : idn;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
          E o = shfl_down_e(x, off);
          if (lane + off < p) x = compose(x, o);
        }
        const E x0 = readlane_aff(x, 0);
        const Dl din = apply(x0, readlane_d(pre, p));
        if (lane == 0) put_pre(mine + AW, ep, apply(tot, din));
        return din;
      }
    }
    if (++spins > kSpinLimit) {
      if (lane == 0) record_fault(ctrl, 1);
      return DeltaOf<E>::zero();
    }
    backoff(spins);
  }
}

// ---------------------------------------------------------------------------------
// One tile (PNR_BLOCK*N consecutive steps of one row): residuals and Jacobians, the
// scan, and the update.  d_in comes from the caller's carry (row walk) or from the
// look-back.  Returns the increment at the tile's last step (the next tile's carry).
template <int CELL>
struct TileShared {
  typename DiagCell<CELL>::E wtot[PNR_WAVES];
  typename DeltaOf<typename DiagCell<CELL>::E>::T din;
};

struct IterView {
  const float* Hcur;
  const float* Hjac;
  float* Hnext;
  bool cur_zero, jac_zero, stale;
  uint32_t ep;
};

// What the tiles of a row share: the cell's per-channel parameters, and the bounded
// iteration's state limit (GRU: max(1, |h0|); LSTM: |c0|, grown by one per step).
template <int CELL>
struct RowPar {
  typename DiagCell<CELL>::Par q;
  float lim;
};

template <int CELL>
__device__ __forceinline__ RowPar<CELL> load_row(const DiagLoopArgs& a, int row) {
  using C = DiagCell<CELL>;
  const int D = a.D, S = D * C::SP;
  const int b = row / D, d = row - b * D;
  RowPar<CELL> r;
  r.q = C::load_par(a.u, a.bh, D, d);
  const float h0 = a.bounded && a.h0 ? fabsf(a.h0[(size_t)b * S + d]) : 0.f;
  r.lim = CELL == PNR_CELL_GRU_DIAG ? fmaxf(1.f, h0) : h0;
  return r;
}

// Everything a tile reads from HBM, gathered before any of it is used.
template <int CELL, int N>
struct TileIn {
  float g[DiagCell<CELL>::G][N];     // gate pre-activations
  float s[DiagCell<CELL>::SP][N];    // current iterate (LSTM: c, then h)
  float sj[DiagCell<CELL>::SP][N];   // state the Jacobian is taken at (reuse passes)
  float p[DiagCell<CELL>::SP];       // lane 0: the state before the wave's first step
  float pj[DiagCell<CELL>::SP];
};

template <int CELL, int N>
__device__ __forceinline__ void load_tile(const DiagLoopArgs& a, int row, int seg, bool walk, bool stale,
                                          const IterView& v, TileIn<CELL, N>& in) {
  using C = DiagCell<CELL>;
  constexpr int G = C::G, SP = C::SP;
  constexpr int TILE = PNR_BLOCK * N;
  const int tid = threadIdx.x, lane = tid & 63;
  const int D = a.D, T = a.T;
  const int S = D * SP;
  const bool vec = (T & 3) == 0;
  const int b = row / D, d = row - b * D;
  const int tb = seg * TILE + tid * N;
#pragma unroll
  for (int gg = 0; gg < G; ++gg) load_n(a.gx + ((size_t)(b * G + gg) * D + d) * T, tb, T, vec, N, in.g[gg]);
  // The state before a thread's first step is the previous lane's last one (DPP); only
  // lane 0 of each wave loads it.  Before a tile's first step it was written by the block
  // owning the previous tile: read it coherently (everything else here is this block's own).
  const bool halo_other = tid == 0 && !walk;
#pragma unroll
  for (int k = 0; k < SP; ++k) {
    const size_t off = ((size_t)b * S + (size_t)k * D + d) * T;
    if (v.cur_zero) { for (int i = 0; i < N; ++i) in.s[k][i] = 0.f; }
    else load_n(v.Hcur + off, tb, T, vec, N, in.s[k]);
    float p = 0.f;
    if (lane == 0) {
      if (tb == 0) p = a.h0 ? a.h0[(size_t)b * S + (size_t)k * D + d] : 0.f;
      else if (v.cur_zero || tb > T) p = 0.f;
      else p = halo_other ? coherent_load(v.Hcur + off + tb - 1) : v.Hcur[off + tb - 1];
    }
    in.p[k] = p;
    if (stale) {
      if (v.jac_zero) { for (int i = 0; i < N; ++i) in.sj[k][i] = 0.f; }
      else load_n(v.Hjac + off, tb, T, vec, N, in.sj[k]);
      float pj = 0.f;
      if (lane == 0) {
        if (tb == 0) pj = a.h0 ? a.h0[(size_t)b * S + (size_t)k * D + d] : 0.f;
        else if (v.jac_zero || tb > T) pj = 0.f;
        else pj = halo_other ? coherent_load(v.Hjac + off + tb - 1) : v.Hjac[off + tb - 1];
      }
      in.pj[k] = pj;
    }
  }
}

// LDS of the staged row walk: one staged tile, and what the waves of a tile pass on.
template <int CELL, int N>
struct WalkStage {
  static constexpr int PLANES = DiagCell<CELL>::G + 2 * DiagCell<CELL>::SP;
  float pl[PLANES][PNR_BLOCK * N];                   // staged planes, in step order
  float edge[2][PNR_WAVES][2 * DiagCell<CELL>::SP];  // each wave's last current / Jacobian state, by tile parity
  RowPar<CELL> rp;                                   // the row's parameters
  int fault;                                         // the block's fault decision
};

// Direct-to-LDS staging of one full tile for the row walk (global_load_lds_dwordx4: lane
// l of a wave's load writes bytes 16l..16l+15 of a 1 KB run, so plane p of the tile lands
// in step order as pl[p][0 .. TILE)).  Planes: the gates, the current iterate, and on
// reuse passes the state the Jacobian is taken at.  No register holds a staged tile, so
// the next tile's loads can be in flight through the whole of the current tile.
template <int CELL, int N>
__device__ __forceinline__ void stage_issue(const DiagLoopArgs& a, const IterView& v, bool stale, int row, int seg,
                                            WalkStage<CELL, N>& st) {
  using C = DiagCell<CELL>;
  constexpr int G = C::G, SP = C::SP, TILE = PNR_BLOCK * N;
  static_assert(N == 4, "one 16-byte load per lane and plane");
  const int tid = threadIdx.x;
  const int D = a.D, T = a.T, S = D * SP;
  const int b = row / D, d = row - b * D;
  const size_t tb = (size_t)seg * TILE + tid * N;
  const int w0 = (tid >> 6) * 64 * N;   // the wave's run in each plane
#pragma unroll
  for (int gg = 0; gg < G; ++gg)
    lds_load16(a.gx + ((size_t)(b * G + gg) * D + d) * T + tb, &st.pl[gg][w0]);
  if (!v.cur_zero) {
#pragma unroll
    for (int k = 0; k < SP; ++k)
      lds_load16(v.Hcur + ((size_t)b * S + (size_t)k * D + d) * T + tb, &st.pl[G + k][w0]);
  }
  if (stale && !v.jac_zero) {
#pragma unroll
    for (int k = 0; k < SP; ++k)
      lds_load16(v.Hjac + ((size_t)b * S + (size_t)k * D + d) * T + tb, &st.pl[G + SP + k][w0]);
  }
}

// A wave's part of a staged tile into registers: only what its own loads brought in, so
// that the wait before these reads (the compiler's) is a wait for this wave's loads alone.
// The steps before the wave's first (in.p, in.pj) are filled in by the caller.
template <int CELL, int N>
__device__ __forceinline__ void stage_read(const IterView& v, bool stale, const WalkStage<CELL, N>& st,
                                           TileIn<CELL, N>& in) {
  using C = DiagCell<CELL>;
  constexpr int G = C::G, SP = C::SP;
  const int tid = threadIdx.x;
  auto rd = [&](const float* p, float* o) {
    const float4 x = *reinterpret_cast<const float4*>(p);
    o[0] = x.x; o[1] = x.y; o[2] = x.z; o[3] = x.w;
  };
#pragma unroll
  for (int gg = 0; gg < G; ++gg) rd(&st.pl[gg][tid * N], in.g[gg]);
#pragma unroll
  for (int k = 0; k < SP; ++k) {
    if (v.cur_zero) { for (int i = 0; i < N; ++i) in.s[k][i] = 0.f; }
    else rd(&st.pl[G + k][tid * N], in.s[k]);
    if (stale) {
      if (v.jac_zero) { for (int i = 0; i < N; ++i) in.sj[k][i] = 0.f; }
      else rd(&st.pl[G + SP + k][tid * N], in.sj[k]);
    }
  }
}

template <int CELL, int N, bool RESID_ONLY>
__device__ __forceinline__ typename DeltaOf<typename DiagCell<CELL>::E>::T diag_tile(
    const DiagLoopArgs& a, TileShared<CELL>& sh, const TileIn<CELL, N>& in, const RowPar<CELL>& rp, int row, int seg,
    int tile, bool walk, typename DeltaOf<typename DiagCell<CELL>::E>::T carry, const IterView& v, uint32_t& blk_max) {
  using C = DiagCell<CELL>;
  using E = typename C::E;
  using Dl = typename DeltaOf<E>::T;
  constexpr int TILE = PNR_BLOCK * N;
  const int tid = threadIdx.x, wid = tid >> 6, lane = tid & 63;
  const int D = a.D, T = a.T;
  const int S = D * C::SP;
  const bool vec = (T & 3) == 0;
  const int b = row / D, d = row - b * D;
  const int tb = seg * TILE + tid * N;
  const bool stale = v.stale && !RESID_ONLY;
  const int jac_mode = a.jac_mode;

  const typename C::Par q = rp.q;
  uint32_t tmax = 0;
  E e[N];
  float hc[C::SP][N];
  if constexpr (CELL == PNR_CELL_GRU_DIAG) {
    const float p0 = wave_shr1(in.s[0][N - 1], in.p[0]);
    float pj[N];
    if (stale) {
      pj[0] = wave_shr1(in.sj[0][N - 1], in.pj[0]);
      for (int i = 1; i < N; ++i) pj[i] = in.sj[0][i - 1];
    }
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const float p = i == 0 ? p0 : in.s[0][i - 1];
      float gi[3] = {in.g[0][i], in.g[1][i], in.g[2][i]};
      float res, ja = 0.f;
      C::eval(q, gi, p, in.s[0][i], jac_mode, !stale && !RESID_ONLY, res, ja);
      if (stale) ja = C::jac_only(q, gi, pj[i], jac_mode);
      if (tb + i >= T) { res = 0.f; ja = 1.f; }
      tmax = max(tmax, abs_bits(res));
      e[i] = Aff1{ja, res};
      hc[0][i] = in.s[0][i];
    }
  } else {
    const float cp0 = wave_shr1(in.s[0][N - 1], in.p[0]);
    const float hp0 = wave_shr1(in.s[1][N - 1], in.p[1]);
    float cpj0 = 0.f, hpj0 = 0.f;
    if (stale) {
      cpj0 = wave_shr1(in.sj[0][N - 1], in.pj[0]);
      hpj0 = wave_shr1(in.sj[1][N - 1], in.pj[1]);
    }
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const float cp = i == 0 ? cp0 : in.s[0][i - 1];
      const float hp = i == 0 ? hp0 : in.s[1][i - 1];
      float gi[4] = {in.g[0][i], in.g[1][i], in.g[2][i], in.g[3][i]};
      float rc, rh;
      Aff2 J = aff_identity2();
      C::eval(q, gi, cp, hp, in.s[0][i], in.s[1][i], jac_mode, !stale && !RESID_ONLY, rc, rh, J);
      if (stale) {
        float dc, dh;
        const float cpj = i == 0 ? cpj0 : in.sj[0][i - 1];
        const float hpj = i == 0 ? hpj0 : in.sj[1][i - 1];
        C::eval(q, gi, cpj, hpj, 0.f, 0.f, jac_mode, true, dc, dh, J);
      }
      if (tb + i >= T) { rc = 0.f; rh = 0.f; J = aff_identity2(); }
      tmax = max(tmax, max(abs_bits(rc), abs_bits(rh)));
      J.b0 = rc; J.b1 = rh;
      e[i] = J;
      hc[0][i] = in.s[0][i];
      hc[1][i] = in.s[1][i];
    }
  }
  blk_max = max(blk_max, tmax);
  if constexpr (RESID_ONLY) {
    return DeltaOf<E>::zero();
  } else {
    // ---- scan: thread-serial, then wave (DPP), then block (LDS), then carry / look-back ----
    E agg = e[0];
#pragma unroll
    for (int i = 1; i < N; ++i) agg = compose(e[i], agg);
    const E idn = identity_of<E>();
    E incl = wave_inclusive_scan(agg, idn);
    if (lane == 63) sh.wtot[wid] = incl;
    __syncthreads();
    E tot = sh.wtot[0];
    for (int w = 1; w < PNR_WAVES; ++w) tot = compose(sh.wtot[w], tot);
    if (walk) {
      if (tid == 0) sh.din = carry;
    } else if (wid == 0) {
      const Dl din = lookback_window<C>(a.slots, tile, seg, v.ep, tot, a.ctrl);
      if (lane == 0) sh.din = din;
    }
    __syncthreads();
    const Dl din = sh.din;
    Dl dw = din;
    for (int w = 0; w < wid; ++w) dw = apply(sh.wtot[w], dw);
    Dl dout = apply(incl, dw);
    Dl dl = wave_shr1(dout, dw);   // increment entering this thread's first step

    // ---- fix-up: d_t = J_t d_{t-1} + r_t along the thread's steps, s <- s + d ----
    // Bounded iteration: the new iterate is projected onto the box every reachable state
    // lies in (a component the step made NaN keeps its current value).  GRU: h' is a
    // convex combination of tanh(.) and h, so |h_t| <= max(1, |h0|).  LSTM: |h_t| < 1 and
    // |c_t| < |c0| + t (c' = f c + i g, 0 < f, i < 1, |g| < 1).
    const bool bounded = a.bounded != 0;
    if constexpr (CELL == PNR_CELL_GRU_DIAG) {
      const float hb = rp.lim;
      float out[N];
#pragma unroll
      for (int i = 0; i < N; ++i) {
        dl = apply(e[i], dl);
        out[i] = hc[0][i] + dl;
        if (bounded) out[i] = project_state(out[i], hc[0][i], hb);
      }
      float* orow = v.Hnext + ((size_t)b * S + d) * T;
      store_n(orow, tb, T, vec, N, out);
      // the tile's last state is the next tile's halo, read by another block next pass
      if (!walk && tid == PNR_BLOCK - 1 && tb + N <= T) coherent_store(orow + tb + N - 1, out[N - 1]);
    } else {
      const float c0b = rp.lim;
      float oc[N], oh[N];
#pragma unroll
      for (int i = 0; i < N; ++i) {
        dl = apply(e[i], dl);
        oc[i] = hc[0][i] + dl.x;
        oh[i] = hc[1][i] + dl.y;
        if (bounded) {
          oc[i] = project_state(oc[i], hc[0][i], c0b + (float)(tb + i + 1));
          oh[i] = project_state(oh[i], hc[1][i], 1.f);
        }
      }
      float* crow = v.Hnext + ((size_t)b * S + d) * T;
      float* hrow = v.Hnext + ((size_t)b * S + D + d) * T;
      store_n(crow, tb, T, vec, N, oc);
      store_n(hrow, tb, T, vec, N, oh);
      // the tile's last state is the next tile's halo, read by another block next pass
      if (!walk && tid == PNR_BLOCK - 1 && tb + N <= T) {
        coherent_store(crow + tb + N - 1, oc[N - 1]);
        coherent_store(hrow + tb + N - 1, oh[N - 1]);
      }
    }
    const Dl tile_out = apply(tot, din);
    __syncthreads();   // sh is reused by the next tile
    return tile_out;
  }
}

// The row walk with the next tile staged in LDS while the current one is computed (full
// tiles only: T a multiple of the tile).  Per tile: publish each wave's last step (the
// next wave's predecessor) in LDS, barrier, issue the next tile's loads into the stage,
// then the tile's arithmetic, scans and stores, and last wait for this wave's staged
// loads and read its part of the next tile.  No wave reads another wave's staged loads,
// so each wave waits for its own only; the wait is explicit (vmcnt), since the compiler
// does not order LDS reads after direct-to-LDS loads by itself.  RESID_ONLY is a template
// argument so that each loop has one pattern of memory operations; its tiles have no
// barriers of their own, so it closes each tile with one (the LDS slots below are reused
// every two tiles).
template <int CELL, int N, bool RESID_ONLY>
__device__ __forceinline__ void walk_staged(const DiagLoopArgs& a, TileShared<CELL>& sh, WalkStage<CELL, N>& st,
                                            const IterView& v, bool stale, int n_items, uint32_t& blk_max) {
  using C = DiagCell<CELL>;
  using E = typename C::E;
  using Dl = typename DeltaOf<E>::T;
  constexpr int SP = C::SP;
  const int tid = threadIdx.x, wid = tid >> 6, lane = tid & 63;
  const int D = a.D, S = D * SP;
  const int tpr = a.tiles_per_row;
  const int my_rows = (int)blockIdx.x < n_items ? (n_items - 1 - (int)blockIdx.x) / (int)gridDim.x + 1 : 0;
  const int n_steps = my_rows * tpr;
  if (n_steps == 0) return;
  stage_issue<CELL, N>(a, v, stale, blockIdx.x, 0, st);
  TileIn<CELL, N> in;
  __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): the first tile's staged loads
  stage_read<CELL, N>(v, stale, st, in);
  int row = blockIdx.x, seg = 0;
  Dl carry = DeltaOf<E>::zero();
  for (int j = 0; j < n_steps; ++j) {
    const int par = j & 1;
    if (lane == 63) {
#pragma unroll
      for (int k = 0; k < SP; ++k) {
        st.edge[par][wid][k] = in.s[k][N - 1];
        if (stale) st.edge[par][wid][SP + k] = in.sj[k][N - 1];
      }
    }
    // a row's parameters and the fault flag, once per row
    if (seg == 0 && tid == 0) {
      st.fault = has_fault(a.ctrl);
      st.rp = load_row<CELL>(a, row);
    }
    __syncthreads();
    if (st.fault) break;   // the same decision in every wave
    const RowPar<CELL> rp = st.rp;
    // the step before the wave's first: h0 at a row's start, else the previous wave's last
    // step (for wave 0, the previous tile's last wave's)
    if (lane == 0) {
      const int b = row / D, d = row - b * D;
      const bool first = seg == 0 && wid == 0;
      const float* e = wid > 0 ? st.edge[par][wid - 1] : st.edge[par ^ 1][PNR_WAVES - 1];
#pragma unroll
      for (int k = 0; k < SP; ++k) {
        const float init = a.h0 ? a.h0[(size_t)b * S + (size_t)k * D + d] : 0.f;
        in.p[k] = first ? init : (v.cur_zero ? 0.f : e[k]);
        if (stale) in.pj[k] = first ? init : (v.jac_zero ? 0.f : e[SP + k]);
      }
    }
    const int nrow = seg + 1 < tpr ? row : row + (int)gridDim.x;
    const int nseg = seg + 1 < tpr ? seg + 1 : 0;
    const bool more = j + 1 < n_steps;
    if (more) stage_issue<CELL, N>(a, v, stale, nrow, nseg, st);
    carry = diag_tile<CELL, N, RESID_ONLY>(a, sh, in, rp, row, seg, 0, true, carry, v, blk_max);
    if (nseg == 0) carry = DeltaOf<E>::zero();
    row = nrow;
    seg = nseg;
    if (more) {
      __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): this wave's staged loads have landed
      stage_read<CELL, N>(v, stale, st, in);
    }
    if constexpr (RESID_ONLY) __syncthreads();
  }
  __builtin_amdgcn_s_waitcnt(0x0F70);   // no staged load outlives the walk
}

__device__ __forceinline__ int pick_next(int cur, int jac, int nbuf) {
  for (int i = 0; i < nbuf; ++i)
    if (i != cur && i != jac) return i;
  return -1;
}

// ---------------------------------------------------------------------------------
// The whole Newton loop in one persistent, co-resident grid.  Iteration k: blocks take
// work items from a ticket (a whole row in walk mode, one tile otherwise), then meet at
// a grid barrier whose last block merges the residual partials and decides; after the
// barrier every block reads the decision and either stops or starts iteration k+1.
// The state buffers rotate exactly as the host would rotate them: the next iterate goes
// to a buffer holding neither the current iterate nor the state the Jacobian is taken at.
// Registers capped at 128 VGPRs (four waves per SIMD) to keep enough loads in flight.
template <int CELL> constexpr int diag_min_waves() { return 4; }

template <int CELL, int N, bool STAGED>
__global__ void __launch_bounds__(PNR_BLOCK, diag_min_waves<CELL>()) diag_newton_kernel(DiagLoopArgs a) {
  using C = DiagCell<CELL>;
  using E = typename C::E;
  using Dl = typename DeltaOf<E>::T;
  __shared__ TileShared<CELL> sh;
  __shared__ uint32_t s_wmax[PNR_WAVES];
  Ctrl* ctrl = a.ctrl;
  const int tid = threadIdx.x, wid = tid >> 6, lane = tid & 63;
  const int n_items = a.walk ? a.n_rows : a.n_tiles;
  int cur = -1, jac = -1;
  for (int k = 0; k <= a.max_iters; ++k) {
    const bool resid_only = k == a.max_iters;
    // a new Jacobian every jac_every updates, or (adaptive refresh) when the finisher of
    // pass k-1 decided so; every block takes the same decision
    const bool refresh = a.refresh_ratio < 0.0
                             ? k % a.jac_every == 0
                             : (k == 0 || __hip_atomic_load(&ctrl->refresh, __ATOMIC_RELAXED,
                                                            __HIP_MEMORY_SCOPE_AGENT) != 0);
    if (!resid_only && refresh) jac = cur;
    const int next = resid_only ? cur : pick_next(cur, jac, a.nbuf);
    IterView v;
    v.Hcur = cur >= 0 ? a.H[cur] : nullptr;
    v.Hjac = jac >= 0 ? a.H[jac] : nullptr;
    v.Hnext = next >= 0 ? a.H[next] : nullptr;
    v.cur_zero = cur < 0;
    v.jac_zero = jac < 0;
    v.stale = jac != cur;
    v.ep = (uint32_t)k + 1u;
    uint32_t blk_max = 0;
    // Static assignment, items in increasing order per block: with a co-resident grid
    // the lowest unfinished tile never waits on anything, so the look-back always ends.
    if constexpr (STAGED) {
      __shared__ __align__(16) WalkStage<CELL, N> st;
      if (resid_only)
        walk_staged<CELL, N, true>(a, sh, st, v, false, n_items, blk_max);
      else
        walk_staged<CELL, N, false>(a, sh, st, v, v.stale, n_items, blk_max);
    } else {
    for (int item = blockIdx.x; item < n_items; item += gridDim.x) {
      if (a.walk) {
        Dl carry = DeltaOf<E>::zero();
        for (int seg = 0; seg < a.tiles_per_row; ++seg) {
          const RowPar<CELL> rp = load_row<CELL>(a, item);
          TileIn<CELL, N> in;
          load_tile<CELL, N>(a, item, seg, true, v.stale && !resid_only, v, in);
          if (resid_only)
            diag_tile<CELL, N, true>(a, sh, in, rp, item, seg, 0, true, carry, v, blk_max);
          else
            carry = diag_tile<CELL, N, false>(a, sh, in, rp, item, seg, 0, true, carry, v, blk_max);
        }
      } else {
        const int row = item / a.tiles_per_row, seg = item - row * a.tiles_per_row;
        const RowPar<CELL> rp = load_row<CELL>(a, row);
        TileIn<CELL, N> in;
        load_tile<CELL, N>(a, row, seg, false, v.stale && !resid_only, v, in);
        if (resid_only)
          diag_tile<CELL, N, true>(a, sh, in, rp, row, seg, item, false, DeltaOf<E>::zero(), v, blk_max);
        else
          diag_tile<CELL, N, false>(a, sh, in, rp, row, seg, item, false, DeltaOf<E>::zero(), v, blk_max);
      }
      if (has_fault(ctrl)) break;
    }
    }
    // ---- two-level residual max: block partial -> global; the barrier's last block merges ----
    blk_max = wave_max_u32(blk_max);
    if (lane == 0) s_wmax[wid] = blk_max;
    __syncthreads();
    if (tid == 0) {
      uint32_t m = s_wmax[0];
      for (int w = 1; w < PNR_WAVES; ++w) m = max(m, s_wmax[w]);
      __hip_atomic_store(&a.partials[blockIdx.x], m, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    grid_barrier(ctrl, [&]() {
      uint32_t m = 0;
      for (int i = tid; i < (int)gridDim.x; i += PNR_BLOCK)
        m = max(m, __hip_atomic_load(&a.partials[i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
      m = wave_max_u32(m);
      __syncthreads();
      if (lane == 0) s_wmax[wid] = m;
      __syncthreads();
      if (tid == 0) {
        for (int w = 0; w < PNR_WAVES; ++w) m = max(m, s_wmax[w]);
        finish_iteration(ctrl, a.rho_hist, bits_to_rho(m), k, cur, a.max_iters, a.tol, a.refresh_ratio,
                         a.jac_every);
      }
    });
    if (__hip_atomic_load(&ctrl->done, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) || has_fault(ctrl)) break;
    cur = next;
  }
}

// ---------------------------------------------------------------------------------
// Standalone scan d_t = A_t d_{t-1} + b_t over R independent rows: the same thread /
// wave / block / look-back machinery as the fused iteration, with the elements read
// from memory.  KIND 1: A, b, d are [R][T]; KIND 2: A [R][4][T], b and d [R][2][T].
struct ScanArgs {
  const float* A; const float* b; float* d;
  uint64_t* slots; Ctrl* ctrl;
  int R, T, tiles_per_row, n_tiles;
};

template <int KIND, int N>
__global__ void __launch_bounds__(PNR_BLOCK) scan_kernel(ScanArgs a) {
  using C = DiagCell<KIND == 1 ? PNR_CELL_GRU_DIAG : PNR_CELL_LSTM_DIAG>;
  using E = typename C::E;
  using Dl = typename DeltaOf<E>::T;
  constexpr int TILE = PNR_BLOCK * N;
  __shared__ int s_tile;
  __shared__ E s_wtot[PNR_WAVES];
  __shared__ Dl s_din;
  const int tid = threadIdx.x, wid = tid >> 6, lane = tid & 63;
  const int T = a.T;
  while (true) {
    if (tid == 0) s_tile = (int)atomicAdd(&a.ctrl->ticket, 1u);
    __syncthreads();
    const int tile = s_tile;
    if (tile >= a.n_tiles || has_fault(a.ctrl)) break;
    const int row = tile / a.tiles_per_row, seg = tile - row * a.tiles_per_row;
    const int tb = seg * TILE + tid * N;
    E e[N];
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const int t = tb + i;
      if (t < T) {
        if constexpr (KIND == 1) {
          e[i] = Aff1{a.A[(size_t)row * T + t], a.b[(size_t)row * T + t]};
        } else {
          const float* Ar = a.A + (size_t)row * 4 * T;
          const float* br = a.b + (size_t)row * 2 * T;
          e[i] = Aff2{Ar[t], Ar[T + t], Ar[2 * T + t], Ar[3 * T + t], br[t], br[T + t]};
        }
      } else {
        e[i] = identity_of<E>();
      }
    }
    E agg = e[0];
#pragma unroll
    for (int i = 1; i < N; ++i) agg = compose(e[i], agg);
    E incl = wave_inclusive_scan(agg, identity_of<E>());
    if (lane == 63) s_wtot[wid] = incl;
    __syncthreads();
    if (wid == 0) {
      E tot = s_wtot[0];
      for (int w = 1; w < PNR_WAVES; ++w) tot = compose(s_wtot[w], tot);
      const Dl din = lookback_window<C>(a.slots, tile, seg, 1u, tot, a.ctrl);
      if (lane == 0) s_din = din;
    }
    __syncthreads();
    Dl dw = s_din;
    for (int w = 0; w < wid; ++w) dw = apply(s_wtot[w], dw);
    Dl dl = wave_shr1(apply(incl, dw), dw);
#pragma unroll
    for (int i = 0; i < N; ++i) {
      dl = apply(e[i], dl);
      const int t = tb + i;
      if (t < T) {
        if constexpr (KIND == 1) {
          a.d[(size_t)row * T + t] = dl;
        } else {
          a.d[(size_t)row * 2 * T + t] = dl.x;
          a.d[(size_t)row * 2 * T + T + t] = dl.y;
        }
      }
    }
    __syncthreads();
  }
}

// consecutive steps per thread in the fused loop kernel (float4 loads per state row)
template <int CELL> constexpr int diag_n() { return CELL == PNR_CELL_LSTM_DIAG ? 4 : 8; }
constexpr int kScanN = 8;

int scan_default_tile(int) { return PNR_BLOCK * kScanN; }
int scan_slot_words(int kind) { return diag_slot_words(kind == 1 ? PNR_CELL_GRU_DIAG : PNR_CELL_LSTM_DIAG); }

template <int KIND, int N>
static hipError_t launch_scan_n(const ScanArgs& a, int num_cu, hipStream_t st) {
  int v = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&v, scan_kernel<KIND, N>, PNR_BLOCK, 0) != hipSuccess || v < 1)
    v = 1;
  long g = (long)v * num_cu;
  if (g > kMaxGrid) g = kMaxGrid;
  if (g > a.n_tiles) g = a.n_tiles;
  if (g < 1) g = 1;
  hipLaunchKernelGGL((scan_kernel<KIND, N>), dim3((int)g), dim3(PNR_BLOCK), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_scan(int kind, int R, int T, const float* A, const float* b, float* d, int tile_len,
                       uint64_t* slots, Ctrl* ctrl, int num_cu, hipStream_t st) {
  const int n = tile_len / PNR_BLOCK;
  ScanArgs a{A, b, d, slots, ctrl, R, T, (T + tile_len - 1) / tile_len, 0};
  a.n_tiles = R * a.tiles_per_row;
  if (a.n_tiles == 0) return hipSuccess;
#define PNR_SCAN_CASE(NN) \
  case NN: return kind == 1 ? launch_scan_n<1, NN>(a, num_cu, st) : launch_scan_n<2, NN>(a, num_cu, st);
  switch (n) {
    PNR_SCAN_CASE(1)
    PNR_SCAN_CASE(2)
    PNR_SCAN_CASE(4)
    PNR_SCAN_CASE(8)
    default: return hipErrorInvalidValue;
  }
#undef PNR_SCAN_CASE
}

// ---------------------------------------------------------------------------------
int diag_items_per_thread(int cell) {
  return cell == PNR_CELL_LSTM_DIAG ? diag_n<PNR_CELL_LSTM_DIAG>() : diag_n<PNR_CELL_GRU_DIAG>();
}
int diag_slot_words(int cell) {
  return cell == PNR_CELL_LSTM_DIAG ? DiagCell<PNR_CELL_LSTM_DIAG>::AGG_WORDS + DiagCell<PNR_CELL_LSTM_DIAG>::PRE_WORDS
                                    : DiagCell<PNR_CELL_GRU_DIAG>::AGG_WORDS + DiagCell<PNR_CELL_GRU_DIAG>::PRE_WORDS;
}

// The row walk with LDS staging: the LSTM with full tiles.
bool diag_staged(int cell, int walk, int T) {
  return cell == PNR_CELL_LSTM_DIAG && walk && T % (PNR_BLOCK * diag_n<PNR_CELL_LSTM_DIAG>()) == 0;
}

template <int CELL>
static int diag_capacity(int num_cu) {
  // per device and thread-safe (cached_occupancy); the smaller of the two variants, so that
  // the grid fits whichever is launched
  int per_cu = cached_occupancy((const void*)diag_newton_kernel<CELL, diag_n<CELL>(), false>, 0);
  if constexpr (CELL == PNR_CELL_LSTM_DIAG) {
    const int staged = cached_occupancy((const void*)diag_newton_kernel<CELL, diag_n<CELL>(), true>, 0);
    if (staged < per_cu) per_cu = staged;
  }
  if (per_cu < 1) per_cu = 1;
  long g = (long)per_cu * num_cu;
  return (int)(g > kMaxGrid ? kMaxGrid : g);
}

int diag_grid_capacity(int cell, int num_cu) {
  return cell == PNR_CELL_GRU_DIAG ? diag_capacity<PNR_CELL_GRU_DIAG>(num_cu)
                                   : diag_capacity<PNR_CELL_LSTM_DIAG>(num_cu);
}

hipError_t launch_diag_newton(int cell, const DiagLoopArgs& a, int grid, hipStream_t st) {
  void* args[] = {const_cast<DiagLoopArgs*>(&a)};
  const void* fn =
      cell == PNR_CELL_GRU_DIAG ? (const void*)diag_newton_kernel<PNR_CELL_GRU_DIAG, diag_n<PNR_CELL_GRU_DIAG>(), false>
      : diag_staged(cell, a.walk, a.T)
          ? (const void*)diag_newton_kernel<PNR_CELL_LSTM_DIAG, diag_n<PNR_CELL_LSTM_DIAG>(), true>
          : (const void*)diag_newton_kernel<PNR_CELL_LSTM_DIAG, diag_n<PNR_CELL_LSTM_DIAG>(), false>;
  return launch_persistent(fn, grid, 0, args, st);
}

// ---------------------------------------------------------------------------------
// Damped (Levenberg-Marquardt) Newton step -- quasi-ELK -- for the cells with elementwise
// recurrent weights ("Towards Scalable and Stable Parallelization of Nonlinear RNNs",
// abstract and the summary's "Approach": a trust region whose linear-Gaussian MAP solve
// is a Kalman filter and smoother; with the diagonal Jacobian, quasi-ELK).
//
// Each state component (the GRU's h; the LSTM's c and h, each with its own diagonal
// Jacobian entry) is its own scalar problem: the step D minimises
// sum_t (D_t - J_t D_{t-1} - r_t)^2 + lam sum_t D_t^2 (D_0 = 0), the smoothed mean of the
// state-space model D_t = J_t D_{t-1} + r_t + w_t (unit noise), 0 = D_t + v_t (noise
// variance 1/lam):
//   filter:   P- = J^2 P + 1,  m- = J m + r,  P = P- / (1 + lam P-),  m = m- / (1 + lam P-)
//   smoother: G_t = P_t J_{t+1} / P-_{t+1},  D_t = m_t + G_t (D_{t+1} - m-_{t+1}),  D_T = m_T.
// In homogeneous coordinates (u, v, n) with P = u / v and m = n / v one filter step is
// linear: u' = J^2 u + v, v' = lam J^2 u + (1 + lam) v, n' = r v + J n.  So the filter is
// one associative scan of 3x3 maps [[a b 0][c d 0][e f g]] (7 numbers), started from
// (0, 1, 0).  The new iterate h'_t = h_t + D_t obeys
//   h'_t = G_t h'_{t+1} + e_t,   e_t = m_t + h_t - G_t (m-_{t+1} + h_{t+1})
// (G = 0 and e = m + h at the last step), so the forward sweep -- which has P, m of each
// step and J, r, h of the step after it -- stores only G and e, and the backward sweep is
// one affine scan of them run backwards in time that writes h' directly: two planes
// written and read per component, and the current iterate is not read again.
//
// One block walks a whole row (channel): a forward sweep over its tiles evaluates the
// cell, residual and Jacobian and runs the filter; a backward sweep runs the smoother.
// Tiles, thread-serial / DPP / LDS scans and the carry between tiles are those of
// diag_newton_kernel; the backward sweep maps thread t to the (255 - t)-th run of steps
// so that lane order is reverse time and the same forward scan machinery applies.
template <> __device__ __forceinline__ Flt identity_of<Flt>() { return flt_identity(); }
__device__ __forceinline__ V3 wave_shr1(const V3& x, const V3& lane0) {
  return V3{wave_shr1(x.u, lane0.u), wave_shr1(x.v, lane0.v), wave_shr1(x.n, lane0.n)};
}

template <int K>   // state components per channel
struct ElkShared {
  Flt ftot[K][PNR_WAVES];
  Aff1 btot[K][PNR_WAVES];
  float nj[K][PNR_WAVES], nr[K][PNR_WAVES], nh[K][PNR_WAVES];   // each wave's first step: J, r, state
  V3 fcarry[K];      // filter state (P, 1, m) after the previous tile's last step
  float bcarry[K];   // new iterate at the step after the tile (backward sweep)
};

// Smoother coefficients of one step from its filtered P, m and state h, and the next
// step's Jacobian j1, residual r1 and state h1 (last: the row's last step).
__device__ __forceinline__ void elk_coeffs(float P, float m, float h, float j1, float r1, float h1, bool last,
                                           float& G, float& e) {
  if (last) {
    G = 0.f;
    e = m + h;
  } else {
    G = P * j1 * fast_rcp(fmaf(j1 * j1, P, 1.f));
    e = (m + h) - G * (fmaf(j1, m, r1) + h1);
  }
}

// Forward sweep over one tile: cell, residual, Jacobian, filter; stores G and e.
template <int CELL, int N>
__device__ __forceinline__ void elk_forward_tile(const ElkArgs& a, ElkShared<DiagCell<CELL>::SP>& sh, int b, int d,
                                                 int seg, const float* Hcur, bool resid_only, uint32_t& blk_max) {
  using C = DiagCell<CELL>;
  constexpr int K = C::SP, NG = C::G;
  constexpr int TILE = PNR_BLOCK * N;
  const int tid = threadIdx.x, wid = tid >> 6, lane = tid & 63;
  const int D = a.D, T = a.T, S = K * D;
  const bool vec = (T & 3) == 0;
  const int tb = seg * TILE + tid * N;
  const typename C::Par q = C::load_par(a.u, a.bh, D, d);
  size_t off[K];
#pragma unroll
  for (int k = 0; k < K; ++k) off[k] = ((size_t)b * S + k * D + d) * T;
  float g[NG][N], h[K][N], p0[K];
#pragma unroll
  for (int gg = 0; gg < NG; ++gg) load_n(a.gx + ((size_t)(b * NG + gg) * D + d) * T, tb, T, vec, N, g[gg]);
#pragma unroll
  for (int k = 0; k < K; ++k) {
    if (!Hcur) {
#pragma unroll
      for (int i = 0; i < N; ++i) h[k][i] = 0.f;
    } else {
      load_n(Hcur + off[k], tb, T, vec, N, h[k]);
    }
    // the state before the thread's first step: the previous lane's last one (DPP); lane 0
    // of each wave loads it (this block wrote it, or it is h0 / the zero guess)
    float v = 0.f;
    if (lane == 0) {
      if (tb == 0) v = a.h0 ? a.h0[(size_t)b * S + k * D + d] : 0.f;
      else if (Hcur && tb <= T) v = Hcur[off[k] + tb - 1];
    }
    p0[k] = wave_shr1(h[k][N - 1], v);
  }
  float jv[K][N], rv[K][N];
  uint32_t tmax = 0;
#pragma unroll
  for (int i = 0; i < N; ++i) {
    const bool in = tb + i < T;
    float gi[NG];
#pragma unroll
    for (int gg = 0; gg < NG; ++gg) gi[gg] = g[gg][i];
    if constexpr (CELL == PNR_CELL_GRU_DIAG) {
      float res, ja = 0.f;
      C::eval(q, gi, i == 0 ? p0[0] : h[0][i - 1], h[0][i], a.jac_mode, true, res, ja);
      rv[0][i] = in ? res : 0.f;
      jv[0][i] = ja;
    } else {
      float rc, rh;
      Aff2 J = aff_identity2();
      C::eval(q, gi, i == 0 ? p0[0] : h[0][i - 1], i == 0 ? p0[1] : h[1][i - 1], h[0][i], h[1][i], PNR_JAC_DIAG,
              true, rc, rh, J);
      rv[0][i] = in ? rc : 0.f;
      rv[1][i] = in ? rh : 0.f;
      jv[0][i] = J.a00;
      jv[1][i] = J.a11;
    }
#pragma unroll
    for (int k = 0; k < K; ++k) tmax = max(tmax, abs_bits(rv[k][i]));
  }
  blk_max = max(blk_max, tmax);
  if (resid_only) return;   // uniform over the block
  // ---- filter scan: thread-serial, wave (DPP), block (LDS), carry ----
  const float lam = a.lam;
  Flt F[K][N], incl[K];
#pragma unroll
  for (int k = 0; k < K; ++k) {
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const float j2 = jv[k][i] * jv[k][i];
      F[k][i] = tb + i < T ? Flt{j2, 1.f, lam * j2, 1.f + lam, 0.f, rv[k][i], jv[k][i]} : flt_identity();
    }
    Flt agg = F[k][0];
#pragma unroll
    for (int i = 1; i < N; ++i) agg = compose(F[k][i], agg);
    incl[k] = wave_inclusive_scan(agg, flt_identity());
    if (lane == 63) sh.ftot[k][wid] = incl[k];
    if (lane == 0) {
      sh.nj[k][wid] = jv[k][0];
      sh.nr[k][wid] = rv[k][0];
      sh.nh[k][wid] = h[k][0];
    }
  }
  __syncthreads();
  // the block's last step takes its coefficients in the next tile (thread 0 there), unless
  // it is the row's last step
  const int lim = (tid == PNR_BLOCK - 1 && tb + N < T) ? tb + N - 1 : T;
  V3 xlast[K];
#pragma unroll
  for (int k = 0; k < K; ++k) {
    V3 xw = sh.fcarry[k];   // filter state entering this wave's first step
    // the previous tile's last step: filtered (P, m) = the carry, state = p0
    float dG = 0.f, dE = 0.f;
    if (tid == 0 && seg > 0) elk_coeffs(xw.u, xw.n, p0[k], jv[k][0], rv[k][0], h[k][0], false, dG, dE);
    for (int w = 0; w < wid; ++w) xw = normalized(apply(sh.ftot[k][w], xw));
    V3 x = wave_shr1(normalized(apply(incl[k], xw)), xw);   // entering this thread's first step
    float Pv[N], mv[N];
#pragma unroll
    for (int i = 0; i < N; ++i) {
      x = normalized(apply(F[k][i], x));
      Pv[i] = x.u;
      mv[i] = x.n;
    }
    xlast[k] = x;
    // the step after the thread's last one: the next lane's first; lane 63 takes the next
    // wave's first from LDS
    float j1 = shfl_down_f(jv[k][0], 1), r1 = shfl_down_f(rv[k][0], 1), h1 = shfl_down_f(h[k][0], 1);
    if (lane == 63 && wid + 1 < PNR_WAVES) {
      j1 = sh.nj[k][wid + 1];
      r1 = sh.nr[k][wid + 1];
      h1 = sh.nh[k][wid + 1];
    }
    float Gv[N], Ev[N];
#pragma unroll
    for (int i = 0; i < N - 1; ++i)
      elk_coeffs(Pv[i], mv[i], h[k][i], jv[k][i + 1], rv[k][i + 1], h[k][i + 1], tb + i + 1 >= T, Gv[i], Ev[i]);
    elk_coeffs(Pv[N - 1], mv[N - 1], h[k][N - 1], j1, r1, h1, tb + N >= T, Gv[N - 1], Ev[N - 1]);
    store_n(a.Gs + off[k], tb, lim, vec, N, Gv);
    store_n(a.Es + off[k], tb, lim, vec, N, Ev);
    if (tid == 0 && seg > 0) {
      a.Gs[off[k] + tb - 1] = dG;
      a.Es[off[k] + tb - 1] = dE;
    }
  }
  __syncthreads();   // everyone has read ftot, nj / nr / nh and fcarry
  if (tid == PNR_BLOCK - 1) {
#pragma unroll
    for (int k = 0; k < K; ++k) sh.fcarry[k] = xlast[k];   // the next tile's carry
  }
  __syncthreads();
}

// Backward sweep over one tile: smoother, next iterate.  Thread t takes the run of N
// steps that starts at step (PNR_BLOCK - 1 - t) * N of the tile and walks it backwards.
template <int K, int N>
__device__ __forceinline__ void elk_backward_tile(const ElkArgs& a, ElkShared<K>& sh, int b, int d, int seg,
                                                  float* Hnext) {
  constexpr int TILE = PNR_BLOCK * N;
  const int tid = threadIdx.x, wid = tid >> 6, lane = tid & 63;
  const int D = a.D, T = a.T, S = K * D;
  const bool vec = (T & 3) == 0;
  const int tb = seg * TILE + (PNR_BLOCK - 1 - tid) * N;
  Aff1 e[K][N], incl[K];
#pragma unroll
  for (int k = 0; k < K; ++k) {
    const size_t off = ((size_t)b * S + k * D + d) * T;
    float Gv[N], Ev[N];
    load_n(a.Gs + off, tb, T, vec, N, Gv);
    load_n(a.Es + off, tb, T, vec, N, Ev);
    // h'_t = G_t h'_{t+1} + e_t, latest step first
#pragma unroll
    for (int i = 0; i < N; ++i) e[k][N - 1 - i] = tb + i < T ? Aff1{Gv[i], Ev[i]} : aff_identity1();
    Aff1 agg = e[k][0];
#pragma unroll
    for (int i = 1; i < N; ++i) agg = compose(e[k][i], agg);
    incl[k] = wave_inclusive_scan(agg, aff_identity1());
    if (lane == 63) sh.btot[k][wid] = incl[k];
  }
  __syncthreads();
  float first[K];
#pragma unroll
  for (int k = 0; k < K; ++k) {
    const size_t off = ((size_t)b * S + k * D + d) * T;
    float hw = sh.bcarry[k];   // new iterate at the step after this wave's runs
    for (int w = 0; w < wid; ++w) hw = apply(sh.btot[k][w], hw);
    float hl = wave_shr1(apply(incl[k], hw), hw);
    float out[N];
#pragma unroll
    for (int i = 0; i < N; ++i) {
      hl = apply(e[k][i], hl);   // step tb + N - 1 - i
      out[N - 1 - i] = hl;
    }
    store_n(Hnext + off, tb, T, vec, N, out);
    first[k] = hl;
  }
  __syncthreads();
  if (tid == PNR_BLOCK - 1) {
#pragma unroll
    for (int k = 0; k < K; ++k) sh.bcarry[k] = first[k];   // the tile's first step
  }
  __syncthreads();
}

template <int CELL, int N>
__global__ void __launch_bounds__(PNR_BLOCK, 2) elk_diag_kernel(ElkArgs a) {
  constexpr int K = DiagCell<CELL>::SP;
  __shared__ ElkShared<K> sh;
  __shared__ uint32_t s_wmax[PNR_WAVES];
  Ctrl* ctrl = a.ctrl;
  const int tid = threadIdx.x, wid = tid >> 6, lane = tid & 63;
  int cur = -1;
  for (int k = 0; k <= a.max_iters; ++k) {
    const bool resid_only = k == a.max_iters;
    const int next = resid_only ? cur : (cur == 0 ? 1 : 0);
    const float* Hcur = cur >= 0 ? a.H[cur] : nullptr;
    float* Hnext = a.H[next < 0 ? 0 : next];
    uint32_t blk_max = 0;
    for (int row = blockIdx.x; row < a.n_rows; row += gridDim.x) {
      const int b = row / a.D, d = row - b * a.D;
      if (tid == 0) {
#pragma unroll
        for (int c = 0; c < K; ++c) sh.fcarry[c] = V3{0.f, 1.f, 0.f};
      }
      __syncthreads();
      for (int seg = 0; seg < a.tiles_per_row; ++seg)
        elk_forward_tile<CELL, N>(a, sh, b, d, seg, Hcur, resid_only, blk_max);
      if (resid_only) continue;
      if (tid == 0) {
#pragma unroll
        for (int c = 0; c < K; ++c) sh.bcarry[c] = 0.f;
      }
      __syncthreads();
      for (int seg = a.tiles_per_row - 1; seg >= 0; --seg) elk_backward_tile<K, N>(a, sh, b, d, seg, Hnext);
      if (__syncthreads_or(has_fault(ctrl))) break;   // the same decision in every wave
    }
    blk_max = wave_max_u32(blk_max);
    if (lane == 0) s_wmax[wid] = blk_max;
    __syncthreads();
    if (tid == 0) {
      uint32_t m = s_wmax[0];
      for (int w = 1; w < PNR_WAVES; ++w) m = max(m, s_wmax[w]);
      __hip_atomic_store(&a.partials[blockIdx.x], m, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    grid_barrier(ctrl, [&]() {
      uint32_t m = 0;
      for (int i = tid; i < (int)gridDim.x; i += PNR_BLOCK)
        m = max(m, __hip_atomic_load(&a.partials[i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
      m = wave_max_u32(m);
      __syncthreads();
      if (lane == 0) s_wmax[wid] = m;
      __syncthreads();
      if (tid == 0) {
        for (int w = 0; w < PNR_WAVES; ++w) m = max(m, s_wmax[w]);
        finish_iteration(ctrl, a.rho_hist, bits_to_rho(m), k, cur, a.max_iters, a.tol);
      }
    });
    if (__hip_atomic_load(&ctrl->done, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) || has_fault(ctrl)) break;
    cur = next;
  }
}

constexpr int kElkN = 4;   // steps per thread (float4 loads per plane)

int elk_items_per_thread() { return kElkN; }

hipError_t launch_elk_diag(int cell, const ElkArgs& a, int num_cu, hipStream_t st) {
  const void* fn = cell == PNR_CELL_GRU_DIAG ? (const void*)elk_diag_kernel<PNR_CELL_GRU_DIAG, kElkN>
                                             : (const void*)elk_diag_kernel<PNR_CELL_LSTM_DIAG, kElkN>;
  const int per_cu = cached_occupancy(fn, 0);
  if (per_cu < 1) return hipErrorInvalidConfiguration;
  long g = (long)per_cu * num_cu;
  if (g > kMaxGrid) g = kMaxGrid;
  if (g > a.n_rows) g = a.n_rows;
  if (g < 1) g = 1;
  void* args[] = {const_cast<ElkArgs*>(&a)};
  return launch_persistent(fn, (int)g, 0, args, st);
}

// ---------------------------------------------------------------------------------
// Backward pass: gradients through the evaluated sequence, for the cells with
// elementwise recurrent weights (ParaRNN overview, "Newton's Iteration": the block
// lower-triangular system is solved by forward and by backward substitution; training
// through the parallel evaluation: "Parallelizing non-linear sequential models over the
// sequence length", abstract).
//
// With g_t = dL/ds_t and mu_t = J_t^T lam_t (what step t sends back to s_{t-1}), the
// adjoint lam_t = g_t + mu_{t+1} (mu_T = 0) gives mu_t = J_t^T mu_{t+1} + J_t^T g_t: an
// affine map built from step t's own state and input, so mu is one scan of such maps run
// backwards in time (the damped smoother's mirrored thread mapping).  Each thread then
// walks its steps from the last to the first, recomputes the gates, and sends lam_t back
// through them: pre-activation gradients (kept for the projection's gradients), the
// recurrent-weight and bias sums of the row, and mu_t.  mu at the row's first step is
// dL/dh0.  One block walks a whole row (channel) from its last tile to its first.

// GRU: h' = (1 - z) n + z p with gates r, z, n (pre-activations gx + u p + b).
__device__ __forceinline__ void vjp_gru(const DiagCell<PNR_CELL_GRU_DIAG>::Par& q, const float* g, float p,
                                        float lam, float* dgx, float* dgh, float& dprev) {
  const float ghr = fmaf(q.ur, p, q.br), ghz = fmaf(q.uz, p, q.bz), ghn = fmaf(q.un, p, q.bn);
  const float r = sigm(g[0] + ghr), z = sigm(g[1] + ghz);
  const float n = tanh_(fmaf(r, ghn, g[2]));
  const float dan = lam * (1.f - z) * (1.f - n * n);
  const float daz = lam * (p - n) * z * (1.f - z);
  const float dar = dan * ghn * r * (1.f - r);
  dgx[0] = dar; dgx[1] = daz; dgx[2] = dan;
  dgh[0] = dar; dgh[1] = daz; dgh[2] = dan * r;
  dprev = fmaf(lam, z, fmaf(q.ur, dgh[0], fmaf(q.uz, dgh[1], q.un * dgh[2])));
}

// LSTM: c' = f c + i g, h' = o tanh(c') with gates i, f, o, g (pre-activations gx + u h + b).
__device__ __forceinline__ void vjp_lstm(const DiagCell<PNR_CELL_LSTM_DIAG>::Par& q, const float* gx, float cp,
                                         float hp, float lc, float lh, float* da, float2& dprev) {
  const float i = sigm(gx[0] + fmaf(q.ui, hp, q.bi));
  const float f = sigm(gx[1] + fmaf(q.uf, hp, q.bf));
  const float o = sigm(gx[2] + fmaf(q.uo, hp, q.bo));
  const float g = tanh_(gx[3] + fmaf(q.ug, hp, q.bg));
  const float tau = tanh_(fmaf(f, cp, i * g));
  const float dcn = fmaf(lh * o, 1.f - tau * tau, lc);   // c' is reached directly and through h'
  da[0] = dcn * g * i * (1.f - i);
  da[1] = dcn * cp * f * (1.f - f);
  da[2] = lh * tau * o * (1.f - o);
  da[3] = dcn * i * (1.f - g * g);
  dprev = make_float2(dcn * f, fmaf(q.ui, da[0], fmaf(q.uf, da[1], fmaf(q.uo, da[2], q.ug * da[3]))));
}

__device__ __forceinline__ float wave_sum_f(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

template <int CELL>
struct BwdShared {
  using E = typename DiagCell<CELL>::E;
  E tot[PNR_WAVES];
  typename DeltaOf<E>::T carry;   // mu at the step after the tile
  float red[PNR_WAVES][3 * DiagCell<CELL>::G];
};

// One tile of the backward walk.  Thread t takes the run of N steps that starts at step
// (PNR_BLOCK - 1 - t) * N of the tile.  acc: the thread's sums (dU, db_h, db_x per gate).
// Returns mu at the thread's first step.
// N bf16 values at row[tb..tb+N) (8-byte stores when T is a multiple of 4), masked at T.
__device__ __forceinline__ void store_n_bf16(__bf16* __restrict__ row, int tb, int T, bool vec, int N,
                                             const float* in) {
  if (vec && tb + N <= T) {
    for (int v = 0; v < N / 4; ++v) {
      typedef __bf16 bf4_t __attribute__((ext_vector_type(4)));
      bf4_t x = {(__bf16)in[4 * v], (__bf16)in[4 * v + 1], (__bf16)in[4 * v + 2], (__bf16)in[4 * v + 3]};
      *reinterpret_cast<bf4_t*>(row + tb + 4 * v) = x;
    }
  } else {
    for (int i = 0; i < N; ++i)
      if (tb + i < T) row[tb + i] = (__bf16)in[i];
  }
}

// Staged backward walk (T a multiple of the tile): the next tile's planes (gates, states,
// loss gradients) go straight from memory into LDS (global_load_lds_dwordx4) while the
// current tile is computed.  Thread t takes steps (PNR_BLOCK - 1 - t) N .. of its tile, so
// wave w's threads take one 1-KB run of each plane, run PNR_WAVES - 1 - w; the wave loads
// exactly that run (lane l writes bytes 16l..16l+15 of it) and reads back only what its
// own loads brought in, so its own vmcnt wait covers every read and no barrier is needed.
template <int CELL, int N>
struct BwdStage {
  static constexpr int PLANES = DiagCell<CELL>::G + 2 * DiagCell<CELL>::SP;
  float pl[PLANES][PNR_BLOCK * N];
};

template <int CELL, int N>
__device__ __forceinline__ void bwd_stage_issue(const BwdArgs& a, int row, int seg, BwdStage<CELL, N>& st) {
  using C = DiagCell<CELL>;
  constexpr int NG = C::G, K = C::SP, TILE = PNR_BLOCK * N;
  static_assert(N == 4, "one 16-byte load per lane and plane");
  const int tid = threadIdx.x, wid = tid >> 6, lane = tid & 63;
  const int D = a.D, T = a.T, S = K * D;
  const int b = row / D, d = row - b * D;
  const int r0 = (PNR_WAVES - 1 - wid) * 64 * N;   // the wave's run in each plane
  const size_t tb = (size_t)seg * TILE + r0 + lane * N;
#pragma unroll
  for (int gg = 0; gg < NG; ++gg) lds_load16(a.gx + ((size_t)(b * NG + gg) * D + d) * T + tb, &st.pl[gg][r0]);
#pragma unroll
  for (int k = 0; k < K; ++k) {
    const size_t off = ((size_t)b * S + (size_t)k * D + d) * T;
    lds_load16(a.hT + off + tb, &st.pl[NG + k][r0]);
    lds_load16(a.gT + off + tb, &st.pl[NG + K + k][r0]);
  }
}

// STAGED: the tile's inputs are read from `st` (this wave's own loads, landed), and the
// loads of the next tile (nrow, nseg) are issued once they are in registers.
template <int CELL, int N, bool BF16OUT, bool STAGED>
__device__ __forceinline__ typename DeltaOf<typename DiagCell<CELL>::E>::T adjoint_tile(
    const BwdArgs& a, BwdShared<CELL>& sh, int b, int d, int seg, float* acc, BwdStage<CELL, N>* st, int nrow,
    int nseg, bool more) {
  using C = DiagCell<CELL>;
  using E = typename C::E;
  using Dl = typename DeltaOf<E>::T;
  constexpr int K = C::SP, NG = C::G;
  constexpr int TILE = PNR_BLOCK * N;
  const int tid = threadIdx.x, wid = tid >> 6, lane = tid & 63;
  const int D = a.D, T = a.T, S = K * D;
  const bool vec = (T & 3) == 0;
  const int tb = seg * TILE + (PNR_BLOCK - 1 - tid) * N;
  const typename C::Par q = C::load_par(a.u, a.bh, D, d);
  size_t off[K];
#pragma unroll
  for (int k = 0; k < K; ++k) off[k] = ((size_t)b * S + k * D + d) * T;
  float gx[NG][N], hv[K][N], gv[K][N], p0[K];
  if constexpr (STAGED) {
    const int i0 = (PNR_BLOCK - 1 - tid) * N;
    auto rd = [&](const float* p, float* o) {
      const float4 x = *reinterpret_cast<const float4*>(p + i0);
      o[0] = x.x; o[1] = x.y; o[2] = x.z; o[3] = x.w;
    };
#pragma unroll
    for (int gg = 0; gg < NG; ++gg) rd(st->pl[gg], gx[gg]);
#pragma unroll
    for (int k = 0; k < K; ++k) {
      rd(st->pl[NG + k], hv[k]);
      rd(st->pl[NG + K + k], gv[k]);
    }
    // the reads have returned before the next tile's loads may overwrite the stage
    __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
    if (more) bwd_stage_issue<CELL, N>(a, nrow, nseg, *st);
  } else {
#pragma unroll
    for (int gg = 0; gg < NG; ++gg) load_n(a.gx + ((size_t)(b * NG + gg) * D + d) * T, tb, T, vec, N, gx[gg]);
#pragma unroll
    for (int k = 0; k < K; ++k) {
      load_n(a.hT + off[k], tb, T, vec, N, hv[k]);
      load_n(a.gT + off[k], tb, T, vec, N, gv[k]);
    }
  }
  // the state before this thread's first step is the last of the next lane's run (the
  // runs go backwards in time with the thread index); only the wave's last lane, whose
  // neighbour is in the next wave (or in the tile before), reads it from memory
#pragma unroll
  for (int k = 0; k < K; ++k) {
    const float nb = shfl_down_f(hv[k][N - 1], 1);
    p0[k] = lane != 63 ? nb
                       : (tb == 0 ? (a.h0 ? a.h0[(size_t)b * S + k * D + d] : 0.f)
                                  : (tb <= T ? a.hT[off[k] + tb - 1] : 0.f));
  }
  // scan elements mu -> J^T mu + J^T g, latest step first
  E e[N];
#pragma unroll
  for (int i = 0; i < N; ++i) {
    float gi[NG];
#pragma unroll
    for (int gg = 0; gg < NG; ++gg) gi[gg] = gx[gg][i];
    const bool in = tb + i < T;
    if constexpr (CELL == PNR_CELL_GRU_DIAG) {
      float res, ja = 0.f;
      C::eval(q, gi, i == 0 ? p0[0] : hv[0][i - 1], 0.f, PNR_JAC_FULL, true, res, ja);
      e[N - 1 - i] = in ? Aff1{ja, ja * gv[0][i]} : aff_identity1();
    } else {
      float rc, rh;
      Aff2 J = aff_identity2();
      C::eval(q, gi, i == 0 ? p0[0] : hv[0][i - 1], i == 0 ? p0[1] : hv[1][i - 1], 0.f, 0.f, PNR_JAC_FULL, true, rc,
              rh, J);
      const float g0 = gv[0][i], g1 = gv[1][i];
      if (a.jdiag) { J.a01 = 0.f; J.a10 = 0.f; }   // the diagonal approximation
      e[N - 1 - i] = in ? Aff2{J.a00, J.a10, J.a01, J.a11, fmaf(J.a00, g0, J.a10 * g1), fmaf(J.a01, g0, J.a11 * g1)}
                        : aff_identity2();
    }
  }
  E agg = e[0];
#pragma unroll
  for (int i = 1; i < N; ++i) agg = compose(e[i], agg);
  const E incl = wave_inclusive_scan(agg, identity_of<E>());
  if (lane == 63) sh.tot[wid] = incl;
  __syncthreads();
  Dl mw = sh.carry;   // mu at the step after this wave's runs
  for (int w = 0; w < wid; ++w) mw = apply(sh.tot[w], mw);
  Dl mu = wave_shr1(apply(incl, mw), mw);   // mu at the step after this thread's run
  float da[NG][N];
#pragma unroll
  for (int i = N - 1; i >= 0; --i) {
    float gi[NG], dg[NG], dh[NG];
#pragma unroll
    for (int gg = 0; gg < NG; ++gg) gi[gg] = gx[gg][i];
    const bool in = tb + i < T;
    if constexpr (CELL == PNR_CELL_GRU_DIAG) {
      const float p = i == 0 ? p0[0] : hv[0][i - 1];
      float dprev;
      vjp_gru(q, gi, p, gv[0][i] + mu, dg, dh, dprev);
#pragma unroll
      for (int gg = 0; gg < NG; ++gg) {
        dg[gg] = in ? dg[gg] : 0.f;
        dh[gg] = in ? dh[gg] : 0.f;
        acc[gg] = fmaf(dh[gg], p, acc[gg]);
        acc[NG + gg] += dh[gg];
        acc[2 * NG + gg] += dg[gg];
        da[gg][i] = dg[gg];
      }
      mu = in ? dprev : mu;
    } else {
      const float cp = i == 0 ? p0[0] : hv[0][i - 1];
      const float hp = i == 0 ? p0[1] : hv[1][i - 1];
      float2 dprev;
      vjp_lstm(q, gi, cp, hp, gv[0][i] + mu.x, gv[1][i] + mu.y, dg, dprev);
      if (a.jdiag) {
        // the diagonal approximation: mu_{t-1} = diag(J_t) lam_t, the step's own scan element
        const Aff2& el = e[N - 1 - i];
        dprev = make_float2(el.a00 * (gv[0][i] + mu.x), el.a11 * (gv[1][i] + mu.y));
      }
#pragma unroll
      for (int gg = 0; gg < NG; ++gg) {
        dg[gg] = in ? dg[gg] : 0.f;
        acc[gg] = fmaf(dg[gg], hp, acc[gg]);
        acc[NG + gg] += dg[gg];
        acc[2 * NG + gg] += dg[gg];
        da[gg][i] = dg[gg];
      }
      mu = in ? dprev : mu;
    }
  }
#pragma unroll
  for (int gg = 0; gg < NG; ++gg) {
    const size_t o = (((size_t)gg * D + d) * a.B + b) * T;
    if constexpr (BF16OUT) store_n_bf16(static_cast<__bf16*>(a.dgx) + o, tb, T, vec, N, da[gg]);
    else store_n(static_cast<float*>(a.dgx) + o, tb, T, vec, N, da[gg]);
  }
  __syncthreads();   // everyone has read tot and carry
  if (tid == PNR_BLOCK - 1) sh.carry = mu;   // mu at the tile's first step
  __syncthreads();
  return mu;
}

template <int CELL, int N, bool BF16OUT, bool STAGED>
__global__ void __launch_bounds__(PNR_BLOCK) adjoint_diag_kernel(BwdArgs a) {
  using C = DiagCell<CELL>;
  using Dl = typename DeltaOf<typename C::E>::T;
  constexpr int NA = 3 * C::G;
  __shared__ BwdShared<CELL> sh;
  // one staged tile (a one-float token when unstaged)
  __shared__ __align__(16) float stg_raw[STAGED ? BwdStage<CELL, N>::PLANES * PNR_BLOCK * N : 1];
  BwdStage<CELL, N>* stg = reinterpret_cast<BwdStage<CELL, N>*>(stg_raw);
  const int tid = threadIdx.x, wid = tid >> 6, lane = tid & 63;
  const int tpr = a.tiles_per_row;
  if (STAGED && (int)blockIdx.x < a.n_rows) bwd_stage_issue<CELL, N>(a, blockIdx.x, tpr - 1, *stg);
  for (int row = blockIdx.x; row < a.n_rows; row += gridDim.x) {
    const int b = row / a.D, d = row - b * a.D;
    float acc[NA];
#pragma unroll
    for (int j = 0; j < NA; ++j) acc[j] = 0.f;
    if (tid == 0) sh.carry = DeltaOf<typename C::E>::zero();
    __syncthreads();
    Dl mu = DeltaOf<typename C::E>::zero();
    for (int seg = tpr - 1; seg >= 0; --seg) {
      const int nrow = seg > 0 ? row : row + (int)gridDim.x, nseg = seg > 0 ? seg - 1 : tpr - 1;
      if (STAGED) __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): this wave's staged loads have landed
      mu = adjoint_tile<CELL, N, BF16OUT, STAGED>(a, sh, b, d, seg, acc, stg, nrow, nseg, nrow < a.n_rows);
    }
    if (tid == PNR_BLOCK - 1 && a.dh0) {   // this thread's run starts at step 0: mu = dL/dh0
      const int S = C::SP * a.D;
      if constexpr (CELL == PNR_CELL_GRU_DIAG) {
        a.dh0[(size_t)b * S + d] = mu;
      } else {
        a.dh0[(size_t)b * S + d] = mu.x;
        a.dh0[(size_t)b * S + a.D + d] = mu.y;
      }
    }
#pragma unroll
    for (int j = 0; j < NA; ++j) {
      const float v = wave_sum_f(acc[j]);
      if (lane == 0) sh.red[wid][j] = v;
    }
    __syncthreads();
    if (tid < NA) {
      float s = 0.f;
      for (int w = 0; w < PNR_WAVES; ++w) s += sh.red[w][tid];
      a.part[((size_t)b * NA + tid) * a.D + d] = s;   // [B][3][G][D]
    }
    __syncthreads();
  }
  if (STAGED) __builtin_amdgcn_s_waitcnt(0x0F70);   // no staged load outlives the block
}

constexpr int kAdjN = 4;   // steps per thread

int adjoint_items_per_thread() { return kAdjN; }

hipError_t launch_adjoint_diag(int cell, const BwdArgs& a, int num_cu, hipStream_t st) {
  // the staged walk loads whole tiles, so T must be a multiple of the tile; it pays for the
  // LSTM (4.79 -> 4.57 ms on the 131072-step backward pass) but not for the GRU, whose
  // lighter tiles run at higher occupancy unstaged (0.344 ms against 0.373)
  const bool staged = cell == PNR_CELL_LSTM_DIAG && a.T % (PNR_BLOCK * kAdjN) == 0;
  const void* fn =
      cell == PNR_CELL_GRU_DIAG
          ? (a.dgx_bf16 ? (const void*)adjoint_diag_kernel<PNR_CELL_GRU_DIAG, kAdjN, true, false>
                        : (const void*)adjoint_diag_kernel<PNR_CELL_GRU_DIAG, kAdjN, false, false>)
          : (a.dgx_bf16 ? (staged ? (const void*)adjoint_diag_kernel<PNR_CELL_LSTM_DIAG, kAdjN, true, true>
                                  : (const void*)adjoint_diag_kernel<PNR_CELL_LSTM_DIAG, kAdjN, true, false>)
                        : (staged ? (const void*)adjoint_diag_kernel<PNR_CELL_LSTM_DIAG, kAdjN, false, true>
                                  : (const void*)adjoint_diag_kernel<PNR_CELL_LSTM_DIAG, kAdjN, false, false>));
  const int per_cu = cached_occupancy(fn, 0);
  if (per_cu < 1) return hipErrorInvalidConfiguration;
  long g = (long)per_cu * num_cu;
  if (g > a.n_rows) g = a.n_rows;
  if (g < 1) g = 1;
  void* args[] = {const_cast<BwdArgs*>(&a)};
  return hipLaunchKernel(fn, dim3((unsigned)g), dim3(PNR_BLOCK), args, 0, st);
}

}  // namespace pnr
