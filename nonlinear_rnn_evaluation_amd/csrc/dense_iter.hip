// The Newton loop for the GRU with a dense recurrent matrix U (D <= 64), one fused pass
// per iteration: recurrent product U s_{t-1} for every step of a tile, gates, residual,
// Jacobian factors, the linear solve d_t = J_t d_{t-1} + r_t (scan of affine maps with
// a decoupled look-back across tiles) and the update s <- s + d.  All iterations run
// inside one persistent, co-resident grid; the residual max is finished by the last
// block to reach the grid barrier.
//
// Method: ParaRNN overview page, "Technical Implementation / Newton's Iteration" and
// "Parallel Reduction"; DEER's dense Jacobian and quasi-DEER's diagonal one from
// "Towards Scalable and Stable Parallelization of Nonlinear RNNs" (abstract).
//
// The dense Jacobian of the linear-before-reset GRU factors as
//   J_t = diag(z) + diag(al) U_z + diag(be) U_r + diag(ga) U_n
//   al = (s - n) z (1 - z),  be = (1 - z)(1 - n^2) gh_n r (1 - r),  ga = (1 - z)(1 - n^2) r
// so it is never formed: the scan applies it with three products by the blocks of U
// (resident in LDS) and an elementwise combination.  Only four D-vectors per step live
// in LDS.
//
// Layout: gx [B][T][3D], states [B][T][D] (channel-contiguous).  A tile is L steps of
// one batch element; blocks take tiles from a ticket counter.
//
// Scan organisation inside a tile:
//  * DIAG: thread (p, i) = part p of the tile, channel i; each part is a run of
//    consecutive steps composed serially; parts are combined in LDS.
//  * FULL: a group of D+1 lanes (inside one wave) owns one part.  Lane j < D carries
//    column j of the part's matrix product, lane D carries the vector part.  The block
//    total and the per-part prefixes are composed serially.
// Across tiles: the tile publishes its aggregate, reads the slots of up to WMAX
// predecessors in one cooperative round trip, and resolves its incoming increment
// from the nearest published prefix by applying the aggregates in between to it
// (matrix-vector products only).
#include "common.h"
#include "kernels.h"

namespace pnr {

template <typename Tt> struct WordsOf { static constexpr int W = sizeof(Tt) / 4; };

// look-back slot values per tile: FULL holds the (D*D + D)-value aggregate then the
// D-value prefix; DIAG holds D values of a, D of b, then D prefixes.
__host__ __device__ inline int dense_slot_values(int D, bool full) { return full ? D * D + 2 * D : 3 * D; }
// dense-Jacobian scan: parts (one lane group of D+1 lanes each) per tile; few enough
// that the serial composition of the part aggregates stays short
__host__ __device__ inline int dense_full_parts(int D) {
  const int groups = (64 / (D + 1)) * PNR_WAVES;
  return groups < 8 ? groups : 8;
}
__host__ __device__ inline int dense_agg_values(int D, bool full) { return full ? D * D + D : 2 * D; }
// predecessors inspected per look-back round trip (bounded by the LDS it takes)
constexpr int kWinPerThread = 16;
constexpr int kBatch = 8;   // loads issued together before any is used
__host__ __device__ inline int dense_window(int D, bool full, int) {
  int w = (PNR_BLOCK * kWinPerThread) / dense_slot_values(D, full);
  return w < 1 ? 1 : (w > 16 ? 16 : w);
}
// staged state values per thread: (L+1)*D <= PNR_BLOCK * kStagePerThread
constexpr int kStagePerThread = 17;

__device__ __forceinline__ void vput(uint64_t* s, uint32_t ep, float v) { slot_put(s, ep, v); }
__device__ __forceinline__ bool vget(const uint64_t* s, uint32_t ep, float& v) { return slot_get(s, ep, v); }
__device__ __forceinline__ void vput(uint64_t* s, uint32_t ep, double v) {
  uint64_t b = (uint64_t)__double_as_longlong(v);
  slot_put(s, ep, __uint_as_float((uint32_t)b));
  slot_put(s + 1, ep, __uint_as_float((uint32_t)(b >> 32)));
}
__device__ __forceinline__ bool vget(const uint64_t* s, uint32_t ep, double& v) {
  float lo, hi;
  bool ok = slot_get(s, ep, lo);
  ok &= slot_get(s + 1, ep, hi);
  uint64_t b = (uint64_t)__float_as_uint(lo) | ((uint64_t)__float_as_uint(hi) << 32);
  v = __longlong_as_double((long long)b);
  return ok;
}

__device__ __forceinline__ uint64_t abs_bits64(float r) { return (uint64_t)abs_bits(r); }
__device__ __forceinline__ uint64_t abs_bits64(double r) { return abs_bits(r); }
template <typename Tt> __device__ __forceinline__ double rho_of(uint64_t b);
template <> __device__ __forceinline__ double rho_of<float>(uint64_t b) { return bits_to_rho((uint32_t)b); }
template <> __device__ __forceinline__ double rho_of<double>(uint64_t b) { return bits_to_rho64(b); }

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
  for (int o = 32; o >= 1; o >>= 1) {
    uint64_t w = __shfl_xor(v, o);
    v = v > w ? v : w;
  }
  return v;
}

__device__ __forceinline__ float mul_add(float a, float b, float c) { return fmaf(a, b, c); }
__device__ __forceinline__ double mul_add(double a, double b, double c) { return fma(a, b, c); }

// ---------------------------------------------------------------------------------
// LDS layout (dynamic shared memory), in units of Tt:
//   Us   [D][3D]     recurrent matrix, transposed (absent when the cell runs on MFMA
//                    and the scan is diagonal: U then lives in registers)
//   Bh   [3D]        recurrent bias
//   Hx   [L+1][LD]   Hx[0] = s_{t0-1}, Hx[1+s] = current iterate at step t0+s; rows
//                    padded to LD = D+4 on the MFMA path (conflict-free operand reads)
//   Hj   [L+1][LD]   same for the state the Jacobian is taken at (Jacobian reuse only)
//   R    [L][D]      residuals
//   Jd   [L][D]      diagonal Jacobian (DIAG)  |  Z, Al, Be, Ga [L][D] factors (FULL)
//   Pagg             per-part aggregates: DIAG [2][parts][D]; FULL [parts][D*D + D]
//   Tot  [D*D + D]   FULL: block total
//   Pin  [parts+1][D] FULL: increment entering each part
//   Fx   [2][parts][D] FULL: fix-up double buffer (also look-back scratch)
//   Win  [WMAX][slot values]  look-back window
//   Din  [D]         increment entering the tile
//   UsJ  [D][3D]     FULL with a low-rank Jacobian: its matrix factors, transposed (the
//                    Jacobian products read these, the gates still read Us)
struct DenseLds {
  int D, L, full, reuse, parts, wmax, ld, has_u, has_uj;
  __host__ __device__ size_t count() const {
    size_t n = (has_u ? (size_t)3 * D * D : 0) + 3 * D + (size_t)(L + 1) * ld * (reuse ? 2 : 1) + (size_t)L * D;
    if (full) {
      n += (size_t)4 * L * D + (size_t)parts * (D * D + D) + (D * D + D) + (size_t)(parts + 1) * D +
           (size_t)2 * parts * D;
    } else {
      n += (size_t)L * D + (size_t)2 * parts * D;
    }
    n += (size_t)wmax * dense_slot_values(D, full) + D;
    if (has_uj) n += (size_t)3 * D * D;   // the Jacobian's own matrix (low-rank), transposed
    return n;
  }
};

// Ut is U transposed, [D][3D] (Ut[k][g*D + i] = U[g*D + i][k]): lanes that compute
// consecutive channels i read consecutive LDS words, so the product is bank-conflict
// free; the state row p is a broadcast.
template <typename Tt>
__device__ __forceinline__ void gru_gates(const Tt* __restrict__ Ut, const Tt* __restrict__ Bh,
                                          const Tt* __restrict__ p, const Tt* __restrict__ g, int D,
                                          int i, Tt& r, Tt& z, Tt& n, Tt& ghn) {
  Tt ar = Bh[i], az = Bh[D + i], an = Bh[2 * D + i];
  const int G3 = 3 * D;
  for (int k = 0; k < D; ++k) {
    const Tt pk = p[k];
    const Tt* u = Ut + (size_t)k * G3;
    ar = mul_add(u[i], pk, ar);
    az = mul_add(u[D + i], pk, az);
    an = mul_add(u[2 * D + i], pk, an);
  }
  r = sigm(g[i] + ar);
  z = sigm(g[D + i] + az);
  ghn = an;
  n = tanh_(mul_add(r, an, g[2 * D + i]));
}

__device__ __forceinline__ int pick_next_dense(int cur, int jac, int nbuf) {
  for (int i = 0; i < nbuf; ++i)
    if (i != cur && i != jac) return i;
  return -1;
}

typedef float f4mf_t __attribute__((ext_vector_type(4)));

// Gate pre-activations from the recurrent product on MFMA (fp32, D in {16, 32, 64}):
// Gh[t][g*D + c] = sum_k Hp[t][k] U[g*D + c][k] for one 16-step x 16-channel block, as
// D/4 chained v_mfma_f32_16x16x4_f32 per gate.  A = Hp rows from LDS (lane l: step l%16,
// k = 4kk + l/16); B = U fragments held in registers for the whole kernel (lane l:
// channel l%16, k = 4kk + l/16).  Result: lane l holds steps 4(l/16)+i, channel l%16.
template <int DM>
__device__ __forceinline__ void mfma_gates(const float* __restrict__ Hrows, int LD, int tb,
                                           const float (&uf)[3][DM / 4], f4mf_t (&acc)[3]) {
  const int l = (int)lane_id();
  const float* arow = Hrows + (size_t)(tb * 16 + (l & 15)) * LD + (l >> 4);
#pragma unroll
  for (int g = 0; g < 3; ++g) acc[g] = f4mf_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int kk = 0; kk < DM / 4; ++kk) {
    const float av = arow[4 * kk];
#pragma unroll
    for (int g = 0; g < 3; ++g) acc[g] = __builtin_amdgcn_mfma_f32_16x16x4f32(av, uf[g][kk], acc[g], 0, 0, 0);
  }
}

template <typename Tt, int DM, bool FULL, bool MF>
__global__ void __launch_bounds__(PNR_BLOCK) dense_newton_kernel(DenseLoopArgs<Tt> a) {
  extern __shared__ __align__(16) unsigned char lds_raw[];
  Tt* lds = reinterpret_cast<Tt*>(lds_raw);
  __shared__ int s_p;
  __shared__ int s_ok[16][2];
  __shared__ uint64_t s_wmax[PNR_WAVES];

  Ctrl* ctrl = a.ctrl;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int D = a.D, T = a.T, L = a.L;
  const bool reuse = a.nbuf > 2;
  const int GS = D + 1;                       // FULL: lanes per group
  const int GPW = FULL ? 64 / GS : 0;         // FULL: groups per wave
  const int parts = FULL ? dense_full_parts(D) : PNR_BLOCK / D;
  constexpr int W = WordsOf<Tt>::W;
  const int SV = dense_slot_values(D, FULL), SA = dense_agg_values(D, FULL);
  const int WMAX = dense_window(D, FULL, (int)sizeof(Tt));
  const int DD = D * D + D;
  constexpr bool HAS_U = !MF || FULL;
  const int LD = MF ? D + 4 : D;

  // carve LDS
  Tt* Us = lds;
  Tt* Bh = Us + (HAS_U ? 3 * D * D : 0);
  Tt* Hx = Bh + 3 * D;
  Tt* Hj = Hx + (L + 1) * LD;
  Tt* R = Hj + (reuse ? (L + 1) * LD : 0);
  Tt* Jd = R + L * D;            // DIAG
  Tt* Zv = R + L * D;            // FULL factors
  Tt* Al = Zv + L * D;
  Tt* Be = Al + L * D;
  Tt* Ga = Be + L * D;
  Tt* Pagg = FULL ? Ga + L * D : Jd + L * D;
  Tt* Tot = Pagg + (FULL ? parts * DD : 2 * parts * D);
  Tt* Pin = Tot + (FULL ? DD : 0);
  Tt* Fx = Pin + (FULL ? (parts + 1) * D : 0);
  Tt* Win = Fx + (FULL ? 2 * parts * D : 0);
  Tt* Din = Win + WMAX * SV;
  const bool own_uj = FULL && a.Uj != nullptr;
  Tt* UsJ = own_uj ? Din + D : Us;

  if constexpr (HAS_U) {
    for (int idx = tid; idx < 3 * D * D; idx += PNR_BLOCK) {
      const int row = idx / D, k = idx - row * D;     // U[row][k] -> Ut[k][row]
      Us[(size_t)k * 3 * D + row] = a.U[idx];
      if (own_uj) UsJ[(size_t)k * 3 * D + row] = a.Uj[idx];
    }
  }
  for (int idx = tid; idx < 3 * D; idx += PNR_BLOCK) Bh[idx] = a.bh ? a.bh[idx] : Tt(0);
  // MFMA path: this wave's U fragments and diagonal entries, in registers for the kernel
  constexpr int KF = MF ? DM / 4 : 1;
  float uf[3][KF];
  float udg[3] = {0.f, 0.f, 0.f};
  const int mf_cb = MF ? wid % (DM / 16) : 0;             // channel block of this wave
  const int mf_tb0 = MF ? wid / (DM / 16) : 0;            // first step block of this wave
  const int mf_tbs = MF ? PNR_WAVES / (DM / 16) : 1;      // step-block stride
  if constexpr (MF) {
    const int c = mf_cb * 16 + (lane & 15);
#pragma unroll
    for (int g = 0; g < 3; ++g) {
#pragma unroll
      for (int kk = 0; kk < KF; ++kk) uf[g][kk] = (float)a.U[(size_t)(g * D + c) * D + 4 * kk + (lane >> 4)];
      udg[g] = (float)a.U[(size_t)(g * D + c) * D + c];
    }
  }
  __syncthreads();

  int cur = -1, jac = -1;
  for (int k = 0; k <= a.max_iters; ++k) {
    const bool resid_only = k == a.max_iters;
    if (!resid_only && k % a.jac_every == 0) jac = cur;
    const int next = resid_only ? cur : pick_next_dense(cur, jac, a.nbuf);
    const Tt* Hcur = cur >= 0 ? a.H[cur] : nullptr;
    const Tt* Hjac = jac >= 0 ? a.H[jac] : nullptr;
    Tt* Hnext = next >= 0 ? a.H[next] : nullptr;
    const bool stale = !resid_only && jac != cur;
    const uint32_t ep = (uint32_t)k + 1u;
    uint64_t blk_max = 0;

    // Static assignment in increasing item order per block (co-resident grid): the
    // lowest unfinished tile never waits, so every look-back ends.  Items go out
    // time-segment-major (segment s of every batch row before segment
    // s+1), so a tile's predecessor always has a smaller item index: it was handed out
    // earlier, and prefixes are usually published before a successor looks back.
    for (int item = blockIdx.x; item < a.n_tiles; item += gridDim.x) {
      if (has_fault(ctrl)) break;
      const int seg = item / a.B, b = item - seg * a.B;
      const int tile = b * a.tiles_per_row + seg;   // slot index: row-major
      const int t0 = seg * L;
      const int Lv = min(L, T - t0);
      const Tt* gxb = a.gx + (size_t)b * T * 3 * D;

      // ---- stage states: Hx[0] = s_{t0-1}; Hx[1+s] = iterate at t0+s ----
      // All of a thread's loads are issued before any is used, so they overlap.  Row
      // s = 0 is the last step of the previous tile, written by another block during
      // this kernel: it is read coherently; the other rows are this block's own.
      for (int j0 = 0; j0 < kStagePerThread; j0 += kBatch) {
        Tt hv[kBatch], jv[kBatch];
#pragma unroll
        for (int j = 0; j < kBatch; ++j) {
          const int idx = tid + (j0 + j) * PNR_BLOCK;
          hv[j] = Tt(0);
          jv[j] = Tt(0);
          if (idx < (L + 1) * D) {
            const int s = idx / D, c = idx - s * D;
            const int t = t0 + s - 1;
            const size_t gi = ((size_t)b * T + t) * D + c;
            if (t < 0) {
              hv[j] = a.h0 ? a.h0[(size_t)b * D + c] : Tt(0);
              jv[j] = hv[j];
            } else if (t < T) {
              if (Hcur) hv[j] = s == 0 ? coherent_load(Hcur + gi) : Hcur[gi];
              if (stale && Hjac) jv[j] = s == 0 ? coherent_load(Hjac + gi) : Hjac[gi];
            }
          }
        }
#pragma unroll
        for (int j = 0; j < kBatch; ++j) {
          const int idx = tid + (j0 + j) * PNR_BLOCK;
          if (idx < (L + 1) * D) {
            const int s = idx / D, c = idx - s * D;
            Hx[s * LD + c] = hv[j];
            if (stale) Hj[s * LD + c] = jv[j];
          }
        }
      }
      __syncthreads();

      // ---- cell: gates, residual, Jacobian (diagonal or factors) ----
      uint64_t tmax = 0;
      if constexpr (MF) {
        // recurrent product on MFMA; lane l then owns steps tb*16 + 4(l/16) + i of
        // channel c for its wave's blocks
        const int c = mf_cb * 16 + (lane & 15);
        const float bhr = Bh[c], bhz = Bh[D + c], bhn = Bh[2 * D + c];
        for (int tb = mf_tb0; tb < L / 16; tb += mf_tbs) {
          // input pre-activations of this lane's 4 steps, loaded before the MFMAs
          float gxv[4][3];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int s = tb * 16 + 4 * (lane >> 4) + i;
            const Tt* g = gxb + (size_t)(t0 + s) * 3 * D;
#pragma unroll
            for (int q = 0; q < 3; ++q) gxv[i][q] = s < Lv ? g[q * D + c] : 0.f;
          }
          f4mf_t acc[3], accj[3];
          mfma_gates<DM>(Hx, LD, tb, uf, acc);
          if (stale) mfma_gates<DM>(Hj, LD, tb, uf, accj);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int s = tb * 16 + 4 * (lane >> 4) + i;
            const int idx = s * D + c;
            if (s >= Lv) {
              R[idx] = Tt(0);
              if (!resid_only) {
                if (FULL) { Zv[idx] = Tt(1); Al[idx] = Tt(0); Be[idx] = Tt(0); Ga[idx] = Tt(0); }
                else Jd[idx] = Tt(1);
              }
              continue;
            }
            const float p = Hx[s * LD + c];
            float r = sigm(gxv[i][0] + acc[0][i] + bhr);
            float z = sigm(gxv[i][1] + acc[1][i] + bhz);
            float ghn = acc[2][i] + bhn;
            float n = tanh_(fmaf(r, ghn, gxv[i][2]));
            const float res = fmaf(z, p - n, n) - Hx[(s + 1) * LD + c];
            R[idx] = res;
            tmax = max(tmax, abs_bits64(res));
            if (resid_only) continue;
            float pj = p;
            if (stale) {
              pj = Hj[s * LD + c];
              r = sigm(gxv[i][0] + accj[0][i] + bhr);
              z = sigm(gxv[i][1] + accj[1][i] + bhz);
              ghn = accj[2][i] + bhn;
              n = tanh_(fmaf(r, ghn, gxv[i][2]));
            }
            const float omz = 1.f - z;
            const float cn = omz * (1.f - n * n);
            const float al = (pj - n) * z * omz;
            const float be = cn * ghn * r * (1.f - r);
            const float ga = cn * r;
            if (a.jac_mode == PNR_JAC_ZERO) {
              if (FULL) { Zv[idx] = Tt(0); Al[idx] = Tt(0); Be[idx] = Tt(0); Ga[idx] = Tt(0); }
              else Jd[idx] = Tt(0);
            } else if (FULL) {
              Zv[idx] = z; Al[idx] = al; Be[idx] = be; Ga[idx] = ga;
            } else {
              Jd[idx] = z + al * udg[1] + be * udg[0] + ga * udg[2];
            }
          }
        }
      } else {
      for (int idx = tid; idx < L * D; idx += PNR_BLOCK) {
        const int s = idx / D, i = idx - s * D;
        if (s >= Lv) {
          R[idx] = Tt(0);
          if (!resid_only) {
            if (FULL) { Zv[idx] = Tt(1); Al[idx] = Tt(0); Be[idx] = Tt(0); Ga[idx] = Tt(0); }
            else Jd[idx] = Tt(1);
          }
          continue;
        }
        const Tt* g = gxb + (size_t)(t0 + s) * 3 * D;
        const Tt* p = Hx + s * LD;
        Tt r, z, n, ghn;
        gru_gates(Us, Bh, p, g, D, i, r, z, n, ghn);
        const Tt f = mul_add(z, p[i] - n, n);
        const Tt res = f - Hx[(s + 1) * LD + i];
        R[idx] = res;
        tmax = max(tmax, abs_bits64(res));
        if (resid_only) continue;
        const Tt* pj = p;
        if (stale) {
          pj = Hj + s * LD;
          gru_gates(Us, Bh, pj, g, D, i, r, z, n, ghn);
        }
        const Tt omz = Tt(1) - z;
        const Tt cn = omz * (Tt(1) - n * n);
        const Tt al = (pj[i] - n) * z * omz;
        const Tt be = cn * ghn * r * (Tt(1) - r);
        const Tt ga = cn * r;
        if (a.jac_mode == PNR_JAC_ZERO) {
          if (FULL) { Zv[idx] = Tt(0); Al[idx] = Tt(0); Be[idx] = Tt(0); Ga[idx] = Tt(0); }
          else Jd[idx] = Tt(0);
        } else if (FULL) {
          Zv[idx] = z; Al[idx] = al; Be[idx] = be; Ga[idx] = ga;
        } else {
          const Tt* ud = Us + (size_t)i * 3 * D;   // U[g*D + i][i] = Ut[i][g*D + i]
          Jd[idx] = z + al * ud[D + i] + be * ud[i] + ga * ud[2 * D + i];
        }
      }
      }
      blk_max = max(blk_max, tmax);
      __syncthreads();
      if (resid_only) continue;

      uint64_t* myslot = a.slots + (size_t)tile * SV * W;
      const int p = tid / D, ci = tid - p * D;                    // DIAG thread layout
      const int lpd = (L + parts - 1) / parts;                    // DIAG steps per part
      const int gi = lane / GS, jl = lane - gi * GS;              // FULL group layout
      const int part = wid * GPW + gi;
      const bool in_group = FULL && gi < GPW && part < parts;
      const int lpf = (L + parts - 1) / parts;
      Tt keep_a = Tt(1), keep_b = Tt(0);   // DIAG: this tile's total (a, b) for channel tid

      // ---- (1) part aggregates and (2) the block total, published for the successors ----
      if constexpr (!FULL) {
        Tt* Sa = Pagg;
        Tt* Sb = Pagg + parts * D;
        if (p < parts) {
          Tt ea = Tt(1), eb = Tt(0);
          for (int s = p * lpd; s < min(L, (p + 1) * lpd); ++s) {
            const Tt ja = Jd[s * D + ci];
            eb = mul_add(ja, eb, R[s * D + ci]);
            ea = ja * ea;
          }
          Sa[p * D + ci] = ea;
          Sb[p * D + ci] = eb;
        }
        __syncthreads();
        if (tid < D) {
          Tt ta = Sa[tid], tb = Sb[tid];
          for (int q = 1; q < parts; ++q) {
            const Tt qa = Sa[q * D + tid], qb = Sb[q * D + tid];
            tb = mul_add(qa, tb, qb);
            ta = qa * ta;
          }
          keep_a = ta;
          keep_b = tb;
          if (seg == 0) {
            vput(myslot + (size_t)(2 * D + tid) * W, ep, tb);
            Din[tid] = Tt(0);
          } else {
            vput(myslot + (size_t)tid * W, ep, ta);
            vput(myslot + (size_t)(D + tid) * W, ep, tb);
          }
        }
      } else {
        if (in_group) {
          Tt col[DM];
#pragma unroll
          for (int m = 0; m < DM; ++m) col[m] = (jl < D && m == jl) ? Tt(1) : Tt(0);
          for (int s = part * lpf; s < min(L, (part + 1) * lpf); ++s) {
            const Tt* zr = Zv + s * D; const Tt* ar = Al + s * D;
            const Tt* br = Be + s * D; const Tt* gr = Ga + s * D;
            Tt nw[DM];
#pragma unroll
            for (int m = 0; m < DM; ++m) {
              Tt ur = 0, uz = 0, un = 0;
              if (m < D) {
#pragma unroll
                for (int kk = 0; kk < DM; ++kk) {
                  if (kk < D) {
                    const Tt* u = UsJ + (size_t)kk * 3 * D;
                    ur = mul_add(u[m], col[kk], ur);
                    uz = mul_add(u[D + m], col[kk], uz);
                    un = mul_add(u[2 * D + m], col[kk], un);
                  }
                }
              }
              Tt v = m < D ? zr[m] * col[m] + ar[m] * uz + br[m] * ur + gr[m] * un : Tt(0);
              if (jl == D && m < D) v += R[s * D + m];
              nw[m] = v;
            }
#pragma unroll
            for (int m = 0; m < DM; ++m) col[m] = nw[m];
          }
          Tt* ag = Pagg + (size_t)part * DD;     // [D][D] row-major, then [D]
#pragma unroll
          for (int m = 0; m < DM; ++m) {
            if (m < D) {
              if (jl < D) ag[m * D + jl] = col[m];
              else ag[D * D + m] = col[m];
            }
          }
        }
        __syncthreads();
        if (tid < GS) {
          Tt col[DM];
#pragma unroll
          for (int m = 0; m < DM; ++m) col[m] = m < D ? (tid < D ? Pagg[m * D + tid] : Pagg[D * D + m]) : Tt(0);
          for (int q = 1; q < parts; ++q) {
            const Tt* ag = Pagg + (size_t)q * DD;
            Tt nw[DM];
#pragma unroll
            for (int m = 0; m < DM; ++m) {
              Tt v = (tid == D && m < D) ? ag[D * D + m] : Tt(0);
              if (m < D) {
#pragma unroll
                for (int kk = 0; kk < DM; ++kk)
                  if (kk < D) v = mul_add(ag[m * D + kk], col[kk], v);
              }
              nw[m] = v;
            }
#pragma unroll
            for (int m = 0; m < DM; ++m) col[m] = nw[m];
          }
#pragma unroll
          for (int m = 0; m < DM; ++m) {
            if (m < D) {
              if (tid < D) Tot[m * D + tid] = col[m];
              else Tot[D * D + m] = col[m];
            }
          }
        }
        __syncthreads();
        if (seg == 0) {
          for (int m = tid; m < D; m += PNR_BLOCK) {
            Din[m] = Tt(0);
            vput(myslot + (size_t)(SA + m) * W, ep, Tot[D * D + m]);
          }
        } else {
          for (int e = tid; e < SA; e += PNR_BLOCK) vput(myslot + (size_t)e * W, ep, Tot[e]);
        }
      }
      __syncthreads();

      // ---- (3) decoupled look-back over a window of predecessors (block-uniform loop) ----
      if (seg > 0) {
        uint32_t spins = 0;
        while (true) {
          const int Wn = min(seg, WMAX);
          if (tid < Wn) { s_ok[tid][0] = 1; s_ok[tid][1] = 1; }
          __syncthreads();
          for (int j0 = 0; j0 < kWinPerThread; j0 += kBatch) {
            // issue a batch of slot reads, then consume them
            Tt wv[kBatch];
            bool wok[kBatch];
#pragma unroll
            for (int j = 0; j < kBatch; ++j) {
              const int idx = tid + (j0 + j) * PNR_BLOCK;
              wok[j] = true;
              wv[j] = Tt(0);
              if (idx < Wn * SV) {
                const int w = idx / SV, e = idx - w * SV;
                wok[j] = vget(a.slots + ((size_t)(tile - 1 - w) * SV + e) * W, ep, wv[j]);
              }
            }
#pragma unroll
            for (int j = 0; j < kBatch; ++j) {
              const int idx = tid + (j0 + j) * PNR_BLOCK;
              if (idx < Wn * SV) {
                const int w = idx / SV, e = idx - w * SV;
                if (!wok[j]) s_ok[w][e < SA ? 0 : 1] = 0;
                Win[w * SV + e] = wv[j];
              }
            }
          }
          __syncthreads();
          if (tid == 0) {
            int pp = -1;
            for (int w = 0; w < Wn; ++w) {
              if (s_ok[w][1]) { pp = w; break; }
              if (!s_ok[w][0]) break;
            }
            s_p = pp;
          }
          __syncthreads();
          const int pp = s_p;
          if (pp >= 0) {
            if constexpr (!FULL) {
              if (tid < D) {
                Tt dl = Win[pp * SV + 2 * D + tid];
                for (int w = pp - 1; w >= 0; --w) dl = mul_add(Win[w * SV + tid], dl, Win[w * SV + D + tid]);
                Din[tid] = dl;
              }
            } else {
              // d <- M_w d + v_w for w = pp-1 .. 0, starting from the prefix of tile pp
              Tt* vec = Fx;                 // scratch: two D-vectors
              if (tid < D) vec[tid] = Win[pp * SV + SA + tid];
              __syncthreads();
              int src = 0;
              for (int w = pp - 1; w >= 0; --w) {
                if (tid < D) {
                  const Tt* M = Win + w * SV;
                  Tt v = M[D * D + tid];
                  for (int kk = 0; kk < D; ++kk) v = mul_add(M[tid * D + kk], vec[src * D + kk], v);
                  vec[(1 - src) * D + tid] = v;
                }
                __syncthreads();
                src = 1 - src;
              }
              if (tid < D) Din[tid] = vec[src * D + tid];
            }
            __syncthreads();
            break;
          }
          if (++spins > kSpinLimit) {
            if (tid == 0) record_fault(ctrl, 1);
            for (int m = tid; m < D; m += PNR_BLOCK) Din[m] = Tt(0);
            __syncthreads();
            break;
          }
          backoff(spins);
        }
        // publish this tile's inclusive prefix
        if constexpr (!FULL) {
          if (tid < D) vput(myslot + (size_t)(2 * D + tid) * W, ep, mul_add(keep_a, Din[tid], keep_b));
        } else {
          for (int m = tid; m < D; m += PNR_BLOCK) {
            Tt v = Tot[D * D + m];
            for (int kk = 0; kk < D; ++kk) v = mul_add(Tot[m * D + kk], Din[kk], v);
            vput(myslot + (size_t)(SA + m) * W, ep, v);
          }
        }
      }
      __syncthreads();

      // ---- (4) fix-up: walk each part from its incoming increment, s <- s + d ----
      if constexpr (!FULL) {
        Tt* Sa = Pagg;
        Tt* Sb = Pagg + parts * D;
        if (p < parts) {
          Tt dl = Din[ci];
          for (int q = 0; q < p; ++q) dl = mul_add(Sa[q * D + ci], dl, Sb[q * D + ci]);
          for (int s = p * lpd; s < min(Lv, (p + 1) * lpd); ++s) {
            dl = mul_add(Jd[s * D + ci], dl, R[s * D + ci]);
            Tt* o = Hnext + ((size_t)b * T + t0 + s) * D + ci;
            // the tile's last row is the next tile's halo, read by another block next pass
            if (s == L - 1) coherent_store(o, Hx[(s + 1) * LD + ci] + dl);
            else *o = Hx[(s + 1) * LD + ci] + dl;
          }
        }
        __syncthreads();
      } else {
        for (int m = tid; m < D; m += PNR_BLOCK) Pin[m] = Din[m];
        __syncthreads();
        for (int q = 0; q < parts; ++q) {
          if (tid < D) {
            const Tt* ag = Pagg + (size_t)q * DD;
            Tt v = ag[D * D + tid];
            for (int kk = 0; kk < D; ++kk) v = mul_add(ag[tid * D + kk], Pin[q * D + kk], v);
            Pin[(q + 1) * D + tid] = v;
          }
          __syncthreads();
        }
        Tt* cb = Fx;
        Tt* nb = Fx + parts * D;
        if (in_group && jl < D) cb[part * D + jl] = Pin[part * D + jl];
        __syncthreads();
        for (int st = 0; st < lpf; ++st) {
          const int s = part * lpf + st;
          if (in_group && jl < D && s < L) {
            const Tt* dv = cb + part * D;
            Tt ur = 0, uz = 0, un = 0;
            for (int kk = 0; kk < D; ++kk) {
              const Tt* u = UsJ + (size_t)kk * 3 * D;
              ur = mul_add(u[jl], dv[kk], ur);
              uz = mul_add(u[D + jl], dv[kk], uz);
              un = mul_add(u[2 * D + jl], dv[kk], un);
            }
            const int qi = s * D + jl;
            const Tt v = Zv[qi] * dv[jl] + Al[qi] * uz + Be[qi] * ur + Ga[qi] * un + R[qi];
            nb[part * D + jl] = v;
            if (s < Lv) {
              Tt* o = Hnext + ((size_t)b * T + t0 + s) * D + jl;
              if (s == L - 1) coherent_store(o, Hx[(s + 1) * LD + jl] + v);   // next tile's halo
              else *o = Hx[(s + 1) * LD + jl] + v;
            }
          }
          __syncthreads();
          Tt* tmp = cb; cb = nb; nb = tmp;
        }
      }
    }

    // ---- two-level residual max: block partial -> global; the barrier's last block merges ----
    blk_max = wave_max_u64(blk_max);
    if (lane == 0) s_wmax[wid] = blk_max;
    __syncthreads();
    if (tid == 0) {
      uint64_t m = s_wmax[0];
      for (int w = 1; w < PNR_WAVES; ++w) m = max(m, s_wmax[w]);
      __hip_atomic_store(&a.partials[blockIdx.x], m, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    grid_barrier(ctrl, [&]() {
      uint64_t m = 0;
      for (int i = tid; i < (int)gridDim.x; i += PNR_BLOCK) {
        const uint64_t v = __hip_atomic_load(&a.partials[i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        m = max(m, v);
      }
      m = wave_max_u64(m);
      __syncthreads();
      if (lane == 0) s_wmax[wid] = m;
      __syncthreads();
      if (tid == 0) {
        for (int w = 0; w < PNR_WAVES; ++w) m = max(m, s_wmax[w]);
        finish_iteration(ctrl, a.rho_hist, rho_of<Tt>(m), k, cur, a.max_iters, a.tol);
      }
    });
    if (__hip_atomic_load(&ctrl->done, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) || has_fault(ctrl)) break;
    cur = next;
  }
}

// ---------------------------------------------------------------------------------
int dense_supported(int D, int full, int is_f64) {
  if (D < 1) return 0;
  if (full) return D <= 32;
  return is_f64 ? D <= 32 : D <= 64;
}

int dense_state_buffers(int D, int full, int is_f64, int reuse) {
  (void)D; (void)full; (void)is_f64;
  return reuse ? 3 : 2;   // the iterate being checked and the next (plus the reused one)
}

int dense_tile_len(int D, int full, int is_f64) {
  if (dense_mfma_supported(D, full, is_f64)) return dense_mfma_tile_len();
  return full ? dense_full_parts(D) * 8 : 64;
}

static int dense_parts(int D, int full) { return full ? dense_full_parts(D) : PNR_BLOCK / D; }

int dense_slot_words(int D, int full, int is_f64) {
  if (dense_mfma_supported(D, full, is_f64)) return dense_mfma_slot_words(D, full);
  return dense_slot_values(D, full) * (is_f64 ? 2 : 1);
}

size_t dense_lds_bytes(int D, int full, int is_f64, int reuse, int lowrank) {
  const int es = is_f64 ? 8 : 4;
  DenseLds l{D, full ? dense_full_parts(D) * 8 : 64, full, reuse, dense_parts(D, full),
             dense_window(D, full != 0, es), D, 1, full && lowrank};
  return l.count() * es;
}

template <typename Tt, int DM, bool FULL, bool MF>
static int dense_capacity_t(int num_cu, size_t lds) {
  const int v = cached_occupancy((const void*)dense_newton_kernel<Tt, DM, FULL, MF>, lds);
  long g = (long)v * num_cu;
  return (int)(g > kMaxGrid ? kMaxGrid : g);
}

template <typename Tt, int DM, bool FULL, bool MF>
static hipError_t launch_t(const DenseLoopArgs<Tt>& a, int num_cu, hipStream_t st) {
  const size_t lds = dense_lds_bytes(a.D, FULL, sizeof(Tt) == 8, a.nbuf > 2, a.Uj != nullptr);
  const int cap = dense_capacity_t<Tt, DM, FULL, MF>(num_cu, lds);
  if (cap < 1) return hipErrorInvalidConfiguration;
  int grid = a.n_tiles < cap ? a.n_tiles : cap;
  if (grid < 1) grid = 1;
  void* args[] = {const_cast<DenseLoopArgs<Tt>*>(&a)};
  return launch_persistent((const void*)dense_newton_kernel<Tt, DM, FULL, MF>, grid, lds, args, st);
}

template <typename Tt>
static hipError_t launch_dense_t(const DenseLoopArgs<Tt>& a, int full, int num_cu, hipStream_t st) {
  if (!full) return launch_t<Tt, 1, false, false>(a, num_cu, st);
  if (a.D <= 4) return launch_t<Tt, 4, true, false>(a, num_cu, st);
  if (a.D <= 8) return launch_t<Tt, 8, true, false>(a, num_cu, st);
  if (a.D <= 16) return launch_t<Tt, 16, true, false>(a, num_cu, st);
  return launch_t<Tt, 32, true, false>(a, num_cu, st);
}

hipError_t launch_dense_newton_f32(const DenseLoopArgs<float>& a, int full, int num_cu, hipStream_t st) {
  if (dense_mfma_supported(a.D, full, 0)) return launch_dense_mfma(a, full, num_cu, st);
  return launch_dense_t<float>(a, full, num_cu, st);
}
hipError_t launch_dense_newton_f64(const DenseLoopArgs<double>& a, int full, int num_cu, hipStream_t st) {
  return launch_dense_t<double>(a, full, num_cu, st);
}

}  // namespace pnr
