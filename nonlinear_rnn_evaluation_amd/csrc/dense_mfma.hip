// The Newton loop for the dense-U GRU on MFMA (fp32, D in {16, 32, 64}): one persistent,
// co-resident grid runs every iteration; a tile is 64 consecutive steps of one batch
// element, taken in a fixed order per block.
//
// Method: ParaRNN overview page, "Technical Implementation / Newton's Iteration" and
// "Parallel Reduction"; the dense Jacobian of DEER and the diagonal one of quasi-DEER
// from "Towards Scalable and Stable Parallelization of Nonlinear RNNs" (abstract).
//
// Per tile and iteration:
//  1. stage the states of the tile (and the step before it) in LDS;
//  2. recurrent product Gh = U s_{t-1} for all 64 steps on v_mfma_f32_16x16x4_f32, with
//     U's operand fragments held in registers for the whole kernel; gates, residual
//     r_t, and the Jacobian: its diagonal (quasi) or the four factor vectors of
//       J_t = diag(z) + diag(al) U_z + diag(be) U_r + diag(ga) U_n
//  3. the scan of the affine maps d -> J_t d + r_t inside the tile, its aggregate
//     published for the successors, the decoupled look-back for the increment
//     entering the tile, and the fix-up s <- s + d.
//
// Dense-Jacobian scan (D = 16) on MFMA.  The tile is cut into 8 parts of 8 steps; each
// wave runs two parts as independent chains.  A part's aggregate M = J_e ... J_b is built
// from the back, S <- S J_t, kept transposed: S^T <- J_t^T S^T is a left product whose
// accumulator layout (lane l: rows 4(l/16)+i of column l%16) is exactly the B-operand
// layout the next product needs when the k index of chunk i is taken as 4(l/16)+i, so
// no lane ever exchanges data; the vector part v = sum_t S r_t accumulates alongside in
// four FMAs per step.  The fix-up runs forward, d <- J_t d + r_t, with d carried as the
// first column of a 16x16 operand, so it is the same MFMA chain.  J_t is never stored:
// each lane forms the four entries it feeds to the MFMA from the factors and twelve
// entries of U held in registers.
#include "common.h"
#include "kernels.h"

namespace pnr {

typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int kTL = 64;            // steps per tile
constexpr int kFParts = 8;         // dense-Jacobian scan: parts per tile
constexpr int kFPartLen = kTL / kFParts;
constexpr int kLoadBatch = 8;

__device__ __forceinline__ v4f mfma4(float a, float b, v4f c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// Stage rows s = 0..kTL of the tile: row s holds the state before step t0+s.  Row 0 is
// the previous tile's last step (another block's): read coherently.  Batched loads.
__device__ __forceinline__ void stage_rows(float* __restrict__ X, const float* __restrict__ H,
                                           const float* __restrict__ h0, int b, int t0, int T, int D,
                                           int LD) {
  const int tid = threadIdx.x;
  const int n = (kTL + 1) * D;
  for (int j0 = 0; j0 < n; j0 += kLoadBatch * PNR_BLOCK) {
    float v[kLoadBatch];
#pragma unroll
    for (int j = 0; j < kLoadBatch; ++j) {
      const int idx = j0 + tid + j * PNR_BLOCK;
      v[j] = 0.f;
      if (idx < n) {
        const int s = idx / D, c = idx - s * D, t = t0 + s - 1;
        if (t < 0) v[j] = h0 ? h0[(size_t)b * D + c] : 0.f;
        else if (t < T && H) {
          const float* p = H + ((size_t)b * T + t) * D + c;
          v[j] = s == 0 ? coherent_load(p) : *p;
        }
      }
    }
#pragma unroll
    for (int j = 0; j < kLoadBatch; ++j) {
      const int idx = j0 + tid + j * PNR_BLOCK;
      if (idx < n) {
        const int s = idx / D, c = idx - s * D;
        X[s * LD + c] = v[j];
      }
    }
  }
}

// Gate pre-activations of one 16-step block: acc[g] lane l = Gh_g[step 4(l/16)+i][ch l%16].
template <int DM>
__device__ __forceinline__ void gates_block(const float* __restrict__ X, int LD, int tb,
                                            const float (&uf)[3][DM / 4], v4f (&acc)[3]) {
  const int l = (int)lane_id();
  const float* arow = X + (size_t)(tb * 16 + (l & 15)) * LD + (l >> 4);
#pragma unroll
  for (int g = 0; g < 3; ++g) acc[g] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int kk = 0; kk < DM / 4; ++kk) {
    const float av = arow[4 * kk];
#pragma unroll
    for (int g = 0; g < 3; ++g) acc[g] = mfma4(av, uf[g][kk], acc[g]);
  }
}

// Residual partial -> grid barrier; the last block merges the partials and decides.
__device__ __forceinline__ void end_pass(const DenseLoopArgs<float>& a, uint32_t blk_max, int k, int cur) {
  __shared__ uint32_t s_wmax[PNR_WAVES];
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  blk_max = wave_max_u32(blk_max);
  if (lane == 0) s_wmax[wid] = blk_max;
  __syncthreads();
  if (tid == 0) {
    uint32_t m = s_wmax[0];
    for (int w = 1; w < PNR_WAVES; ++w) m = max(m, s_wmax[w]);
    __hip_atomic_store(reinterpret_cast<uint32_t*>(a.partials) + blockIdx.x, m, __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
  }
  Ctrl* ctrl = a.ctrl;
  grid_barrier(ctrl, [&]() {
    uint32_t m = 0;
    for (int i = tid; i < (int)gridDim.x; i += PNR_BLOCK)
      m = max(m, __hip_atomic_load(reinterpret_cast<uint32_t*>(a.partials) + i, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT));
    m = wave_max_u32(m);
    __syncthreads();
    if (lane == 0) s_wmax[wid] = m;
    __syncthreads();
    if (tid == 0) {
      for (int w = 0; w < PNR_WAVES; ++w) m = max(m, s_wmax[w]);
      finish_iteration(ctrl, a.rho_hist, bits_to_rho(m), k, cur, a.max_iters, a.tol);
    }
  });
}

__device__ __forceinline__ int next_buffer(int cur, int jac, int nbuf) {
  for (int i = 0; i < nbuf; ++i)
    if (i != cur && i != jac) return i;
  return -1;
}

// Read up to Wn predecessor slots (SV values each, aggregate first) into Win and find
// the nearest predecessor with a published prefix whose successors (up to this tile)
// all published their aggregates.  Returns that window index, or -1.  Block-uniform.
__device__ __forceinline__ int window_read(const uint64_t* __restrict__ slots, int tile, int Wn, int SV, int SA,
                                           uint32_t ep, float* __restrict__ Win) {
  __shared__ int s_ok[16][2];
  __shared__ int s_p;
  const int tid = threadIdx.x;
  if (tid < Wn) { s_ok[tid][0] = 1; s_ok[tid][1] = 1; }
  __syncthreads();
  for (int j0 = 0; j0 < Wn * SV; j0 += kLoadBatch * PNR_BLOCK) {
    float v[kLoadBatch];
    bool ok[kLoadBatch];
#pragma unroll
    for (int j = 0; j < kLoadBatch; ++j) {
      const int idx = j0 + tid + j * PNR_BLOCK;
      ok[j] = true;
      v[j] = 0.f;
      if (idx < Wn * SV) {
        const int w = idx / SV, e = idx - w * SV;
        ok[j] = slot_get(slots + (size_t)(tile - 1 - w) * SV + e, ep, v[j]);
      }
    }
#pragma unroll
    for (int j = 0; j < kLoadBatch; ++j) {
      const int idx = j0 + tid + j * PNR_BLOCK;
      if (idx < Wn * SV) {
        const int w = idx / SV, e = idx - w * SV;
        if (!ok[j]) s_ok[w][e < SA ? 0 : 1] = 0;
        Win[w * SV + e] = v[j];
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
  return s_p;
}

// =====================================================================================
// Diagonal (quasi-Newton) Jacobian.  LDS: Bh[3D] | X[(kTL+1) LD] | Xj (reuse) | R[kTL D] |
// Jd[kTL D] | Sa,Sb[parts D] | Win[W * 3D] | Din[D].
__host__ __device__ inline int mfd_window(int D) {
  const int w = (PNR_BLOCK * 16) / (3 * D);
  return w > 16 ? 16 : w;
}
__host__ __device__ inline size_t mfd_lds_floats(int D, int reuse) {
  const int LD = D + 4, parts = PNR_BLOCK / D;
  return (size_t)3 * D + (size_t)(kTL + 1) * LD * (reuse ? 2 : 1) + (size_t)2 * kTL * D + (size_t)2 * parts * D +
         (size_t)mfd_window(D) * 3 * D + D;
}

template <int DM>
__global__ void __launch_bounds__(PNR_BLOCK) dense_diag_mfma_kernel(DenseLoopArgs<float> a) {
  extern __shared__ __align__(16) float lds[];
  Ctrl* ctrl = a.ctrl;
  constexpr int D = DM, LD = DM + 4, P = PNR_BLOCK / DM, LP = kTL / P, SV = 3 * DM, SA = 2 * DM;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int T = a.T;
  const bool reuse = a.nbuf > 2;
  const int WMAX = mfd_window(D);
  float* Bh = lds;
  float* X = Bh + 3 * D;
  float* Xj = X + (kTL + 1) * LD;
  float* R = Xj + (reuse ? (kTL + 1) * LD : 0);
  float* Jd = R + kTL * D;
  float* Sa = Jd + kTL * D;
  float* Sb = Sa + P * D;
  float* Win = Sb + P * D;
  float* Din = Win + WMAX * SV;

  for (int i = tid; i < 3 * D; i += PNR_BLOCK) Bh[i] = a.bh ? a.bh[i] : 0.f;
  // this wave's U fragments (recurrent product) and the diagonal of each gate block
  const int cb = wid % (D / 16), tb0 = wid / (D / 16), tbs = PNR_WAVES / (D / 16);
  const int c_mf = cb * 16 + (lane & 15);
  float uf[3][D / 4], udg[3];
#pragma unroll
  for (int g = 0; g < 3; ++g) {
#pragma unroll
    for (int kk = 0; kk < D / 4; ++kk) uf[g][kk] = a.U[(size_t)(g * D + c_mf) * D + 4 * kk + (lane >> 4)];
    udg[g] = a.U[(size_t)(g * D + c_mf) * D + c_mf];
  }
  __syncthreads();
  const float bhr = Bh[c_mf], bhz = Bh[D + c_mf], bhn = Bh[2 * D + c_mf];
  const int pp_ = tid / D, ci = tid - pp_ * D;   // scan layout: part, channel

  int cur = -1, jac = -1;
  for (int k = 0; k <= a.max_iters; ++k) {
    const bool resid_only = k == a.max_iters;
    if (!resid_only && k % a.jac_every == 0) jac = cur;
    const int next = resid_only ? cur : next_buffer(cur, jac, a.nbuf);
    const float* Hcur = cur >= 0 ? a.H[cur] : nullptr;
    const float* Hjac = jac >= 0 ? a.H[jac] : nullptr;
    float* Hnext = next >= 0 ? a.H[next] : nullptr;
    const bool stale = !resid_only && jac != cur;
    const uint32_t ep = (uint32_t)k + 1u;
    uint32_t blk_max = 0;
    // Items go out time-segment-major (segment s of every batch row before segment
    // s+1), so a tile's predecessor always has a smaller item index: it was handed out
    // earlier, and prefixes are usually published before a successor looks back.
    for (int item = blockIdx.x; item < a.n_tiles; item += gridDim.x) {
      if (has_fault(ctrl)) break;
      const int seg = item / a.B, b = item - seg * a.B;
      const int tile = b * a.tiles_per_row + seg;   // slot index: row-major
      const int t0 = seg * kTL, Lv = min(kTL, T - t0);
      const float* gxb = a.gx + (size_t)b * T * 3 * D;
      stage_rows(X, Hcur, a.h0, b, t0, T, D, LD);
      if (stale) stage_rows(Xj, Hjac, a.h0, b, t0, T, D, LD);
      __syncthreads();

      // ---- cell on MFMA: residual and diagonal Jacobian ----
      uint32_t tmax = 0;
      for (int tb = tb0; tb < kTL / 16; tb += tbs) {
        float gxv[4][3];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int s = tb * 16 + 4 * (lane >> 4) + i;
          const float* g = gxb + (size_t)(t0 + s) * 3 * D;
#pragma unroll
          for (int q = 0; q < 3; ++q) gxv[i][q] = s < Lv ? g[q * D + c_mf] : 0.f;
        }
        v4f acc[3], accj[3];
        gates_block<D>(X, LD, tb, uf, acc);
        if (stale) gates_block<D>(Xj, LD, tb, uf, accj);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int s = tb * 16 + 4 * (lane >> 4) + i;
          const int idx = s * D + c_mf;
          if (s >= Lv) {
            R[idx] = 0.f;
            Jd[idx] = 1.f;
            continue;
          }
          const float p = X[s * LD + c_mf];
          float r = sigm(gxv[i][0] + acc[0][i] + bhr);
          float z = sigm(gxv[i][1] + acc[1][i] + bhz);
          float ghn = acc[2][i] + bhn;
          float n = tanh_(fmaf(r, ghn, gxv[i][2]));
          const float res = fmaf(z, p - n, n) - X[(s + 1) * LD + c_mf];
          R[idx] = res;
          tmax = max(tmax, abs_bits(res));
          if (resid_only) continue;
          float pj = p;
          if (stale) {
            pj = Xj[s * LD + c_mf];
            r = sigm(gxv[i][0] + accj[0][i] + bhr);
            z = sigm(gxv[i][1] + accj[1][i] + bhz);
            ghn = accj[2][i] + bhn;
            n = tanh_(fmaf(r, ghn, gxv[i][2]));
          }
          const float omz = 1.f - z, cn = omz * (1.f - n * n);
          Jd[idx] = a.jac_mode == PNR_JAC_ZERO
                        ? 0.f
                        : z + (pj - n) * z * omz * udg[1] + cn * ghn * r * (1.f - r) * udg[0] + cn * r * udg[2];
        }
      }
      blk_max = max(blk_max, tmax);
      __syncthreads();
      if (resid_only) continue;

      // ---- scan inside the tile: part aggregates, tile total, publication ----
      float ea = 1.f, eb = 0.f;
      for (int s = pp_ * LP; s < (pp_ + 1) * LP; ++s) {
        const float ja = Jd[s * D + ci];
        eb = fmaf(ja, eb, R[s * D + ci]);
        ea *= ja;
      }
      Sa[pp_ * D + ci] = ea;
      Sb[pp_ * D + ci] = eb;
      __syncthreads();
      uint64_t* myslot = a.slots + (size_t)tile * SV;
      float ta = 1.f, tbv = 0.f;
      if (tid < D) {
        for (int q = 0; q < P; ++q) {
          tbv = fmaf(Sa[q * D + tid], tbv, Sb[q * D + tid]);
          ta *= Sa[q * D + tid];
        }
        if (seg == 0) {
          slot_put(myslot + 2 * D + tid, ep, tbv);
          Din[tid] = 0.f;
        } else {
          slot_put(myslot + tid, ep, ta);
          slot_put(myslot + D + tid, ep, tbv);
        }
      }
      // ---- decoupled look-back over a window of predecessors ----
      if (seg > 0) {
        uint32_t spins = 0;
        while (true) {
          const int pw = window_read(a.slots, tile, min(seg, WMAX), SV, SA, ep, Win);
          if (pw >= 0) {
            if (tid < D) {
              float dl = Win[pw * SV + 2 * D + tid];
              for (int w = pw - 1; w >= 0; --w) dl = fmaf(Win[w * SV + tid], dl, Win[w * SV + D + tid]);
              Din[tid] = dl;
              slot_put(myslot + 2 * D + tid, ep, fmaf(ta, dl, tbv));
            }
            break;
          }
          if (++spins > kSpinLimit) {
            if (tid == 0) record_fault(ctrl, 1);
            if (tid < D) Din[tid] = 0.f;
            break;
          }
          backoff(spins);
        }
      }
      __syncthreads();
      // ---- fix-up: each (part, channel) walks its steps from its incoming increment ----
      {
        float dl = Din[ci];
        for (int q = 0; q < pp_; ++q) dl = fmaf(Sa[q * D + ci], dl, Sb[q * D + ci]);
        for (int s = pp_ * LP; s < min(Lv, (pp_ + 1) * LP); ++s) {
          dl = fmaf(Jd[s * D + ci], dl, R[s * D + ci]);
          float* o = Hnext + ((size_t)b * T + t0 + s) * D + ci;
          const float v = X[(s + 1) * LD + ci] + dl;
          if (s == kTL - 1) coherent_store(o, v);   // the next tile's halo
          else *o = v;
        }
      }
      __syncthreads();
    }
    end_pass(a, blk_max, k, cur);
    if (__hip_atomic_load(&ctrl->done, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) || has_fault(ctrl)) break;
    cur = next;
  }
}

// =====================================================================================
// Dense 16x16 Jacobian.  LDS: Bh[48] | X[65 LD] | Xj (reuse) | R, Z, Al, Be, Ga [64][16] |
// Pagg[8][272] | Tot[272] | Tmp[272] | Pin[9][16] | Vec[2][16] | Win[W][288] | Din[16].
constexpr int kF = 16;
constexpr int kFAgg = kF * kF + kF;      // aggregate values: M (row-major) then v
constexpr int kFSlot = kFAgg + kF;       // slot values: aggregate, then prefix
constexpr int kFWin = 16;
__host__ __device__ inline size_t mff_lds_floats(int reuse) {
  const int LD = kF + 4;
  return (size_t)3 * kF + (size_t)(kTL + 1) * LD * (reuse ? 2 : 1) + (size_t)5 * kTL * kF +
         (size_t)kFParts * kFAgg + 2 * kFAgg + (size_t)(kFParts + 1) * kF + 2 * kF + (size_t)kFWin * kFSlot + kF;
}

// Entry J_t[row][col] from the factors of `row` and U_g[row][col] (g = r, z, n).
__device__ __forceinline__ float jac_entry(float z, float al, float be, float ga, float ur, float uz, float un,
                                           bool diag) {
  return fmaf(al, uz, fmaf(be, ur, ga * un)) + (diag ? z : 0.f);
}

__global__ void __launch_bounds__(PNR_BLOCK) dense_full_mfma_kernel(DenseLoopArgs<float> a) {
  extern __shared__ __align__(16) float lds[];
  Ctrl* ctrl = a.ctrl;
  constexpr int D = kF, LD = kF + 4;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int m = lane & 15, q = lane >> 4;
  const int T = a.T;
  const bool reuse = a.nbuf > 2;
  float* Bh = lds;
  float* X = Bh + 3 * D;
  float* Xj = X + (kTL + 1) * LD;
  float* R = Xj + (reuse ? (kTL + 1) * LD : 0);
  float* Zv = R + kTL * D;
  float* Al = Zv + kTL * D;
  float* Be = Al + kTL * D;
  float* Ga = Be + kTL * D;
  float* Pagg = Ga + kTL * D;
  float* Tot = Pagg + kFParts * kFAgg;
  float* Tmp = Tot + kFAgg;
  float* Pin = Tmp + kFAgg;
  float* Vec = Pin + (kFParts + 1) * D;
  float* Win = Vec + 2 * D;
  float* Din = Win + kFWin * kFSlot;

  for (int i = tid; i < 3 * D; i += PNR_BLOCK) Bh[i] = a.bh ? a.bh[i] : 0.f;
  // U in registers: MFMA B fragments for the recurrent product, and the entries each
  // lane needs to form J^T (aggregate pass) and J (fix-up pass) operands
  float uf[3][D / 4], ubT[3][4], ubN[3][4];
#pragma unroll
  for (int g = 0; g < 3; ++g) {
#pragma unroll
    for (int kk = 0; kk < D / 4; ++kk) uf[g][kk] = a.U[(size_t)(g * D + m) * D + 4 * kk + q];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      ubT[g][i] = a.U[(size_t)(g * D + 4 * q + i) * D + m];   // U_g[4q+i][m]
      ubN[g][i] = a.U[(size_t)(g * D + m) * D + 4 * q + i];   // U_g[m][4q+i]
    }
  }
  __syncthreads();
  const float bhr = Bh[m], bhz = Bh[D + m], bhn = Bh[2 * D + m];

  int cur = -1, jac = -1;
  for (int k = 0; k <= a.max_iters; ++k) {
    const bool resid_only = k == a.max_iters;
    if (!resid_only && k % a.jac_every == 0) jac = cur;
    const int next = resid_only ? cur : next_buffer(cur, jac, a.nbuf);
    const float* Hcur = cur >= 0 ? a.H[cur] : nullptr;
    const float* Hjac = jac >= 0 ? a.H[jac] : nullptr;
    float* Hnext = next >= 0 ? a.H[next] : nullptr;
    const bool stale = !resid_only && jac != cur;
    const uint32_t ep = (uint32_t)k + 1u;
    uint32_t blk_max = 0;
    // Items go out time-segment-major (segment s of every batch row before segment
    // s+1), so a tile's predecessor always has a smaller item index: it was handed out
    // earlier, and prefixes are usually published before a successor looks back.
    for (int item = blockIdx.x; item < a.n_tiles; item += gridDim.x) {
      if (has_fault(ctrl)) break;
      const int seg = item / a.B, b = item - seg * a.B;
      const int tile = b * a.tiles_per_row + seg;   // slot index: row-major
      const int t0 = seg * kTL, Lv = min(kTL, T - t0);
      const float* gxb = a.gx + (size_t)b * T * 3 * D;
      stage_rows(X, Hcur, a.h0, b, t0, T, D, LD);
      if (stale) stage_rows(Xj, Hjac, a.h0, b, t0, T, D, LD);
      __syncthreads();

      // ---- cell on MFMA: residual and the Jacobian factors; wave w owns step block w ----
      uint32_t tmax = 0;
      {
        const int tb = wid;
        float gxv[4][3];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int s = tb * 16 + 4 * q + i;
          const float* g = gxb + (size_t)(t0 + s) * 3 * D;
#pragma unroll
          for (int gg = 0; gg < 3; ++gg) gxv[i][gg] = s < Lv ? g[gg * D + m] : 0.f;
        }
        v4f acc[3], accj[3];
        gates_block<D>(X, LD, tb, uf, acc);
        if (stale) gates_block<D>(Xj, LD, tb, uf, accj);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int s = tb * 16 + 4 * q + i;
          const int idx = s * D + m;
          if (s >= Lv) {   // padding steps: identity maps
            R[idx] = 0.f; Zv[idx] = 1.f; Al[idx] = 0.f; Be[idx] = 0.f; Ga[idx] = 0.f;
            continue;
          }
          const float p = X[s * LD + m];
          float r = sigm(gxv[i][0] + acc[0][i] + bhr);
          float z = sigm(gxv[i][1] + acc[1][i] + bhz);
          float ghn = acc[2][i] + bhn;
          float n = tanh_(fmaf(r, ghn, gxv[i][2]));
          const float res = fmaf(z, p - n, n) - X[(s + 1) * LD + m];
          R[idx] = res;
          tmax = max(tmax, abs_bits(res));
          if (resid_only) continue;
          float pj = p;
          if (stale) {
            pj = Xj[s * LD + m];
            r = sigm(gxv[i][0] + accj[0][i] + bhr);
            z = sigm(gxv[i][1] + accj[1][i] + bhz);
            ghn = accj[2][i] + bhn;
            n = tanh_(fmaf(r, ghn, gxv[i][2]));
          }
          const float omz = 1.f - z, cn = omz * (1.f - n * n);
          const bool zero = a.jac_mode == PNR_JAC_ZERO;
          Zv[idx] = zero ? 0.f : z;
          Al[idx] = zero ? 0.f : (pj - n) * z * omz;
          Be[idx] = zero ? 0.f : cn * ghn * r * (1.f - r);
          Ga[idx] = zero ? 0.f : cn * r;
        }
      }
      blk_max = max(blk_max, tmax);
      __syncthreads();
      if (resid_only) continue;

      // ---- part aggregates on MFMA, built from the back: S^T <- J_t^T S^T, v += S r_t ----
      {
        const int pa = 2 * wid, pb = 2 * wid + 1;
        v4f xa, xb;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          xa[i] = (4 * q + i == m) ? 1.f : 0.f;
          xb[i] = xa[i];
        }
        float va = 0.f, vb = 0.f;
#pragma unroll 1
        for (int st = kFPartLen - 1; st >= 0; --st) {
          const int sa = pa * kFPartLen + st, sb = pb * kFPartLen + st;
          float aa[4], ab[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int row = 4 * q + i;
            va = fmaf(xa[i], R[sa * D + row], va);
            vb = fmaf(xb[i], R[sb * D + row], vb);
            aa[i] = jac_entry(Zv[sa * D + row], Al[sa * D + row], Be[sa * D + row], Ga[sa * D + row], ubT[0][i],
                              ubT[1][i], ubT[2][i], row == m);
            ab[i] = jac_entry(Zv[sb * D + row], Al[sb * D + row], Be[sb * D + row], Ga[sb * D + row], ubT[0][i],
                              ubT[1][i], ubT[2][i], row == m);
          }
          v4f ya = v4f{0.f, 0.f, 0.f, 0.f}, yb = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            ya = mfma4(aa[i], xa[i], ya);
            yb = mfma4(ab[i], xb[i], yb);
          }
          xa = ya;
          xb = yb;
        }
        // lane (q, m) holds S^T[4q+i][m] = M[m][4q+i]; v[m] = sum over q of the partials
        va += __shfl_xor(va, 16);
        va += __shfl_xor(va, 32);
        vb += __shfl_xor(vb, 16);
        vb += __shfl_xor(vb, 32);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          Pagg[pa * kFAgg + m * D + 4 * q + i] = xa[i];
          Pagg[pb * kFAgg + m * D + 4 * q + i] = xb[i];
        }
        if (q == 0) {
          Pagg[pa * kFAgg + D * D + m] = va;
          Pagg[pb * kFAgg + D * D + m] = vb;
        }
      }
      __syncthreads();

      // ---- tile total: (M, v) <- part_p o (M, v) for p = 1..7 ----
      for (int i = tid; i < kFAgg; i += PNR_BLOCK) Tot[i] = Pagg[i];
      __syncthreads();
#pragma unroll 1
      for (int p = 1; p < kFParts; ++p) {
        const float* Mp = Pagg + p * kFAgg;
        {
          const int r_ = tid >> 4, c_ = tid & 15;   // 256 threads = 16 x 16 entries
          float s_ = 0.f;
#pragma unroll
          for (int l = 0; l < D; ++l) s_ = fmaf(Mp[r_ * D + l], Tot[l * D + c_], s_);
          Tmp[r_ * D + c_] = s_;
          if (tid < D) {
            float v_ = Mp[D * D + tid];
#pragma unroll
            for (int l = 0; l < D; ++l) v_ = fmaf(Mp[tid * D + l], Tot[D * D + l], v_);
            Tmp[D * D + tid] = v_;
          }
        }
        __syncthreads();
        for (int i = tid; i < kFAgg; i += PNR_BLOCK) Tot[i] = Tmp[i];
        __syncthreads();
      }
      uint64_t* myslot = a.slots + (size_t)tile * kFSlot;
      if (seg == 0) {
        if (tid < D) {
          slot_put(myslot + kFAgg + tid, ep, Tot[D * D + tid]);
          Din[tid] = 0.f;
        }
      } else {
        for (int i = tid; i < kFAgg; i += PNR_BLOCK) slot_put(myslot + i, ep, Tot[i]);
        // ---- decoupled look-back: apply the aggregates after the nearest prefix to it ----
        uint32_t spins = 0;
        while (true) {
          const int pw = window_read(a.slots, tile, min(seg, kFWin), kFSlot, kFAgg, ep, Win);
          if (pw >= 0) {
            if (tid < D) Vec[tid] = Win[pw * kFSlot + kFAgg + tid];
            __syncthreads();
            int src = 0;
            for (int w = pw - 1; w >= 0; --w) {
              if (tid < D) {
                const float* Mw = Win + w * kFSlot;
                float v_ = Mw[D * D + tid];
#pragma unroll
                for (int l = 0; l < D; ++l) v_ = fmaf(Mw[tid * D + l], Vec[src * D + l], v_);
                Vec[(1 - src) * D + tid] = v_;
              }
              __syncthreads();
              src = 1 - src;
            }
            if (tid < D) Din[tid] = Vec[src * D + tid];
            __syncthreads();
            if (tid < D) {
              float v_ = Tot[D * D + tid];
#pragma unroll
              for (int l = 0; l < D; ++l) v_ = fmaf(Tot[tid * D + l], Din[l], v_);
              slot_put(myslot + kFAgg + tid, ep, v_);
            }
            break;
          }
          if (++spins > kSpinLimit) {
            if (tid == 0) record_fault(ctrl, 1);
            if (tid < D) Din[tid] = 0.f;
            break;
          }
          backoff(spins);
        }
      }
      __syncthreads();

      // ---- increments entering the parts: Pin[p+1] = M_p Pin[p] + v_p ----
      if (tid < D) Pin[tid] = Din[tid];
      __syncthreads();
      for (int p = 0; p < kFParts - 1; ++p) {
        if (tid < D) {
          const float* Mp = Pagg + p * kFAgg;
          float v_ = Mp[D * D + tid];
#pragma unroll
          for (int l = 0; l < D; ++l) v_ = fmaf(Mp[tid * D + l], Pin[p * D + l], v_);
          Pin[(p + 1) * D + tid] = v_;
        }
        __syncthreads();
      }

      // ---- fix-up on MFMA: d <- J_t d + r_t with d in column 0; s <- s + d ----
      {
        const int pa = 2 * wid, pb = 2 * wid + 1;
        v4f xa, xb;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          xa[i] = m == 0 ? Pin[pa * D + 4 * q + i] : 0.f;
          xb[i] = m == 0 ? Pin[pb * D + 4 * q + i] : 0.f;
        }
#pragma unroll 1
        for (int st = 0; st < kFPartLen; ++st) {
          const int sa = pa * kFPartLen + st, sb = pb * kFPartLen + st;
          const float za = Zv[sa * D + m], ala = Al[sa * D + m], bea = Be[sa * D + m], gaa = Ga[sa * D + m];
          const float zb = Zv[sb * D + m], alb = Al[sb * D + m], beb = Be[sb * D + m], gab = Ga[sb * D + m];
          v4f ya, yb;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            ya[i] = m == 0 ? R[sa * D + 4 * q + i] : 0.f;
            yb[i] = m == 0 ? R[sb * D + 4 * q + i] : 0.f;
          }
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float ja = jac_entry(za, ala, bea, gaa, ubN[0][i], ubN[1][i], ubN[2][i], 4 * q + i == m);
            const float jb = jac_entry(zb, alb, beb, gab, ubN[0][i], ubN[1][i], ubN[2][i], 4 * q + i == m);
            ya = mfma4(ja, xa[i], ya);
            yb = mfma4(jb, xb[i], yb);
          }
          xa = ya;
          xb = yb;
          if (m == 0) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int c = 4 * q + i;
              if (sa < Lv) {
                float* o = Hnext + ((size_t)b * T + t0 + sa) * D + c;
                const float v = X[(sa + 1) * LD + c] + xa[i];
                if (sa == kTL - 1) coherent_store(o, v);
                else *o = v;
              }
              if (sb < Lv) {
                float* o = Hnext + ((size_t)b * T + t0 + sb) * D + c;
                const float v = X[(sb + 1) * LD + c] + xb[i];
                if (sb == kTL - 1) coherent_store(o, v);   // the next tile's halo
                else *o = v;
              }
            }
          }
        }
      }
      __syncthreads();
    }
    end_pass(a, blk_max, k, cur);
    if (__hip_atomic_load(&ctrl->done, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) || has_fault(ctrl)) break;
    cur = next;
  }
}

// =====================================================================================
int dense_mfma_supported(int D, int full, int is_f64) {
  if (is_f64) return 0;
  return full ? D == kF : (D == 16 || D == 32 || D == 64);
}
int dense_mfma_tile_len() { return kTL; }
int dense_mfma_slot_words(int D, int full) { return full ? kFSlot : 3 * D; }

template <class F>
static hipError_t coop_launch(F fn, const DenseLoopArgs<float>& a, size_t lds, int num_cu, hipStream_t st) {
  if (lds > 65536) {
    hipError_t e = hipFuncSetAttribute((const void*)fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  int v = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&v, fn, PNR_BLOCK, lds) != hipSuccess || v < 1)
    return hipErrorInvalidConfiguration;
  long g = (long)v * num_cu;
  if (g > kMaxGrid) g = kMaxGrid;
  if (g > a.n_tiles) g = a.n_tiles;
  if (g < 1) g = 1;
  void* args[] = {const_cast<DenseLoopArgs<float>*>(&a)};
  return hipLaunchCooperativeKernel((const void*)fn, dim3((int)g), dim3(PNR_BLOCK), args, (unsigned)lds, st);
}

hipError_t launch_dense_mfma(const DenseLoopArgs<float>& a, int full, int num_cu, hipStream_t st) {
  const int reuse = a.nbuf > 2;
  if (full) return coop_launch(dense_full_mfma_kernel, a, mff_lds_floats(reuse) * 4, num_cu, st);
  const size_t lds = mfd_lds_floats(a.D, reuse) * 4;
  if (a.D == 16) return coop_launch(dense_diag_mfma_kernel<16>, a, lds, num_cu, st);
  if (a.D == 32) return coop_launch(dense_diag_mfma_kernel<32>, a, lds, num_cu, st);
  return coop_launch(dense_diag_mfma_kernel<64>, a, lds, num_cu, st);
}

}  // namespace pnr
