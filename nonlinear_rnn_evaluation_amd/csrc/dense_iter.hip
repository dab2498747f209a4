// One Newton iteration for the GRU with a dense recurrent matrix U (D <= 64), fused:
// recurrent product U s_{t-1} for every step of a tile, gates, residual, Jacobian
// factors, the linear solve d_t = J_t d_{t-1} + r_t (scan of affine maps with a
// decoupled look-back across tiles) and the update s <- s + d.
//
// Method: ParaRNN overview page, "Technical Implementation / Newton's Iteration" and
// "Parallel Reduction"; DEER's dense Jacobian and quasi-DEER's diagonal one from
// "Towards Scalable and Stable Parallelization of Nonlinear RNNs" (abstract).
//
// The dense Jacobian of the linear-before-reset GRU factors as
//   J_t = diag(z) + diag(al) U_z + diag(be) U_r + diag(ga) U_n
//   al = (s - n) z (1 - z),  be = (1 - z)(1 - n^2) gh_n r (1 - r),  ga = (1 - z)(1 - n^2) r
// so it is never formed: the scan applies it to a vector with three products by the
// blocks of U (resident in LDS) and an elementwise combination.  Only four D-vectors
// per step live in LDS.
//
// Layout: gx [B][T][3D], states [B][T][D] (channel-contiguous).  A tile is L steps of
// one batch element; blocks are persistent and take tiles from a ticket counter.
//
// Scan organisation inside a tile:
//  * DIAG: thread (p, i) = part p of the tile, channel i; each part is a run of
//    consecutive steps composed serially; parts are combined in LDS; the look-back is
//    per channel.
//  * FULL: a group of D+1 lanes (inside one wave) owns one part.  Lane j < D carries
//    column j of the part's matrix product, lane D carries the vector part.  The block
//    total and the per-part prefixes are composed serially; the look-back moves a
//    (D*D + D)-value aggregate and a D-value prefix.
#include "common.h"
#include "kernels.h"

namespace pnr {

template <typename Tt> struct WordsOf { static constexpr int W = sizeof(Tt) / 4; };

// look-back slot words per tile: FULL holds the (D*D + D)-value aggregate then the
// D-value prefix; DIAG holds D values of a, D of b, then D prefixes.  W words per value.
__host__ __device__ inline int dense_slot_words_dev(int D, bool full, int W) {
  return full ? (D * D + 2 * D) * W : 3 * D * W;
}

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
// LDS layout (dynamic shared memory), all in units of Tt:
//   Us   [3D][D]     recurrent matrix
//   Bh   [3D]        recurrent bias
//   Hx   [L+1][D]    Hx[0] = s_{t0-1}, Hx[1+s] = current iterate at step t0+s
//   Hj   [L+1][D]    same for the state the Jacobian is taken at (only when stale)
//   R    [L][D]      residuals
//   Jd   [L][D]      diagonal Jacobian            (DIAG)
//   Z, Al, Be, Ga [L][D] Jacobian factors          (FULL)
//   scan scratch (see the two scan paths)
template <typename Tt>
struct DenseLds {
  int D, L, full, stale, parts;
  __host__ __device__ size_t count() const {
    size_t n = (size_t)3 * D * D + 3 * D + (size_t)(L + 1) * D * (stale ? 2 : 1) + (size_t)L * D;
    if (full) {
      n += (size_t)4 * L * D;
      n += (size_t)parts * (D * D + D);   // per-part aggregates
      n += (size_t)2 * (D * D + D);       // block total, look-back accumulator
      n += (size_t)(D * D + D);           // look-back scratch (predecessor aggregate)
      n += (size_t)(parts + 1) * D;       // per-part incoming increments
      n += (size_t)2 * parts * D;         // fix-up double buffer
      n += (size_t)D;                     // tile incoming increment
    } else {
      n += (size_t)L * D;                 // Jd
      n += (size_t)2 * parts * D;         // per-part aggregates (a, b)
      n += (size_t)D;                     // tile incoming increment
    }
    return n;
  }
};

template <typename Tt>
__device__ __forceinline__ void gru_gates(const Tt* __restrict__ Us, const Tt* __restrict__ Bh,
                                          const Tt* __restrict__ p, const Tt* __restrict__ g, int D,
                                          int i, Tt& r, Tt& z, Tt& n, Tt& ghn) {
  Tt ar = Bh[i], az = Bh[D + i], an = Bh[2 * D + i];
  const Tt* ur = Us + (size_t)i * D;
  const Tt* uz = Us + (size_t)(D + i) * D;
  const Tt* un = Us + (size_t)(2 * D + i) * D;
  for (int k = 0; k < D; ++k) {
    const Tt pk = p[k];
    ar = mul_add(ur[k], pk, ar);
    az = mul_add(uz[k], pk, az);
    an = mul_add(un[k], pk, an);
  }
  r = sigm(g[i] + ar);
  z = sigm(g[D + i] + az);
  ghn = an;
  n = tanh_(mul_add(r, an, g[2 * D + i]));
}

template <typename Tt, int DM, bool FULL, bool RESID_ONLY>
__global__ void __launch_bounds__(PNR_BLOCK) dense_iter_kernel(DenseIterArgs<Tt> a) {
  extern __shared__ __align__(16) unsigned char lds_raw[];
  Tt* lds = reinterpret_cast<Tt*>(lds_raw);
  __shared__ int s_tile;
  __shared__ int s_flag;
  __shared__ uint64_t s_wmax[PNR_WAVES];
  __shared__ int s_last;

  Ctrl* ctrl = a.ctrl;
  if (__hip_atomic_load(&ctrl->done, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) return;

  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int D = a.D, T = a.T, L = a.L;
  const bool stale = !RESID_ONLY && ((a.Hjac != a.Hcur) || a.jac_zero != a.cur_zero);
  const int GS = D + 1;                       // FULL: lanes per group
  const int GPW = FULL ? 64 / GS : 0;         // FULL: groups per wave
  const int parts = FULL ? GPW * PNR_WAVES : PNR_BLOCK / D;
  constexpr int W = WordsOf<Tt>::W;
  const uint32_t ep = (uint32_t)a.k + 1u;

  // carve LDS
  Tt* Us = lds;
  Tt* Bh = Us + 3 * D * D;
  Tt* Hx = Bh + 3 * D;
  Tt* Hj = Hx + (L + 1) * D;
  Tt* R = Hj + (stale ? (L + 1) * D : 0);
  Tt* Jd = R + L * D;            // DIAG
  Tt* Zv = R + L * D;            // FULL factors
  Tt* Al = Zv + L * D;
  Tt* Be = Al + L * D;
  Tt* Ga = Be + L * D;
  Tt* Pagg = FULL ? Ga + L * D : Jd + L * D;   // FULL: [parts][D*D + D]; DIAG: [2][parts][D]
  Tt* Tot = Pagg + (FULL ? parts * (D * D + D) : 2 * parts * D);   // FULL: [D*D + D]
  Tt* Acc = Tot + (FULL ? (D * D + D) : 0);                          // FULL: [D*D + D]
  Tt* Prd = Acc + (FULL ? (D * D + D) : 0);                          // FULL: [D*D + D]
  Tt* Pin = Prd + (FULL ? (D * D + D) : 0);                          // FULL: [parts + 1][D]
  Tt* Fx = Pin + (FULL ? (parts + 1) * D : 0);                       // FULL: [2][parts][D]
  Tt* Din = Fx + (FULL ? 2 * parts * D : 0);                         // [D]

  for (int idx = tid; idx < 3 * D * D; idx += PNR_BLOCK) Us[idx] = a.U[idx];
  for (int idx = tid; idx < 3 * D; idx += PNR_BLOCK) Bh[idx] = a.bh ? a.bh[idx] : Tt(0);

  uint64_t blk_max = 0;
  while (true) {
    if (tid == 0) s_tile = (int)atomicAdd(&ctrl->ticket, 1u);
    __syncthreads();
    const int tile = s_tile;
    if (tile >= a.n_tiles) break;
    const int b = tile / a.tiles_per_row;
    const int seg = tile - b * a.tiles_per_row;
    const int t0 = seg * L;
    const int Lv = min(L, T - t0);
    const Tt* gxb = a.gx + (size_t)b * T * 3 * D;

    // ---- stage states: Hx[0] = s_{t0-1}; Hx[1+s] = iterate at t0+s ----
    for (int idx = tid; idx < (L + 1) * D; idx += PNR_BLOCK) {
      const int s = idx / D, c = idx - s * D;
      const int t = t0 + s - 1;
      Tt v = Tt(0);
      if (t < 0) v = a.h0 ? a.h0[(size_t)b * D + c] : Tt(0);
      else if (t < T && !a.cur_zero) v = a.Hcur[((size_t)b * T + t) * D + c];
      Hx[idx] = v;
      if (stale) {
        Tt w = Tt(0);
        if (t < 0) w = a.h0 ? a.h0[(size_t)b * D + c] : Tt(0);
        else if (t < T && !a.jac_zero) w = a.Hjac[((size_t)b * T + t) * D + c];
        Hj[idx] = w;
      }
    }
    __syncthreads();

    // ---- cell: gates, residual, Jacobian (diagonal or factors) ----
    uint64_t tmax = 0;
    for (int idx = tid; idx < L * D; idx += PNR_BLOCK) {
      const int s = idx / D, i = idx - s * D;
      if (s >= Lv) {
        R[idx] = Tt(0);
        if (!RESID_ONLY) {
          if (FULL) { Zv[idx] = Tt(1); Al[idx] = Tt(0); Be[idx] = Tt(0); Ga[idx] = Tt(0); }
          else Jd[idx] = Tt(1);
        }
        continue;
      }
      const Tt* g = gxb + (size_t)(t0 + s) * 3 * D;
      const Tt* p = Hx + s * D;
      Tt r, z, n, ghn;
      gru_gates(Us, Bh, p, g, D, i, r, z, n, ghn);
      const Tt f = mul_add(z, p[i] - n, n);
      const Tt res = f - Hx[(s + 1) * D + i];
      R[idx] = res;
      tmax = max(tmax, abs_bits64(res));
      if (RESID_ONLY) continue;
      const Tt* pj = p;
      if (stale) {
        pj = Hj + s * D;
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
        Jd[idx] = z + al * Us[(size_t)(D + i) * D + i] + be * Us[(size_t)i * D + i] +
                  ga * Us[(size_t)(2 * D + i) * D + i];
      }
    }
    blk_max = max(blk_max, tmax);
    __syncthreads();
    if (RESID_ONLY) continue;

    uint64_t* myslot = a.slots + (size_t)tile * dense_slot_words_dev(D, FULL, W);

    if constexpr (!FULL) {
      // ================= DIAG: per-channel scalar scan =================
      const int p = tid / D, i = tid - p * D;
      const int lp = (L + parts - 1) / parts;
      Tt* Sa = Pagg;
      Tt* Sb = Pagg + parts * D;
      if (p < parts) {
        Tt ea = Tt(1), eb = Tt(0);
        for (int s = p * lp; s < min(L, (p + 1) * lp); ++s) {
          const Tt ja = Jd[s * D + i];
          eb = mul_add(ja, eb, R[s * D + i]);
          ea = ja * ea;
        }
        Sa[p * D + i] = ea; Sb[p * D + i] = eb;
      }
      __syncthreads();
      if (tid < D) {
        // block total for channel i and the look-back on that channel
        Tt ta = Sa[tid], tb = Sb[tid];
        for (int q = 1; q < parts; ++q) {
          const Tt qa = Sa[q * D + tid], qb = Sb[q * D + tid];
          tb = mul_add(qa, tb, qb);
          ta = qa * ta;
        }
        uint64_t* aggA = myslot + (size_t)tid * W;
        uint64_t* aggB = myslot + (size_t)(D + tid) * W;
        uint64_t* pre = myslot + (size_t)(2 * D + tid) * W;
        Tt din = Tt(0);
        if (seg == 0) {
          vput(pre, ep, tb);
        } else {
          vput(aggA, ep, ta);
          vput(aggB, ep, tb);
          Tt acc_a = Tt(1), acc_b = Tt(0);
          int j = tile - 1;
          const size_t sw = (size_t)dense_slot_words_dev(D, FULL, W);
          while (true) {
            const uint64_t* js = a.slots + (size_t)j * sw;
            Tt pv;
            if (vget(js + (size_t)(2 * D + tid) * W, ep, pv)) {
              din = mul_add(acc_a, pv, acc_b);
              break;
            }
            Tt qa, qb;
            bool ok = vget(js + (size_t)tid * W, ep, qa);
            ok &= vget(js + (size_t)(D + tid) * W, ep, qb);
            if (ok) {
              acc_b = mul_add(acc_a, qb, acc_b);
              acc_a = acc_a * qa;
              --j;
              continue;
            }
            __builtin_amdgcn_s_sleep(1);
          }
          vput(pre, ep, mul_add(ta, din, tb));
        }
        Din[tid] = din;
      }
      __syncthreads();
      if (p < parts) {
        Tt dl = Din[i];
        for (int q = 0; q < p; ++q) dl = mul_add(Sa[q * D + i], dl, Sb[q * D + i]);
        for (int s = p * lp; s < min(Lv, (p + 1) * lp); ++s) {
          dl = mul_add(Jd[s * D + i], dl, R[s * D + i]);
          a.Hnext[((size_t)b * T + t0 + s) * D + i] = Hx[(s + 1) * D + i] + dl;
        }
      }
      __syncthreads();
    } else {
      // ================= FULL: dense D x D scan =================
      const int gi = lane / GS;                // group inside the wave
      const int j = lane - gi * GS;            // lane inside the group
      const bool in_group = gi < GPW;
      const int part = wid * GPW + gi;
      const int lp = (L + parts - 1) / parts;
      const int DD = D * D + D;
      // (1) part aggregates: lane j < D carries column j of the matrix product, lane D the vector
      if (in_group) {
        Tt col[DM];
#pragma unroll
        for (int m = 0; m < DM; ++m) col[m] = (j < D && m == j) ? Tt(1) : Tt(0);
        for (int s = part * lp; s < min(L, (part + 1) * lp); ++s) {
          const Tt* zr = Zv + s * D; const Tt* ar = Al + s * D;
          const Tt* br = Be + s * D; const Tt* gr = Ga + s * D;
          Tt nw[DM];
#pragma unroll
          for (int m = 0; m < DM; ++m) {
            Tt ur = 0, uz = 0, un = 0;
            if (m < D) {
              const Tt* rr = Us + (size_t)m * D;
              const Tt* rz = Us + (size_t)(D + m) * D;
              const Tt* rn = Us + (size_t)(2 * D + m) * D;
#pragma unroll
              for (int k = 0; k < DM; ++k) {
                if (k < D) {
                  ur = mul_add(rr[k], col[k], ur);
                  uz = mul_add(rz[k], col[k], uz);
                  un = mul_add(rn[k], col[k], un);
                }
              }
            }
            Tt v = m < D ? zr[m] * col[m] + ar[m] * uz + br[m] * ur + gr[m] * un : Tt(0);
            if (j == D && m < D) v += R[s * D + m];
            nw[m] = v;
          }
#pragma unroll
          for (int m = 0; m < DM; ++m) col[m] = nw[m];
        }
        Tt* ag = Pagg + (size_t)part * DD;     // [D][D] row-major, then [D]
#pragma unroll
        for (int m = 0; m < DM; ++m) {
          if (m < D) {
            if (j < D) ag[m * D + j] = col[m];
            else ag[D * D + m] = col[m];
          }
        }
      }
      __syncthreads();
      // (2) block total = agg_{parts-1} o ... o agg_0 (one group, column per lane)
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
              for (int k = 0; k < DM; ++k)
                if (k < D) v = mul_add(ag[m * D + k], col[k], v);
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
      // (3) decoupled look-back over whole tiles (all threads poll together)
      const size_t sw = (size_t)dense_slot_words_dev(D, true, W);
      uint64_t* mpre = myslot + (size_t)DD * W;
      if (seg == 0) {
        for (int m = tid; m < D; m += PNR_BLOCK) {
          Din[m] = Tt(0);
          vput(mpre + (size_t)m * W, ep, Tot[D * D + m]);
        }
        __syncthreads();
      } else {
        for (int e = tid; e < DD; e += PNR_BLOCK) {
          vput(myslot + (size_t)e * W, ep, Tot[e]);
          Acc[e] = (e < D * D) ? ((e / D == e % D) ? Tt(1) : Tt(0)) : Tt(0);
        }
        int jt = tile - 1;
        while (true) {
          const uint64_t* js = a.slots + (size_t)jt * sw;
          if (tid == 0) s_flag = 1;
          __syncthreads();
          // predecessor's inclusive prefix?
          for (int m = tid; m < D; m += PNR_BLOCK) {
            Tt v;
            if (!vget(js + (size_t)(DD + m) * W, ep, v)) s_flag = 0;
            Prd[m] = v;
          }
          __syncthreads();
          if (s_flag) {
            for (int m = tid; m < D; m += PNR_BLOCK) {
              Tt v = Acc[D * D + m];
              for (int k = 0; k < D; ++k) v = mul_add(Acc[m * D + k], Prd[k], v);
              Din[m] = v;
            }
            __syncthreads();
            break;
          }
          __syncthreads();
          if (tid == 0) s_flag = 1;
          __syncthreads();
          for (int e = tid; e < DD; e += PNR_BLOCK) {
            Tt v;
            if (!vget(js + (size_t)e * W, ep, v)) s_flag = 0;
            Prd[e] = v;
          }
          __syncthreads();
          if (s_flag) {
            // Acc <- Acc o Prd = (Acc_M Prd_M, Acc_M Prd_v + Acc_v); new values staged in Tot's
            // tail is not safe, so compute into registers per entry first.
            Tt vals[(DM * DM + DM + PNR_BLOCK - 1) / PNR_BLOCK];
            int c = 0;
            for (int e = tid; e < DD; e += PNR_BLOCK, ++c) {
              Tt v;
              if (e < D * D) {
                const int m = e / D, n = e - m * D;
                v = Tt(0);
                for (int k = 0; k < D; ++k) v = mul_add(Acc[m * D + k], Prd[k * D + n], v);
              } else {
                const int m = e - D * D;
                v = Acc[D * D + m];
                for (int k = 0; k < D; ++k) v = mul_add(Acc[m * D + k], Prd[D * D + k], v);
              }
              vals[c] = v;
            }
            __syncthreads();
            c = 0;
            for (int e = tid; e < DD; e += PNR_BLOCK, ++c) Acc[e] = vals[c];
            __syncthreads();
            --jt;
            continue;
          }
          __syncthreads();   // every thread has read s_flag before thread 0 resets it
          __builtin_amdgcn_s_sleep(1);
        }
        // publish this tile's inclusive prefix: Tot applied to Din
        for (int m = tid; m < D; m += PNR_BLOCK) {
          Tt v = Tot[D * D + m];
          for (int k = 0; k < D; ++k) v = mul_add(Tot[m * D + k], Din[k], v);
          vput(mpre + (size_t)m * W, ep, v);
        }
      }
      // (4) increments entering each part: Pin[0] = Din, Pin[q+1] = agg_q(Pin[q])
      for (int m = tid; m < D; m += PNR_BLOCK) Pin[m] = Din[m];
      __syncthreads();
      for (int q = 0; q < parts; ++q) {
        if (tid < D) {
          const Tt* ag = Pagg + (size_t)q * DD;
          Tt v = ag[D * D + tid];
          for (int k = 0; k < D; ++k) v = mul_add(ag[tid * D + k], Pin[q * D + k], v);
          Pin[(q + 1) * D + tid] = v;
        }
        __syncthreads();
      }
      // (5) fix-up: each group walks its part with the dense J applied to its increment
      Tt* cur = Fx;
      Tt* nxt = Fx + parts * D;
      if (in_group && j < D) cur[part * D + j] = Pin[part * D + j];
      __syncthreads();
      for (int st = 0; st < lp; ++st) {
        const int s = part * lp + st;
        if (in_group && j < D && s < L) {
          const Tt* dv = cur + part * D;
          Tt ur = 0, uz = 0, un = 0;
          const Tt* rr = Us + (size_t)j * D;
          const Tt* rz = Us + (size_t)(D + j) * D;
          const Tt* rn = Us + (size_t)(2 * D + j) * D;
          for (int k = 0; k < D; ++k) {
            ur = mul_add(rr[k], dv[k], ur);
            uz = mul_add(rz[k], dv[k], uz);
            un = mul_add(rn[k], dv[k], un);
          }
          const int q = s * D + j;
          const Tt v = Zv[q] * dv[j] + Al[q] * uz + Be[q] * ur + Ga[q] * un + R[q];
          nxt[part * D + j] = v;
          if (s < Lv) a.Hnext[((size_t)b * T + t0 + s) * D + j] = Hx[(s + 1) * D + j] + v;
        }
        __syncthreads();
        Tt* tmp = cur; cur = nxt; nxt = tmp;
      }
    }
  }

  // ---- level 2 of the residual max: block partial -> global -> the last block merges ----
  blk_max = wave_max_u64(blk_max);
  if (lane == 0) s_wmax[wid] = blk_max;
  __syncthreads();
  if (tid == 0) {
    uint64_t m = s_wmax[0];
    for (int w = 1; w < PNR_WAVES; ++w) m = max(m, s_wmax[w]);
    __hip_atomic_store(&a.partials[blockIdx.x], m, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __threadfence();
    const uint32_t prev = atomicAdd(&ctrl->finished, 1u);
    s_last = prev == gridDim.x - 1;
  }
  __syncthreads();
  if (!s_last) return;
  __threadfence();
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
    finish_iteration(ctrl, a.rho_hist, rho_of<Tt>(m), a.k, a.cur_buf, a.max_iters, a.tol);
  }
}

// ---------------------------------------------------------------------------------
int dense_supported(int D, int full, int is_f64) {
  if (D < 1) return 0;
  if (full) return D <= 32;
  return is_f64 ? D <= 32 : D <= 64;
}

int dense_tile_len(int D, int full, int) {
  if (full) {
    const int parts = (64 / (D + 1)) * PNR_WAVES;
    const int lp = D <= 4 ? 2 : (D <= 8 ? 4 : 8);
    return parts * lp;
  }
  return 64;
}

static int dense_parts(int D, int full) { return full ? (64 / (D + 1)) * PNR_WAVES : PNR_BLOCK / D; }

int dense_slot_words(int D, int full, int is_f64) { return dense_slot_words_dev(D, full, is_f64 ? 2 : 1); }

size_t dense_lds_bytes(int D, int full, int is_f64, int stale) {
  DenseLds<float> l{D, dense_tile_len(D, full, is_f64), full, stale, dense_parts(D, full)};
  return l.count() * (is_f64 ? 8 : 4);
}

template <typename Tt, int DM, bool FULL, bool R>
static hipError_t launch_one(const DenseIterArgs<Tt>& a, int num_cu, hipStream_t st, size_t lds) {
  auto fn = dense_iter_kernel<Tt, DM, FULL, R>;
  static size_t attr_set = 0;
  if (lds > 65536 && lds > attr_set) {
    hipError_t e = hipFuncSetAttribute((const void*)fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    attr_set = lds;
  }
  int v = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&v, fn, PNR_BLOCK, lds) != hipSuccess || v < 1) v = 1;
  long g = (long)v * num_cu;
  if (g > kMaxGrid) g = kMaxGrid;
  if (g > a.n_tiles) g = a.n_tiles;
  if (g < 1) g = 1;
  hipLaunchKernelGGL(fn, dim3((int)g), dim3(PNR_BLOCK), lds, st, a);
  return hipGetLastError();
}

template <typename Tt, int DM, bool FULL>
static hipError_t launch_dm(const DenseIterArgs<Tt>& a, int num_cu, hipStream_t st) {
  const bool stale = !a.resid_only && ((a.Hjac != a.Hcur) || a.jac_zero != a.cur_zero);
  const size_t lds = dense_lds_bytes(a.D, FULL, sizeof(Tt) == 8, stale);
  return a.resid_only ? launch_one<Tt, DM, FULL, true>(a, num_cu, st, lds)
                      : launch_one<Tt, DM, FULL, false>(a, num_cu, st, lds);
}

template <typename Tt>
static hipError_t launch_dense_t(const DenseIterArgs<Tt>& a, int full, int num_cu, hipStream_t st) {
  if (!full) return launch_dm<Tt, 1, false>(a, num_cu, st);
  if (a.D <= 4) return launch_dm<Tt, 4, true>(a, num_cu, st);
  if (a.D <= 8) return launch_dm<Tt, 8, true>(a, num_cu, st);
  if (a.D <= 16) return launch_dm<Tt, 16, true>(a, num_cu, st);
  return launch_dm<Tt, 32, true>(a, num_cu, st);
}

hipError_t launch_dense_iter_f32(const DenseIterArgs<float>& a, int full, int num_cu, hipStream_t st) {
  return launch_dense_t<float>(a, full, num_cu, st);
}
hipError_t launch_dense_iter_f64(const DenseIterArgs<double>& a, int full, int num_cu, hipStream_t st) {
  return launch_dense_t<double>(a, full, num_cu, st);
}

}  // namespace pnr
