// Damped (Levenberg-Marquardt) iteration for the GRU with a dense recurrent matrix U, with
// the diagonal Jacobian: quasi-ELK ("Towards Scalable and Stable Parallelization of
// Nonlinear RNNs", abstract and the summary's "Approach": a trust region whose
// linear-Gaussian MAP solve is a Kalman filter and smoother; with the diagonal Jacobian,
// quasi-ELK).
//
// One iteration on the iterate H [B][T][D]:
//   1. gh = U h_{t-1} + b_h for every step (the channels couple only here), the cell:
//      residual R_t = f(h_{t-1}, x_t) - h_t, the quasi Jacobian J_t = diag(df/dh), max |R|;
//   2. per channel the scalar filter P- = J^2 P + 1, m- = J m + R, P = P- / (1 + lam P-),
//      m = m- / (1 + lam P-) -- a forward scan of 3x3 maps in homogeneous coordinates --
//      and from it the smoother's gain and offset in new-iterate space,
//        G_t = P_t J_{t+1} / P-_{t+1},  e_t = m_t + h_t - G_t (m-_{t+1} + h_{t+1})
//      (G = 0, e = m + h at the last step);
//   3. the smoother h'_t = G_t h'_{t+1} + e_t, a backward affine scan, gives the next
//      iterate.
//
// The whole loop runs in one persistent, co-resident grid.  The sequence is cut into
// chunks of 16 steps (one MFMA row tile); a wave owns a fixed set of chunks for the whole
// launch, and per iteration:
//   A. per chunk: the 16 rows of gh on fp32 MFMA (16x16x4: 12 column tiles of 16 over the
//      three gates, 16 k-steps over the 64 padded channels; U's operand fragments in LDS),
//      the cell in lane = channel order from an LDS transpose, and the chunk's composed
//      filter map;
//   grid barrier: the last block merges the residual maxima, records rho_k and decides
//      (stop when rho_k <= tol, on a non-finite rho, or after max_iters updates);
//   B. one wave per (b, channel) scans the chunk maps into each chunk's entering filter
//      state (lanes = chunks, shuffles);
//   C. per chunk: the filter walk from that state, G and e per step, and the chunk's
//      composed smoother map;
//   D. one wave per (b, channel) scans the smoother maps backwards into the smoothed
//      state after each chunk;
//   E. per chunk: the smoother walk, which writes the next iterate.
// Grid barriers separate A..E (four per iteration).  Values that cross waves -- chunk maps
// and carries, and per chunk its first step's (J, R, h) and its last step's (G, e) -- are
// written and read with agent-scope atomics; everything else a wave reads it wrote itself.
// The state before a chunk's first step, which step 1 needs, is formed by the chunk
// itself at the end of E from its predecessor's last (G, e) and its own first smoothed
// state: the value the predecessor writes for that step, up to rounding, so the next
// iteration needs no fifth barrier.
#include "common.h"
#include "kernels.h"

namespace pnr {

constexpr int kEChunk = 16;                 // steps per chunk: one 16-row MFMA tile
constexpr int kElkWaves = 8;
constexpr int kStLd = 64 + 4;               // staged h_{t-1} rows: 16 rows x 4 k of an A fragment hit 64 banks
constexpr int kGhLd = 3 * 64 + 4;           // transposed gh rows
constexpr int kCarryGroups = 4;             // chunk maps loaded together per carry round trip
typedef float v4f_t __attribute__((ext_vector_type(4)));

int elk_dense_chunks(int T) { return (T + kEChunk - 1) / kEChunk; }

__device__ __forceinline__ Flt filter_step(float j, float r, float lam) {
  const float j2 = j * j;
  return Flt{j2, 1.f, lam * j2, 1.f + lam, 0.f, r, j};
}
__device__ __forceinline__ Flt flt_shfl_up(const Flt& f, int off) {
  return Flt{__shfl_up(f.a, off, 64), __shfl_up(f.b, off, 64), __shfl_up(f.c, off, 64), __shfl_up(f.d, off, 64),
             __shfl_up(f.e, off, 64), __shfl_up(f.f, off, 64), __shfl_up(f.g, off, 64)};
}
__device__ __forceinline__ Flt flt_shfl(const Flt& f, int src) {
  return Flt{__shfl(f.a, src, 64), __shfl(f.b, src, 64), __shfl(f.c, src, 64), __shfl(f.d, src, 64),
             __shfl(f.e, src, 64), __shfl(f.f, src, 64), __shfl(f.g, src, 64)};
}
// the rows this wave just wrote to LDS are read back by every lane of the wave
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
  __builtin_amdgcn_wave_barrier();
}

__global__ void __launch_bounds__(64 * kElkWaves, 1) gru_elk_loop_kernel(ElkLoopArgs a) {
  // per wave: the staged h_{t-1} rows [16][kStLd] (MFMA A operand), then, over them, gh
  // transposed [16][kGhLd]
  __shared__ __align__(16) float wbuf[kElkWaves][kEChunk * kGhLd];
  // uf[kk][nt][l] = U_g[c][j], g = nt / 4, c = 16 (nt % 4) + l % 16, j = 4 kk + l / 16
  // (zero past D): the B operand of k-step kk, column tile nt, for lane l
  __shared__ float uf[16][12][64];
  __shared__ uint32_t s_wmax[kElkWaves];
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6, tid = threadIdx.x;
  const int D = a.D, T = a.T, nch = a.nch;
  const bool act = lane < D;
  const float lam = a.lam;
  Ctrl* ctrl = a.ctrl;
  for (int idx = tid; idx < 16 * 12 * 64; idx += 64 * kElkWaves) {
    const int kk = idx / (12 * 64), nt = (idx >> 6) % 12, l = idx & 63;
    const int g = nt >> 2, c = 16 * (nt & 3) + (l & 15), j = 4 * kk + (l >> 4);
    uf[kk][nt][l] = (c < D && j < D) ? a.U[(size_t)(g * D + c) * D + j] : 0.f;
  }
  // per lane (channel): the diagonals U_r[i][i], U_z[i][i], U_n[i][i] and b_h
  float ud[3] = {0.f, 0.f, 0.f}, bhv[3] = {0.f, 0.f, 0.f};
  if (act) {
#pragma unroll
    for (int g = 0; g < 3; ++g) {
      ud[g] = a.U[(size_t)(g * D + lane) * D + lane];
      bhv[g] = a.bh ? a.bh[g * D + lane] : 0.f;
    }
  }
  __syncthreads();
  const int gw = blockIdx.x * kElkWaves + wid, nw = gridDim.x * kElkWaves;
  const int ntask = a.B * nch, nrow = a.B * D;
  float* st = wbuf[wid];
  const int m16 = lane & 15, q4 = lane >> 4;
  int cur = 0;
  for (int k = 0; k <= a.max_iters; ++k) {
    const float* Hc = a.H[cur];
    // ---- A: recurrent product, cell, filter chunk maps ----
    uint32_t m = 0;
    for (int task = gw; task < ntask; task += nw) {
      const int b = task / nch, c = task - b * nch;
      const int t0 = c * kEChunk, len = min(kEChunk, T - t0);
      const size_t base = (size_t)b * T * D + lane;
      const float* gxb = a.gx + (size_t)b * T * 3 * D + lane;
      // every load of the chunk first (rows clamped into it)
      float hv[kEChunk], xg[kEChunk][3];
      float hp = 0.f;
      if (act) {
#pragma unroll
        for (int u = 0; u < kEChunk; ++u) {
          const int t = t0 + min(u, len - 1);
          hv[u] = Hc[base + (size_t)t * D];
#pragma unroll
          for (int g = 0; g < 3; ++g) xg[u][g] = gxb[(size_t)t * 3 * D + g * D];
        }
        hp = t0 == 0 ? (a.h0 ? a.h0[(size_t)b * D + lane] : 0.f) : a.hb[(size_t)task * D + lane];
      } else {
#pragma unroll
        for (int u = 0; u < kEChunk; ++u) {
          hv[u] = 0.f;
          xg[u][0] = xg[u][1] = xg[u][2] = 0.f;
        }
      }
      // row u of the A operand: h_{t0+u-1} over the 64 (padded) channels
#pragma unroll
      for (int u = 0; u < kEChunk; ++u) st[u * kStLd + lane] = u == 0 ? hp : hv[u - 1];
      wave_lds_sync();
      // lane l ends with gh[row 4 (l / 16) + i][column 16 nt + l % 16], column = 64 g + c
      v4f_t acc[12];
#pragma unroll
      for (int nt = 0; nt < 12; ++nt) acc[nt] = v4f_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
      for (int kk = 0; kk < 16; ++kk) {
        const float av = st[m16 * kStLd + 4 * kk + q4];
#pragma unroll
        for (int nt = 0; nt < 12; ++nt)
          acc[nt] = __builtin_amdgcn_mfma_f32_16x16x4f32(av, uf[kk][nt][lane], acc[nt], 0, 0, 0);
      }
      wave_lds_sync();   // every read of the staged rows before they are overwritten
#pragma unroll
      for (int nt = 0; nt < 12; ++nt)
#pragma unroll
        for (int i = 0; i < 4; ++i) st[(4 * q4 + i) * kGhLd + 16 * nt + m16] = acc[nt][i];
      wave_lds_sync();
      // the cell and the filter map, lane = channel
      Flt F = flt_identity();
      if (act) {
#pragma unroll
        for (int u = 0; u < kEChunk; ++u) {
          if (u < len) {
            const float ghr = st[u * kGhLd + lane] + bhv[0];
            const float ghz = st[u * kGhLd + 64 + lane] + bhv[1];
            const float ghn = st[u * kGhLd + 128 + lane] + bhv[2];
            const float r = sigm(xg[u][0] + ghr);
            const float z = sigm(xg[u][1] + ghz);
            const float nn = tanh_(fmaf(r, ghn, xg[u][2]));
            const float p = u == 0 ? hp : hv[u - 1];
            const float res = fmaf(z, p - nn, nn) - hv[u];
            const float fz = (p - nn) * z * (1.f - z);
            const float fn = (1.f - z) * (1.f - nn * nn);
            const float jj = z + fz * ud[1] + fn * r * ud[2] + fn * ghn * r * (1.f - r) * ud[0];
            const size_t e = base + (size_t)(t0 + u) * D;
            a.R[e] = res;
            a.J[e] = jj;
            m = max(m, abs_bits(res));
            F = compose(filter_step(jj, res, lam), F);
            if (u == 0) {
              float* hd = a.head + (size_t)task * 3 * D + lane;
              coherent_store(hd, jj);
              coherent_store(hd + D, res);
              coherent_store(hd + 2 * D, hv[0]);
            }
          }
        }
        float* ag = a.agg + (((size_t)b * D + lane) * nch + c) * 8;
        coherent_store(ag, F.a);
        coherent_store(ag + 1, F.b);
        coherent_store(ag + 2, F.c);
        coherent_store(ag + 3, F.d);
        coherent_store(ag + 4, F.e);
        coherent_store(ag + 5, F.f);
        coherent_store(ag + 6, F.g);
      }
      wave_lds_sync();   // the transposed rows are read before the next chunk stages its own
    }
    m = wave_max_u32(m);
    if (lane == 0) s_wmax[wid] = m;
    __syncthreads();
    if (tid == 0) {
      uint32_t bm = s_wmax[0];
      for (int w = 1; w < kElkWaves; ++w) bm = max(bm, s_wmax[w]);
      __hip_atomic_store(&a.partials[blockIdx.x], bm, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    grid_barrier(ctrl, [&]() {
      uint32_t mm = 0;
      for (int i = tid; i < (int)gridDim.x; i += 64 * kElkWaves)
        mm = max(mm, __hip_atomic_load(&a.partials[i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
      mm = wave_max_u32(mm);
      __syncthreads();
      if (lane == 0) s_wmax[wid] = mm;
      __syncthreads();
      if (tid == 0) {
        for (int w = 0; w < kElkWaves; ++w) mm = max(mm, s_wmax[w]);
        finish_iteration(ctrl, a.hist, bits_to_rho(mm), k, cur, a.max_iters, a.tol);
      }
    });
    if (__hip_atomic_load(&ctrl->done, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) || has_fault(ctrl)) break;

    // ---- B: filter state (u, 1, n) entering each chunk; lane order = time ----
    for (int task = gw; task < nrow; task += nw) {
      const int b = task / D, i = task - b * D;
      const float* ag = a.agg + ((size_t)b * D + i) * nch * 8;
      V3 x{0.f, 1.f, 0.f};   // entering the first chunk: P = 0, m = 0
      for (int h0 = 0; h0 < nch; h0 += 64 * kCarryGroups) {
        Flt F[kCarryGroups];
#pragma unroll
        for (int h = 0; h < kCarryGroups; ++h) {
          const int c = h0 + 64 * h + lane;
          F[h] = flt_identity();
          if (c < nch) {
            const float* p = ag + (size_t)c * 8;
            F[h] = Flt{coherent_load(p), coherent_load(p + 1), coherent_load(p + 2), coherent_load(p + 3),
                       coherent_load(p + 4), coherent_load(p + 5), coherent_load(p + 6)};
          }
        }
#pragma unroll
        for (int h = 0; h < kCarryGroups; ++h) {
          const int c = h0 + 64 * h + lane;
          Flt f = F[h];
#pragma unroll
          for (int off = 1; off < 64; off <<= 1) {
            const Flt prev = flt_shfl_up(f, off);
            if (lane >= off) f = compose(f, prev);
          }
          const Flt before = flt_shfl_up(f, 1);
          const V3 xin = lane == 0 ? x : normalized(apply(before, x));
          if (c < nch) {
            float* cp = a.carry + ((size_t)b * nch + c) * 2 * D + i;
            coherent_store(cp, xin.u);
            coherent_store(cp + D, xin.n);
          }
          x = normalized(apply(flt_shfl(f, 63), x));
        }
      }
    }
    grid_barrier(ctrl, [] {});
    if (has_fault(ctrl)) break;

    // ---- C: filter walk, smoother gain and offset, smoother chunk maps ----
    for (int task = gw; task < ntask; task += nw) {
      if (!act) continue;
      const int b = task / nch, c = task - b * nch;
      const int t0 = c * kEChunk, len = min(kEChunk, T - t0);
      const size_t base = (size_t)b * T * D + lane;
      float jv[kEChunk], rv[kEChunk], hv[kEChunk];
#pragma unroll
      for (int u = 0; u < kEChunk; ++u) {
        const size_t e = base + (size_t)(t0 + min(u, len - 1)) * D;
        jv[u] = a.J[e];
        rv[u] = a.R[e];
        hv[u] = Hc[e];
      }
      const float* cp = a.carry + (size_t)task * 2 * D + lane;
      V3 x{coherent_load(cp), 1.f, coherent_load(cp + D)};
      const bool tail = t0 + len < T;   // the next chunk exists
      float jt = 0.f, rt = 0.f, ht = 0.f;
      if (tail) {
        const float* hd = a.head + (size_t)(task + 1) * 3 * D + lane;
        jt = coherent_load(hd);
        rt = coherent_load(hd + D);
        ht = coherent_load(hd + 2 * D);
      }
      float SP = 1.f, SQ = 0.f;   // the chunk's smoother map h'_{t1} -> h'_{t0}, composed forwards
#pragma unroll
      for (int u = 0; u < kEChunk; ++u) {
        if (u < len) {
          x = normalized(apply(filter_step(jv[u], rv[u], lam), x));
          const float P = x.u, mm = x.n;
          const bool last = u == len - 1;
          float G = 0.f, e = mm + hv[u];
          if (!last || tail) {
            const float jn = last ? jt : jv[min(u + 1, kEChunk - 1)];
            const float rn = last ? rt : rv[min(u + 1, kEChunk - 1)];
            const float hn = last ? ht : hv[min(u + 1, kEChunk - 1)];
            G = P * jn * fast_rcp(fmaf(jn * jn, P, 1.f));
            e = (mm + hv[u]) - G * (fmaf(jn, mm, rn) + hn);
          }
          const size_t o = base + (size_t)(t0 + u) * D;
          a.G[o] = G;
          a.E[o] = e;
          SQ = fmaf(SP, e, SQ);
          SP *= G;
          if (last) {
            float* tg = a.tailge + (size_t)task * 2 * D + lane;
            coherent_store(tg, G);
            coherent_store(tg + D, e);
          }
        }
      }
      float* ag2 = a.agg2 + (((size_t)b * D + lane) * nch + c) * 2;
      coherent_store(ag2, SP);
      coherent_store(ag2 + 1, SQ);
    }
    grid_barrier(ctrl, [] {});
    if (has_fault(ctrl)) break;

    // ---- D: smoothed state at the step after each chunk; lane order = reverse time ----
    for (int task = gw; task < nrow; task += nw) {
      const int b = task / D, i = task - b * D;
      const float* ag2 = a.agg2 + ((size_t)b * D + i) * nch * 2;
      float x = 0.f;   // after the last chunk: unused (the last step's gain is 0)
      for (int h0 = 0; h0 < nch; h0 += 64 * kCarryGroups) {
        float P[kCarryGroups], Q[kCarryGroups];
#pragma unroll
        for (int h = 0; h < kCarryGroups; ++h) {
          const int c = nch - 1 - (h0 + 64 * h + lane);
          P[h] = 1.f;
          Q[h] = 0.f;
          if (c >= 0) {
            P[h] = coherent_load(ag2 + (size_t)c * 2);
            Q[h] = coherent_load(ag2 + (size_t)c * 2 + 1);
          }
        }
#pragma unroll
        for (int h = 0; h < kCarryGroups; ++h) {
          const int c = nch - 1 - (h0 + 64 * h + lane);
          float p_ = P[h], q_ = Q[h];
#pragma unroll
          for (int off = 1; off < 64; off <<= 1) {
            const float pp = __shfl_up(p_, off, 64), pq = __shfl_up(q_, off, 64);
            if (lane >= off) {
              q_ = fmaf(p_, pq, q_);
              p_ *= pp;
            }
          }
          const float pp = __shfl_up(p_, 1, 64), pq = __shfl_up(q_, 1, 64);
          const float xin = lane == 0 ? x : fmaf(pp, x, pq);
          if (c >= 0) coherent_store(a.carry2 + ((size_t)b * nch + c) * D + i, xin);
          x = fmaf(__shfl(p_, 63, 64), x, __shfl(q_, 63, 64));
        }
      }
    }
    grid_barrier(ctrl, [] {});
    if (has_fault(ctrl)) break;

    // ---- E: smoother walk, the next iterate, and the state before the chunk ----
    float* Hn = a.H[cur ^ 1];
    for (int task = gw; task < ntask; task += nw) {
      if (!act) continue;
      const int b = task / nch, c = task - b * nch;
      const int t0 = c * kEChunk, len = min(kEChunk, T - t0);
      const size_t base = (size_t)b * T * D + lane;
      float gv[kEChunk], ev[kEChunk];
#pragma unroll
      for (int u = 0; u < kEChunk; ++u) {
        const size_t e = base + (size_t)(t0 + min(u, len - 1)) * D;
        gv[u] = a.G[e];
        ev[u] = a.E[e];
      }
      float x = coherent_load(a.carry2 + (size_t)task * D + lane);
      float gl = 0.f, el = 0.f;
      if (c > 0) {
        const float* tg = a.tailge + (size_t)(task - 1) * 2 * D + lane;
        gl = coherent_load(tg);
        el = coherent_load(tg + D);
      }
#pragma unroll
      for (int u = kEChunk - 1; u >= 0; --u) {
        if (u < len) {
          x = fmaf(gv[u], x, ev[u]);
          Hn[base + (size_t)(t0 + u) * D] = x;
        }
      }
      if (c > 0) a.hb[(size_t)task * D + lane] = fmaf(gl, x, el);
    }
    cur ^= 1;
  }
}

// The returned iterate (the buffer the loop's decision names) into the caller's output.
__global__ void __launch_bounds__(256) elk_dense_output_kernel(const float* __restrict__ H0,
                                                               const float* __restrict__ H1,
                                                               const Ctrl* __restrict__ ctrl, float* __restrict__ out,
                                                               size_t n, bool vec) {
  const float* src = ctrl->result_buf == 1 ? H1 : H0;
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (vec) {
    for (; i < n / 4; i += stride) reinterpret_cast<float4*>(out)[i] = reinterpret_cast<const float4*>(src)[i];
  } else {
    for (; i < n; i += stride) out[i] = src[i];
  }
}

hipError_t launch_elk_dense_output(const float* H0, const float* H1, const Ctrl* ctrl, float* out, size_t n,
                                   hipStream_t st) {
  if (n == 0) return hipSuccess;
  const bool vec = n % 4 == 0 && (reinterpret_cast<uintptr_t>(out) | reinterpret_cast<uintptr_t>(H0) |
                                  reinterpret_cast<uintptr_t>(H1)) % 16 == 0;
  const size_t items = vec ? n / 4 : n;
  size_t blocks = (items + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(elk_dense_output_kernel, dim3((unsigned)blocks), dim3(256), 0, st, H0, H1, ctrl, out, n, vec);
  return hipGetLastError();
}

hipError_t launch_gru_elk_loop(const ElkLoopArgs& a, int num_cu, hipStream_t st) {
  if (a.D > 64 || a.D < 1) return hipErrorInvalidValue;
  constexpr int threads = 64 * kElkWaves;
  const int per_cu = cached_occupancy((const void*)gru_elk_loop_kernel, 0, threads);
  if (per_cu < 1) return hipErrorInvalidConfiguration;
  long g = (long)per_cu * num_cu;
  if (g > kMaxGrid) g = kMaxGrid;
  const long work = ((long)a.B * a.nch + kElkWaves - 1) / kElkWaves;
  if (g > work) g = work;
  if (g < 1) g = 1;
  void* args[] = {const_cast<ElkLoopArgs*>(&a)};
  return launch_persistent((const void*)gru_elk_loop_kernel, (int)g, 0, args, st, threads);
}

}  // namespace pnr
