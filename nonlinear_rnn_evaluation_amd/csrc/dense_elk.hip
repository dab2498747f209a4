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
constexpr int kWaveLds = 3 * 64 * kEChunk;  // per wave: the staged rows, then gh transposed
static_assert(kEChunk * kStLd <= kWaveLds, "staged rows fit the per-wave buffer");
typedef float v4f_t __attribute__((ext_vector_type(4)));

int elk_dense_chunks(int T) { return (T + kEChunk - 1) / kEChunk; }

__device__ __forceinline__ Flt filter_step(float j, float r, float lam) {
  const float j2 = j * j;
  return Flt{j2, 1.f, lam * j2, 1.f + lam, 0.f, r, j};
}
// the rows this wave just wrote to LDS are read back by every lane of the wave
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
  __builtin_amdgcn_wave_barrier();
}

// A chunk's per-step values in one wave's registers (lane = channel).
struct ChunkRegs {
  float xg[kEChunk][3];   // gate inputs x W^T + b_x
  float hv[kEChunk];      // the iterate
  float hp;               // the state before the chunk's first step
  float jv[kEChunk];      // quasi Jacobian (cell -> filter)
  float rv[kEChunk];      // residual (cell -> filter)
  float gv[kEChunk];      // smoother gain (filter -> smoother)
  float ev[kEChunk];      // smoother offset (filter -> smoother)
};

// RES: every chunk has a wave of its own (B * nch <= waves of the grid), and the chunk's
// per-step values stay in that wave's registers for the whole launch; the iterate is still
// written out every iteration (the last one written is the result).  Otherwise a wave
// loops over its chunks and keeps those values in the workspace planes.
// Every array of a ChunkRegs is assigned in full by the phase that produces it (rows past
// a ragged chunk's end and lanes past D compute on clamped, finite inputs, and only their
// side effects are masked), so each value is live only from its producer to its consumer.
template <bool RES>
__global__ void __launch_bounds__(64 * kElkWaves, 1) gru_elk_loop_kernel(ElkLoopArgs a) {
  // One pool, the operand table first (so that every read of it is a base register plus an
  // immediate offset below 64 KiB):
  //  ufv[kk][l][nt] = U_g[c][j], g = nt / 4, c = 16 (nt % 4) + l % 16, j = 16 (l / 16) + kk
  //    (zero past D): the B operands of k-step kk for lane l, 12 column tiles, read as three
  //    16-byte vectors (a lane stride of 48 bytes: 16 lanes cover the 64 banks once);
  //  then per wave the staged h_{t-1} rows [16][kStLd] (MFMA A operand), and over them gh
  //    transposed [3][64][16].
  // The k index is split across lane groups (k = 16 (l / 16) + kk in k-step kk), so a lane's
  // A operands for all 16 k-steps are 16 consecutive floats of its row.
  __shared__ __align__(16) float pool[16 * 64 * 12 + kElkWaves * kWaveLds];
  float* const ufv = pool;
  __shared__ uint32_t s_wmax[kElkWaves];
  __shared__ uint32_t s_rbits;
  __shared__ Flt s_tot[kElkWaves];       // carry scans: each wave's group total
  __shared__ float2 s_tot2[kElkWaves];
  // the wave index is uniform across the wave: saying so keeps every chunk index and base
  // address derived from it in scalar registers
  const int lane = threadIdx.x & 63, wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), tid = threadIdx.x;
  const int D = a.D, T = a.T, nch = a.nch;
  // carry scans: groups of 64 chunks per row, waves per row (a power of two up to 8), rows per block
  const int ngr = (nch + 63) / 64;
  const int wpr = ngr >= 8 ? 8 : ngr > 2 ? 4 : ngr;
  const int rpb = kElkWaves / wpr;
  const bool act = lane < D;
  const int ln = act ? lane : 0;   // the channel whose addresses a lane uses
  const float lam = a.lam;
  Ctrl* ctrl = a.ctrl;
  for (int idx = tid; idx < 16 * 64 * 12; idx += 64 * kElkWaves) {
    const int kk = idx / (64 * 12), l = (idx / 12) & 63, nt = idx % 12;
    const int g = nt >> 2, c = 16 * (nt & 3) + (l & 15), j = 16 * (l >> 4) + kk;
    ufv[idx] = (c < D && j < D) ? a.U[(size_t)(g * D + c) * D + j] : 0.f;
  }
  // per lane (channel): the diagonals U_r[i][i], U_z[i][i], U_n[i][i] and b_h
  float ud[3], bhv[3];
#pragma unroll
  for (int g = 0; g < 3; ++g) {
    ud[g] = a.U[(size_t)(g * D + ln) * D + ln];
    bhv[g] = a.bh ? a.bh[g * D + ln] : 0.f;
  }
  __syncthreads();
  const int gw = blockIdx.x * kElkWaves + wid, nw = gridDim.x * kElkWaves;
  const int ntask = a.B * nch, nrow = a.B * D;
  float* st = pool + 16 * 64 * 12 + wid * kWaveLds;
  const int m16 = lane & 15, q4 = lane >> 4;

  // per-step gate inputs, iterate (from Hc) and the state before the chunk
  auto load_inputs = [&](ChunkRegs& r, int task, const float* Hc) {
    const int b = task / nch, c = task - b * nch;
    const int t0 = c * kEChunk, len = min(kEChunk, T - t0);
    const size_t base = (size_t)b * T * D + ln;
    const float* gxb = a.gx + (size_t)b * T * 3 * D + ln;
#pragma unroll
    for (int u = 0; u < kEChunk; ++u) {
      const int t = t0 + min(u, len - 1);
      r.hv[u] = Hc ? Hc[base + (size_t)t * D] : 0.f;
#pragma unroll
      for (int g = 0; g < 3; ++g) r.xg[u][g] = gxb[(size_t)t * 3 * D + g * D];
    }
    const float h0v = a.h0 ? a.h0[(size_t)b * D + ln] : 0.f;
    r.hp = t0 == 0 ? h0v : (Hc ? a.hb[(size_t)task * D + ln] : 0.f);
  };

  // A: recurrent product, cell, the chunk's filter map; max |R| into m
  auto phase_a = [&](ChunkRegs& r, int task, bool valid, uint32_t& m) {
    const int b = task / nch, c = task - b * nch;
    const int t0 = c * kEChunk, len = min(kEChunk, T - t0);
    const size_t base = (size_t)b * T * D + ln;
    // row u of the A operand: h_{t0+u-1} over the 64 (padded) channels
#pragma unroll
    for (int u = 0; u < kEChunk; ++u) st[u * kStLd + lane] = act ? (u == 0 ? r.hp : r.hv[u - 1]) : 0.f;
    wave_lds_sync();
    // lane l ends with gh[row 4 (l / 16) + i][column 16 nt + l % 16], column = 64 g + c
    v4f_t acc[12];
#pragma unroll
    for (int nt = 0; nt < 12; ++nt) acc[nt] = v4f_t{0.f, 0.f, 0.f, 0.f};
    float4 av[4];
    const float4* arow = reinterpret_cast<const float4*>(st + m16 * kStLd + 16 * q4);
#pragma unroll
    for (int j = 0; j < 4; ++j) av[j] = arow[j];
    const float4* ub = reinterpret_cast<const float4*>(ufv) + lane * 3;
    float4 bcur[3], bnxt[3];
#pragma unroll
    for (int j = 0; j < 3; ++j) bcur[j] = ub[j];
#pragma unroll
    for (int kk = 0; kk < 16; ++kk) {
      if (kk + 1 < 16) {
#pragma unroll
        for (int j = 0; j < 3; ++j) bnxt[j] = ub[(kk + 1) * 192 + j];
      }
      const float4 a4 = av[kk >> 2];
      const float aval = (kk & 3) == 0 ? a4.x : (kk & 3) == 1 ? a4.y : (kk & 3) == 2 ? a4.z : a4.w;
      const float bvals[12] = {bcur[0].x, bcur[0].y, bcur[0].z, bcur[0].w, bcur[1].x, bcur[1].y,
                               bcur[1].z, bcur[1].w, bcur[2].x, bcur[2].y, bcur[2].z, bcur[2].w};
#pragma unroll
      for (int nt = 0; nt < 12; ++nt)
        acc[nt] = __builtin_amdgcn_mfma_f32_16x16x4f32(aval, bvals[nt], acc[nt], 0, 0, 0);
      if (kk + 1 < 16) {
#pragma unroll
        for (int j = 0; j < 3; ++j) bcur[j] = bnxt[j];
      }
    }
    wave_lds_sync();   // every read of the staged rows before they are overwritten
    // gh transposed to [gate][channel][16 steps] (4-step groups XOR-swizzled by bits 2..3
    // of the channel: the 16-byte writes below and the reads after them are conflict-free)
    float4* gt = reinterpret_cast<float4*>(st);
#pragma unroll
    for (int nt = 0; nt < 12; ++nt)
      gt[((nt >> 2) * 64 + 16 * (nt & 3) + m16) * 4 + (q4 ^ (m16 >> 2))] =
          make_float4(acc[nt][0], acc[nt][1], acc[nt][2], acc[nt][3]);
    wave_lds_sync();
    const int sw = (lane >> 2) & 3;
    // this lane's channel: gh of the three gates for steps 4j..4j+3, the next group's
    // loads issued before the current group is used
    float4 gcur[3], gnxt[3];
#pragma unroll
    for (int g = 0; g < 3; ++g) gcur[g] = gt[(g * 64 + lane) * 4 + sw];
    // the cell and the filter map, lane = channel; every step is computed (rows past a
    // ragged end on clamped inputs) and only steps < len enter the map and the maximum
    const bool live = valid && act;
    Flt F = flt_identity();
    uint32_t mloc = 0;
#pragma unroll
    for (int u = 0; u < kEChunk; ++u) {
      if ((u & 3) == 0 && u + 4 < kEChunk) {
#pragma unroll
        for (int g = 0; g < 3; ++g) gnxt[g] = gt[(g * 64 + lane) * 4 + (((u >> 2) + 1) ^ sw)];
      }
      const float4 g0 = gcur[0], g1 = gcur[1], g2 = gcur[2];
      const int i = u & 3;
      const float ghr = (i == 0 ? g0.x : i == 1 ? g0.y : i == 2 ? g0.z : g0.w) + bhv[0];
      const float ghz = (i == 0 ? g1.x : i == 1 ? g1.y : i == 2 ? g1.z : g1.w) + bhv[1];
      const float ghn = (i == 0 ? g2.x : i == 1 ? g2.y : i == 2 ? g2.z : g2.w) + bhv[2];
      const float rr = sigm(r.xg[u][0] + ghr);
      const float z = sigm(r.xg[u][1] + ghz);
      const float nn = tanh_(fmaf(rr, ghn, r.xg[u][2]));
      const float p = u == 0 ? r.hp : r.hv[u - 1];
      const float res = fmaf(z, p - nn, nn) - r.hv[u];
      const float fz = (p - nn) * z * (1.f - z);
      const float fn = (1.f - z) * (1.f - nn * nn);
      const float jj = z + fz * ud[1] + fn * rr * ud[2] + fn * ghn * rr * (1.f - rr) * ud[0];
      r.jv[u] = jj;
      r.rv[u] = res;
      const bool in = u < len;
      const Flt Fn = compose(filter_step(jj, res, lam), F);
      F = Flt{in ? Fn.a : F.a, in ? Fn.b : F.b, in ? Fn.c : F.c, in ? Fn.d : F.d,
              in ? Fn.e : F.e, in ? Fn.f : F.f, in ? Fn.g : F.g};
      mloc = in ? max(mloc, abs_bits(res)) : mloc;
      if ((u & 3) == 3 && u + 1 < kEChunk) {
#pragma unroll
        for (int g = 0; g < 3; ++g) gcur[g] = gnxt[g];
      }
    }
    if (live) {
      m = max(m, mloc);
      if constexpr (!RES) {
#pragma unroll
        for (int u = 0; u < kEChunk; ++u) {
          if (u < len) {
            const size_t e = base + (size_t)(t0 + u) * D;
            a.R[e] = r.rv[u];
            a.J[e] = r.jv[u];
          }
        }
      }
      float* hd = a.head + (size_t)task * 3 * D + lane;
      coherent_store(hd, r.jv[0]);
      coherent_store(hd + D, r.rv[0]);
      coherent_store(hd + 2 * D, r.hv[0]);
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
  };

  // C: filter walk from the chunk's entering state, smoother gain and offset, the chunk's
  // smoother map
  auto phase_c = [&](ChunkRegs& r, int task, bool valid) {
    const int b = task / nch, c = task - b * nch;
    const int t0 = c * kEChunk, len = min(kEChunk, T - t0);
    const size_t base = (size_t)b * T * D + ln;
    const bool live = valid && act;
    const float* cp = a.carry + (size_t)task * 2 * D + ln;
    V3 x{coherent_load(cp), 1.f, coherent_load(cp + D)};
    const bool tail = t0 + len < T;   // the next chunk exists
    float jt = 0.f, rt = 0.f, ht = 0.f;
    if (tail) {
      const float* hd = a.head + (size_t)(task + 1) * 3 * D + ln;
      jt = coherent_load(hd);
      rt = coherent_load(hd + D);
      ht = coherent_load(hd + 2 * D);
    }
    float SP = 1.f, SQ = 0.f;   // the chunk's smoother map h'_{t1} -> h'_{t0}, composed forwards
#pragma unroll
    for (int u = 0; u < kEChunk; ++u) {
      x = normalized(apply(filter_step(r.jv[u], r.rv[u], lam), x));
      const float P = x.u, mm = x.n;
      const bool last = u == len - 1;
      const bool has_next = !last || tail;
      const float jn = last ? jt : r.jv[min(u + 1, kEChunk - 1)];
      const float rn = last ? rt : r.rv[min(u + 1, kEChunk - 1)];
      const float hn = last ? ht : r.hv[min(u + 1, kEChunk - 1)];
      const float G = has_next ? P * jn * fast_rcp(fmaf(jn * jn, P, 1.f)) : 0.f;
      const float e = has_next ? (mm + r.hv[u]) - G * (fmaf(jn, mm, rn) + hn) : mm + r.hv[u];
      r.gv[u] = G;
      r.ev[u] = e;
      if (u < len) {
        SQ = fmaf(SP, e, SQ);
        SP *= G;
        if (live) {
          if constexpr (!RES) {
            const size_t o = base + (size_t)(t0 + u) * D;
            a.G[o] = G;
            a.E[o] = e;
          }
          if (last) {
            float* tg = a.tailge + (size_t)task * 2 * D + lane;
            coherent_store(tg, G);
            coherent_store(tg + D, e);
          }
        }
      }
    }
    if (live) {
      float* ag2 = a.agg2 + (((size_t)b * D + lane) * nch + c) * 2;
      coherent_store(ag2, SP);
      coherent_store(ag2 + 1, SQ);
    }
  };

  // E: smoother walk from the smoothed state after the chunk: the next iterate, and the
  // state before the chunk from the predecessor's last gain and offset
  auto phase_e = [&](ChunkRegs& r, int task, bool valid, float* Hn) {
    const int b = task / nch, c = task - b * nch;
    const int t0 = c * kEChunk, len = min(kEChunk, T - t0);
    const size_t base = (size_t)b * T * D + ln;
    const bool live = valid && act;
    float x = coherent_load(a.carry2 + (size_t)task * D + ln);
    float gl = 0.f, el = 0.f;
    if (c > 0) {
      const float* tg = a.tailge + (size_t)(task - 1) * 2 * D + ln;
      gl = coherent_load(tg);
      el = coherent_load(tg + D);
    }
#pragma unroll
    for (int u = kEChunk - 1; u >= 0; --u) {
      if (u < len) {
        x = fmaf(r.gv[u], x, r.ev[u]);
        if (live) Hn[base + (size_t)(t0 + u) * D] = x;
      }
      r.hv[u] = x;
    }
    const float hb = c > 0 ? fmaf(gl, x, el) : r.hp;
    if constexpr (RES) r.hp = hb;
    else if (live && c > 0) a.hb[(size_t)task * D + lane] = hb;
  };

  // the per-step planes of a chunk, for the looping variant
  auto load_planes_c = [&](ChunkRegs& r, int task, const float* Hc) {
    const int b = task / nch, c = task - b * nch;
    const int t0 = c * kEChunk, len = min(kEChunk, T - t0);
    const size_t base = (size_t)b * T * D + ln;
#pragma unroll
    for (int u = 0; u < kEChunk; ++u) {
      const size_t e = base + (size_t)(t0 + min(u, len - 1)) * D;
      r.jv[u] = a.J[e];
      r.rv[u] = a.R[e];
      r.hv[u] = Hc[e];
    }
  };
  auto load_planes_e = [&](ChunkRegs& r, int task) {
    const int b = task / nch, c = task - b * nch;
    const int t0 = c * kEChunk, len = min(kEChunk, T - t0);
    const size_t base = (size_t)b * T * D + ln;
#pragma unroll
    for (int u = 0; u < kEChunk; ++u) {
      const size_t e = base + (size_t)(t0 + min(u, len - 1)) * D;
      r.gv[u] = a.G[e];
      r.ev[u] = a.E[e];
    }
    r.hp = 0.f;
  };

  // RES: the wave's one chunk (a wave past the last chunk repeats it with its effects masked)
  const int rtask = min(gw, ntask - 1);
  const bool rvalid = gw < ntask;
  ChunkRegs rr;
  if constexpr (RES) load_inputs(rr, rtask, nullptr);   // the zero guess

  int cur = 0;
  uint32_t gen = 0;   // generation of the next grid barrier
  for (int k = 0; k <= a.max_iters; ++k) {
    const float* Hc = a.H[cur];
    // ---- A ----
    uint32_t m = 0;
    if constexpr (RES) {
      phase_a(rr, rtask, rvalid, m);
    } else {
      for (int task = gw; task < ntask; task += nw) {
        ChunkRegs r;
        load_inputs(r, task, Hc);
        phase_a(r, task, true, m);
      }
    }
    // max |R| of the block into this iteration's word; after the barrier every block reads
    // it and takes the same decision (stop when rho_k <= tol, on a non-finite rho, or
    // after max_iters updates), which block 0 records
    m = wave_max_u32(m);
    if (lane == 0) s_wmax[wid] = m;
    __syncthreads();
    if (tid == 0) {
      uint32_t bm = s_wmax[0];
      for (int w = 1; w < kElkWaves; ++w) bm = max(bm, s_wmax[w]);
      if (bm) __hip_atomic_fetch_max(&a.rmax[k], bm, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    if (!grid_sync(ctrl, gen)) break;
    // the word is read here and the decision taken after B, so that its round trip overlaps
    // B (whose writes are harmless when the loop stops)
    uint32_t rbits = 0;
    if (tid == 0) rbits = __hip_atomic_load(&a.rmax[k], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);

    // ---- B: filter state (u, 1, n) entering each chunk; lane order = time ----
    // A row (b, channel) has ngr groups of 64 chunks; wpr waves of a block take wpr
    // consecutive groups at once, scan them in registers, and exchange the group totals
    // through LDS (every wave forms the same entering state from them).
    for (int r0 = blockIdx.x * rpb; r0 < nrow; r0 += gridDim.x * rpb) {
      const int row = r0 + wid / wpr, sub = wid % wpr;
      const bool live = row < nrow;
      const int b = live ? row / D : 0, i = live ? row - b * D : 0;
      const float* ag = a.agg + ((size_t)b * D + i) * nch * 8;
      V3 x{0.f, 1.f, 0.f};   // entering the row's first chunk: P = 0, m = 0
      for (int g0 = 0; g0 < ngr; g0 += wpr) {
        const int c = (g0 + sub) * 64 + lane;
        Flt f = flt_identity();
        if (live && c < nch) {
          const float* p = ag + (size_t)c * 8;
          f = Flt{coherent_load(p), coherent_load(p + 1), coherent_load(p + 2), coherent_load(p + 3),
                  coherent_load(p + 4), coherent_load(p + 5), coherent_load(p + 6)};
        }
        f = wave_inclusive_scan(f, flt_identity());
        if (lane == 63) s_tot[wid] = f;
        __syncthreads();
        V3 xg = x;   // entering this wave's group
        for (int s2 = wid - sub; s2 < wid; ++s2) xg = normalized(apply(s_tot[s2], xg));
        const Flt before = flt_wave_shr1(f, flt_identity());
        const V3 xin = lane == 0 ? xg : normalized(apply(before, xg));
        if (live && c < nch) {
          float* cp = a.carry + ((size_t)b * nch + c) * 2 * D + i;
          coherent_store(cp, xin.u);
          coherent_store(cp + D, xin.n);
        }
        for (int s2 = wid - sub; s2 < wid - sub + wpr; ++s2) x = normalized(apply(s_tot[s2], x));
        __syncthreads();   // the totals are read before the next round writes them
      }
    }
    if (tid == 0) s_rbits = rbits;
    if (!grid_sync(ctrl, gen)) break;   // (its closing block-wide sync publishes s_rbits)
    {
      const double rho = bits_to_rho(s_rbits);
      if (blockIdx.x == 0 && tid == 0) finish_iteration(ctrl, a.hist, rho, k, cur, a.max_iters, a.tol);
      if (!(rho < __builtin_inf()) || rho <= a.tol || k >= a.max_iters) break;
    }

    // ---- C ----
    if constexpr (RES) {
      phase_c(rr, rtask, rvalid);
    } else {
      for (int task = gw; task < ntask; task += nw) {
        ChunkRegs r;
        load_planes_c(r, task, Hc);
        phase_c(r, task, true);
      }
    }
    if (!grid_sync(ctrl, gen)) break;

    // ---- D: smoothed state at the step after each chunk; lane order = reverse time ----
    // (the same split of a row over wpr waves as in B)
    for (int r0 = blockIdx.x * rpb; r0 < nrow; r0 += gridDim.x * rpb) {
      const int row = r0 + wid / wpr, sub = wid % wpr;
      const bool live = row < nrow;
      const int b = live ? row / D : 0, i = live ? row - b * D : 0;
      const float* ag2 = a.agg2 + ((size_t)b * D + i) * nch * 2;
      float x = 0.f;   // after the row's last chunk: unused (the last step's gain is 0)
      for (int g0 = 0; g0 < ngr; g0 += wpr) {
        const int c = nch - 1 - ((g0 + sub) * 64 + lane);
        float p_ = 1.f, q_ = 0.f;
        if (live && c >= 0) {
          p_ = coherent_load(ag2 + (size_t)c * 2);
          q_ = coherent_load(ag2 + (size_t)c * 2 + 1);
        }
        const Aff1 f = wave_inclusive_scan(Aff1{p_, q_}, aff_identity1());
        if (lane == 63) s_tot2[wid] = make_float2(f.a, f.b);
        __syncthreads();
        float xg = x;   // after this wave's group
        for (int s2 = wid - sub; s2 < wid; ++s2) xg = fmaf(s_tot2[s2].x, xg, s_tot2[s2].y);
        const Aff1 before = aff_wave_shr1(f, aff_identity1());
        const float xin = fmaf(before.a, xg, before.b);
        if (live && c >= 0) coherent_store(a.carry2 + ((size_t)b * nch + c) * D + i, xin);
        for (int s2 = wid - sub; s2 < wid - sub + wpr; ++s2) x = fmaf(s_tot2[s2].x, x, s_tot2[s2].y);
        __syncthreads();
      }
    }
    if (!grid_sync(ctrl, gen)) break;

    // ---- E ----
    float* Hn = a.H[cur ^ 1];
    if constexpr (RES) {
      phase_e(rr, rtask, rvalid, Hn);
    } else {
      for (int task = gw; task < ntask; task += nw) {
        ChunkRegs r;
        load_planes_e(r, task);
        phase_e(r, task, true, Hn);
      }
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
  const int per_cu = min(cached_occupancy((const void*)gru_elk_loop_kernel<true>, 0, threads),
                         cached_occupancy((const void*)gru_elk_loop_kernel<false>, 0, threads));
  if (per_cu < 1) return hipErrorInvalidConfiguration;
  long g = (long)per_cu * num_cu;
  if (g > kMaxGrid) g = kMaxGrid;
  const long ntask = (long)a.B * a.nch;
  const long work = (ntask + kElkWaves - 1) / kElkWaves;
  const bool res = work <= g;   // a wave per chunk
  if (g > work) g = work;
  if (g < 1) g = 1;
  void* args[] = {const_cast<ElkLoopArgs*>(&a)};
  const void* fn = res ? (const void*)gru_elk_loop_kernel<true> : (const void*)gru_elk_loop_kernel<false>;
  return launch_persistent(fn, (int)g, 0, args, st, threads);
}

}  // namespace pnr
