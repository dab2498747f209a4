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
#include <cstdlib>

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

// Stage rows s = 0..TL of the tile: row s holds the state before step t0+s.  Rows 1..TL
// are this block's own states of the pass before: plain loads, every load of a batch
// issued before any is used (addresses clamped into the sequence, values past its end
// replaced afterwards), so a batch costs one memory round trip.  Row 0 is the previous
// tile's last step, written by another block: threads tid < D read it coherently.
template <int TL = kTL>
__device__ __forceinline__ void stage_rows(float* __restrict__ X, const float* __restrict__ H,
                                           const float* __restrict__ h0, int b, int t0, int T, int D,
                                           int LD) {
  const int tid = threadIdx.x;
  const int n = (TL + 1) * D;
  for (int j0 = D; j0 < n; j0 += kLoadBatch * PNR_BLOCK) {
    float v[kLoadBatch];
#pragma unroll
    for (int j = 0; j < kLoadBatch; ++j) v[j] = 0.f;
    if (H) {
#pragma unroll
      for (int j = 0; j < kLoadBatch; ++j) {
        const int idx = min(j0 + tid + j * PNR_BLOCK, n - 1);
        const int s = idx / D, c = idx - s * D, t = min(t0 + s - 1, T - 1);
        v[j] = H[((size_t)b * T + t) * D + c];
      }
    }
#pragma unroll
    for (int j = 0; j < kLoadBatch; ++j) {
      const int idx = j0 + tid + j * PNR_BLOCK;
      if (idx < n) {
        const int s = idx / D, c = idx - s * D;
        X[s * LD + c] = t0 + s - 1 < T ? v[j] : 0.f;
      }
    }
  }
  if (tid < D) {
    const int t = t0 - 1;
    X[tid] = t < 0 ? (h0 ? h0[(size_t)b * D + tid] : 0.f)
                   : (H ? coherent_load(H + ((size_t)b * T + t) * D + tid) : 0.f);
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

// The same product with the K index split so that, in MFMA kk, lane group q = lane/16
// contributes k = q*(D/4) + kk: a lane's A operands for one 16-step block are then D/4
// consecutive floats of one LDS row, read as D/16 vectors before the MFMA chain starts.
// The B fragments must follow the same split: ufp[g][kk] = U_g[c][q*(D/4) + kk].
template <int DM>
__device__ __forceinline__ void load_afrag(const float* __restrict__ X, int LD, int tb, v4f (&f)[DM / 16]) {
  const int l = (int)lane_id();
  const v4f* p = reinterpret_cast<const v4f*>(X + (size_t)(tb * 16 + (l & 15)) * LD + (l >> 4) * (DM / 4));
#pragma unroll
  for (int j = 0; j < DM / 16; ++j) f[j] = p[j];
}
template <int DM>
__device__ __forceinline__ void gates_frag(const v4f (&f)[DM / 16], const float (&ufp)[3][DM / 4], v4f (&acc)[3]) {
#pragma unroll
  for (int g = 0; g < 3; ++g) acc[g] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int kk = 0; kk < DM / 4; ++kk) {
    const float av = f[kk >> 2][kk & 3];
#pragma unroll
    for (int g = 0; g < 3; ++g) acc[g] = mfma4(av, ufp[g][kk], acc[g]);
  }
}

// The pass's residual maximum into this iteration's word (the zeroed partials area), the
// lean grid barrier, then every block reads the word and takes the same decision (stop when
// rho_k <= tol, on a non-finite rho, or at the residual-only pass after max_iters), which
// block 0 records.  Returns true when the loop stops or this block's barrier wait ran out.
__device__ __forceinline__ bool end_pass(const DenseLoopArgs<float>& a, uint32_t blk_max, int k, int cur,
                                         uint32_t& gen) {
  __shared__ uint32_t s_wmax[PNR_WAVES];
  __shared__ uint32_t s_bits;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  uint32_t* word = reinterpret_cast<uint32_t*>(a.partials) + k;
  blk_max = wave_max_u32(blk_max);
  if (lane == 0) s_wmax[wid] = blk_max;
  __syncthreads();
  if (tid == 0) {
    uint32_t m = s_wmax[0];
    for (int w = 1; w < PNR_WAVES; ++w) m = max(m, s_wmax[w]);
    if (m) __hip_atomic_fetch_max(word, m, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  if (!grid_sync(a.ctrl, gen)) return true;
  if (tid == 0) s_bits = __hip_atomic_load(word, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  const double rho = bits_to_rho(s_bits);
  if (blockIdx.x == 0 && tid == 0) finish_iteration(a.ctrl, a.rho_hist, rho, k, cur, a.max_iters, a.tol);
  return !(rho < __builtin_inf()) || rho <= a.tol || k >= a.max_iters;
}

__device__ __forceinline__ int next_buffer(int cur, int jac, int nbuf) {
  for (int i = 0; i < nbuf; ++i)
    if (i != cur && i != jac) return i;
  return -1;
}

// Read up to Wn predecessor slots (SV values each, aggregate first) into Win and find
// the nearest predecessor with a published prefix whose successors (up to this tile)
// all published their aggregates.  Returns that window index, or -1.  Block-uniform.
// BATCH loads per thread are issued before any is used: with BATCH * PNR_BLOCK >= Wn * SV
// the whole window costs one memory round trip.
template <int BATCH = kLoadBatch>
__device__ __forceinline__ int window_read(const uint64_t* __restrict__ slots, int tile, int Wn, int SV, int SA,
                                           uint32_t ep, float* __restrict__ Win) {
  __shared__ int s_ok[16][2];
  __shared__ int s_p;
  const int tid = threadIdx.x;
  if (tid < Wn) { s_ok[tid][0] = 1; s_ok[tid][1] = 1; }
  __syncthreads();
  // every load of a batch first (indices clamped into the window), then the tag checks
  for (int j0 = 0; j0 < Wn * SV; j0 += BATCH * PNR_BLOCK) {
    uint64_t x[BATCH];
#pragma unroll
    for (int j = 0; j < BATCH; ++j) {
      const int idx = min(j0 + tid + j * PNR_BLOCK, Wn * SV - 1);
      const int w = idx / SV, e = idx - w * SV;
      x[j] = __hip_atomic_load(slots + (size_t)(tile - 1 - w) * SV + e, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
#pragma unroll
    for (int j = 0; j < BATCH; ++j) {
      const int idx = j0 + tid + j * PNR_BLOCK;
      if (idx < Wn * SV) {
        const int w = idx / SV, e = idx - w * SV;
        if ((uint32_t)(x[j] >> 32) != ep) s_ok[w][e < SA ? 0 : 1] = 0;
        Win[w * SV + e] = __uint_as_float((uint32_t)x[j]);
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
// Diagonal (quasi-Newton) Jacobian, without a grid barrier.
//
// The only values that cross blocks are 64-bit words tagged with their pass (value |
// epoch << 32), kept in three copies, one per pass modulo 3: the tile aggregates and
// prefixes of the look-back, and each block's residual maximum.  A tile needs no state
// of its predecessor: the state before its first step (the halo) starts at the initial
// guess and every fix-up adds the increment entering the tile, which the look-back
// delivers -- the same sum the predecessor forms for its last step, up to rounding.  A
// tile starts pass k+1 right after its own fix-up of pass k.  The stopping test is off
// the critical path: each block publishes its residual maximum of pass k right after
// its cells; block 0, the head of the first row and otherwise idle at that point,
// merges them at its own fix-up of pass k+1, records rho_k and publishes the decision;
// every block reads the decision on pass k-1 only before its fix-up of pass k, the
// first write over iterate k-1.  If it says stop, the decided iterate (k-1 or k) is
// still held.
//
// Why three copies suffice: a word of pass k is rewritten in pass k+3, by a tile past
// its fix-up of pass k+2, so after the decision on pass k+1, which was merged after every
// block finished its cells of pass k+1 and hence its look-back of pass k (the last read
// of the words of pass k).
//
// Two modes, chosen on the host:
//  * streaming: a block may own several tiles of 64 steps; every pass stages the tile's
//    states from HBM, streams its gate inputs, and writes the next iterate back;
//  * resident (every tile owns a co-resident block): the tile's states stay in LDS for
//    the whole launch, in two buffers (the iterate being checked, and the next one);
//    the returned iterate is written to the caller's output once, at the end.  Tiles are
//    64 steps, or 128 (D = 64 only) when there are more 64-step tiles than co-resident
//    blocks.  The gate inputs are streamed a block of 16 steps ahead of their use; with
//    every tile on the same CU in every pass they stay in that XCD's L2.
//
// LDS: Bh[3D] | X0[(TL+1) LD] | X1 (resident) | Xj (streaming with Jacobian reuse) |
//      R[D][TL+4] | Jd[D][TL+4] | Sa, Sb[P D] | Agg[2 P D] | Din[D]   (P = 256 / D;
//      r and J channel-major, so that a lane's 4 or 16 consecutive steps are vectors)
// Slots per tile and pass modulo 3: A[D] | b[D] | prefix[D]; then per tile (streaming) the
// halo and the refresh-point halo of a reused Jacobian (D floats each).

// Look-back window: each thread reads mfd_lookback_chunks() chunks of
// mfd_lookback_per_thread() predecessor tiles; the window is 256 / D times their product
// (8 tiles for D = 64).  Measured on gru-shaped rows, short windows resolve sooner than
// long ones: every poll of a long window waits for the slowest of many predecessors,
// while a tile beyond a short window takes the published prefix of a nearer one.
__host__ __device__ constexpr int mfd_lookback_per_thread(int D) { return D >= 32 ? 2 : 1; }
__host__ __device__ constexpr int mfd_lookback_chunks(int D) { return 1; }

__host__ __device__ inline size_t mfd_lds_floats(int D, int TL, int reuse, int resident) {
  const int LD = D + 4, P = PNR_BLOCK / D;
  const size_t xs = (size_t)(TL + 1) * LD;
  return (size_t)3 * D + xs * (1 + (resident ? 1 : 0) + (reuse ? 1 : 0)) + (size_t)2 * D * (TL + 4) +
         (size_t)4 * P * D + D;
}

__device__ __forceinline__ uint64_t load_dec(Ctrl* c) {
  return __hip_atomic_load(&c->dec, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void short_backoff(uint32_t spins) {
  if (spins < 32) __builtin_amdgcn_s_sleep(1);
  else __builtin_amdgcn_s_sleep(4);
}

// Bounded wait for ready(); every few polls it also looks for a published stop
// decision (which makes the awaited value unnecessary) or a fault.  Returns 0 when
// ready, 1 when stopped, 2 on a fault or when the spin budget ran out.
template <class Ready>
__device__ __forceinline__ int wait_for(Ready ready, Ctrl* c) {
  uint32_t spins = 0;
  while (!ready()) {
    if ((++spins & 7) == 0) {
      if (has_fault(c)) return 2;
      if (load_dec(c) & 1ull) return 1;
    }
    if (spins > kSpinLimit) {
      record_fault(c, 1);
      return 2;
    }
    short_backoff(spins);
  }
  return 0;
}

// Increment entering tile `seg` of its row (valid in threads tid < DM).  Thread
// (group g, channel c) covers a run of NCH * kLBPer consecutive predecessors of a window
// of min(seg, G * NCH * kLBPer) tiles: it reads their aggregates (A, b) -- except the
// farthest tile of the window, whose inclusive prefix it reads instead -- in NCH chunks,
// far to near, and composes them; the groups' maps are then composed in LDS.  Returns
// the wait status (0 ok) through `st`, block-uniform.
template <int DM, int kLBPer, int NCH>
__device__ __forceinline__ float lookback_regs(const uint64_t* __restrict__ slots, int tile, int seg, int km3,
                                               uint32_t ep, float* __restrict__ Agg, Ctrl* ctrl, int& st) {
  constexpr int G = PNR_BLOCK / DM, SVP = 3 * DM, RUN = NCH * kLBPer;
  __shared__ int s_st;
  const int tid = threadIdx.x, c = tid % DM, grp = tid / DM;
  const int Wn = min(seg, G * RUN);
  const int g_lo = grp * RUN + 1, g_hi = min(Wn, g_lo + RUN - 1);
  if (tid == 0) s_st = 0;
  float ga = 1.f, gb = 0.f;
  __syncthreads();
  for (int ch = NCH - 1; ch >= 0; --ch) {
    const int w_lo = g_lo + ch * kLBPer, w_hi = min(g_hi, w_lo + kLBPer - 1);
    if (w_lo > w_hi) continue;
    uint32_t spins = 0;
    bool give_up = false;
    while (true) {
      // All loads first (addresses clamped into the window, so every one is valid and
      // none waits on another), then the tag checks: one memory round trip per poll.
      uint64_t wa[kLBPer], wb[kLBPer];
#pragma unroll
      for (int j = 0; j < kLBPer; ++j) {
        const int w = min(w_lo + j, Wn);
        const uint64_t* sp = slots + ((size_t)(tile - w) * 3 + km3) * SVP;
        wa[j] = __hip_atomic_load(sp + c, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        wb[j] = __hip_atomic_load(sp + (w == Wn ? 2 * DM : DM) + c, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
      bool ok = true;
#pragma unroll
      for (int j = 0; j < kLBPer; ++j) {
        const int w = w_lo + j;
        const bool live = w <= w_hi, pre = w == Wn;
        const bool tb_ok = (uint32_t)(wb[j] >> 32) == ep, ta_ok = pre || (uint32_t)(wa[j] >> 32) == ep;
        ok = ok & (!live | (tb_ok & ta_ok));
      }
      if (ok) {
#pragma unroll
        for (int j = kLBPer - 1; j >= 0; --j) {
          const int w = w_lo + j;
          const bool live = w <= w_hi, pre = w == Wn;
          const float va = live ? (pre ? 0.f : __uint_as_float((uint32_t)wa[j])) : 1.f;
          const float vb = live ? __uint_as_float((uint32_t)wb[j]) : 0.f;
          gb = fmaf(va, gb, vb);
          ga *= va;
        }
        break;
      }
      // same policy as wait_for: give up on a published stop or a fault
      if ((++spins & 7) == 0) {
        const int w = has_fault(ctrl) ? 2 : ((load_dec(ctrl) & 1ull) ? 1 : 0);
        if (w) {
          atomicMax(&s_st, w);
          give_up = true;
          break;
        }
      }
      if (spins > kSpinLimit) {
        record_fault(ctrl, 1);
        atomicMax(&s_st, 2);
        give_up = true;
        break;
      }
      short_backoff(spins);
    }
    if (give_up) break;
  }
  Agg[grp * 2 * DM + c] = ga;
  Agg[grp * 2 * DM + DM + c] = gb;
  __syncthreads();
  st = s_st;
  float din = 0.f;
  if (tid < DM)
    for (int g2 = G - 1; g2 >= 0; --g2) din = fmaf(Agg[g2 * 2 * DM + tid], din, Agg[g2 * 2 * DM + DM + tid]);
  return din;
}

// Input projection of one tile inside the loop kernel (fp32 inputs):
//   gx[b][t0 + s][m] = sum_k x[b][t0 + s][k] W[m][k] + b_x[m],   s < Lv, m < 3D.
// The tile's inputs are staged in LDS in chunks of 64 k (zero-padded); wave w owns the
// column blocks w, w+4, ... of 16 output columns and every row block of 16 steps, on
// v_mfma_f32_16x16x4f32 with the k split of load_afrag (lane group q takes k = 16q + kk),
// its W fragments read straight from global memory (W is small and stays in L2).  All
// loads of a chunk (the x rows as float4s, every W fragment of the wave) are issued
// before the first one is used, so the chunk costs one memory round trip.  Each tile's
// gate inputs are read later only by the block that owns the tile.
template <int DM, int TL>
__device__ __forceinline__ void project_tile(const DenseLoopArgs<float>& a, float* __restrict__ Xs, int b, int t0,
                                             int Lv) {
  constexpr int N = 3 * DM, NCB = N / 16, MCB = (NCB + PNR_WAVES - 1) / PNR_WAVES, RB = TL / 16, XLD = 68;
  constexpr int XV = TL * 16 / PNR_BLOCK;   // float4s of x per thread and chunk
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6, q = lane >> 4, r16 = lane & 15;
  const int K = a.D_in, T = a.T;
  const bool wvec = (K % 4) == 0 && ((uintptr_t)a.W % 16) == 0;
  const bool xvec = (K % 4) == 0 && ((uintptr_t)a.x % 16) == 0;
  v4f acc[MCB][RB];
#pragma unroll
  for (int c = 0; c < MCB; ++c)
#pragma unroll
    for (int r = 0; r < RB; ++r) acc[c][r] = v4f{0.f, 0.f, 0.f, 0.f};
  for (int kc = 0; kc < K; kc += 64) {
    // ---- issue every load of the chunk ----
    v4f xv[XV];
#pragma unroll
    for (int j = 0; j < XV; ++j) {
      const int e = tid + j * PNR_BLOCK, srow = e >> 4, k = kc + 4 * (e & 15);
      const float* xp = a.x + ((size_t)b * T + t0 + srow) * K + k;
      if (srow >= Lv) {
        xv[j] = v4f{0.f, 0.f, 0.f, 0.f};
      } else if (xvec && k + 3 < K) {
        xv[j] = *reinterpret_cast<const v4f*>(xp);
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) xv[j][i] = k + i < K ? xp[i] : 0.f;
      }
    }
    float bf[MCB][16];
#pragma unroll
    for (int c = 0; c < MCB; ++c) {
      const int cbk = wid + c * PNR_WAVES;
      // W fragment: column n, k = kc + 16q + kk
      const int n = (cbk < NCB ? cbk : 0) * 16 + r16, k0 = kc + 16 * q;
      const float* wp = a.W + (size_t)n * K + k0;
      if (wvec && k0 + 15 < K) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const v4f v = *reinterpret_cast<const v4f*>(wp + 4 * j);
#pragma unroll
          for (int e = 0; e < 4; ++e) bf[c][4 * j + e] = v[e];
        }
      } else {
#pragma unroll
        for (int j = 0; j < 16; ++j) bf[c][j] = k0 + j < K ? wp[j] : 0.f;
      }
    }
    __syncthreads();   // the previous chunk's reads are done
#pragma unroll
    for (int j = 0; j < XV; ++j) {
      const int e = tid + j * PNR_BLOCK;
      *reinterpret_cast<v4f*>(Xs + (e >> 4) * XLD + 4 * (e & 15)) = xv[j];
    }
    __syncthreads();
#pragma unroll
    for (int c = 0; c < MCB; ++c) {
      const int cbk = wid + c * PNR_WAVES;
      if (cbk >= NCB) break;
#pragma unroll
      for (int r = 0; r < RB; ++r) {
        v4f af[4];
        const v4f* ap = reinterpret_cast<const v4f*>(Xs + (r * 16 + r16) * XLD + 16 * q);
#pragma unroll
        for (int j = 0; j < 4; ++j) af[j] = ap[j];
#pragma unroll
        for (int kk = 0; kk < 16; ++kk) acc[c][r] = mfma4(af[kk >> 2][kk & 3], bf[c][kk], acc[c][r]);
      }
    }
  }
  // lane holds rows 4q + e, column r16 of each 16 x 16 tile
#pragma unroll
  for (int c = 0; c < MCB; ++c) {
    const int cbk = wid + c * PNR_WAVES;
    if (cbk >= NCB) break;
    const int m = cbk * 16 + r16;
    const float bias = a.bx ? a.bx[m] : 0.f;
#pragma unroll
    for (int r = 0; r < RB; ++r)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int s = r * 16 + 4 * q + e;
        if (s < Lv) a.gx_out[((size_t)b * T + t0 + s) * N + m] = acc[c][r][e] + bias;
      }
  }
}

template <int DM, int TL, bool RES, bool REUSE>
__global__ void __launch_bounds__(PNR_BLOCK, (RES && TL > 64) ? 1 : 2)
    dense_diag_mfma_kernel(DenseLoopArgs<float> a) {
  static_assert(!(RES && REUSE), "the resident variant keeps no refresh-point iterate");
  extern __shared__ __align__(16) float lds[];
  __shared__ uint32_t s_wmax[PNR_WAVES];
  __shared__ int s_flag;
  Ctrl* ctrl = a.ctrl;
  constexpr int D = DM, LD = DM + 4, P = PNR_BLOCK / DM, LP = TL / P, SVP = 3 * DM;
  constexpr int NCB = D / 16, TBS = PNR_WAVES / NCB, NTB = (TL / 16) / TBS;   // MFMA work split
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int T = a.T;
  constexpr size_t XS = (size_t)(TL + 1) * LD;
  float* Bh = lds;
  float* Xb0 = Bh + 3 * D;
  float* Xb1 = Xb0 + XS;
  float* Xj = Xb1 + (RES ? XS : 0);
  float* R = Xj + (REUSE ? XS : 0);
  constexpr int RLD = TL + 4;   // channel-major row length of R and Jd
  float* Jd = R + D * RLD;
  float* Sa = Jd + D * RLD;
  float* Sb = Sa + P * D;
  float* Agg = Sb + P * D;
  float* Din = Agg + 2 * P * D;

  if (a.x) {
    // the input projection of this block's tiles (see project_tile); every wave drains
    // its stores before the barrier, so the loop below may read any of them
    for (int item = blockIdx.x; item < a.n_tiles; item += gridDim.x) {
      const int seg = item / a.B, b = item - seg * a.B;
      project_tile<D, TL>(a, lds, b, seg * TL, min(TL, T - seg * TL));
    }
    drain_memory_ops();
    __syncthreads();
  }
  for (int i = tid; i < 3 * D; i += PNR_BLOCK) Bh[i] = a.bh ? a.bh[i] : 0.f;
  // this wave's U fragments (recurrent product) and the diagonal of each gate block
  const int cb = wid % NCB, tb0 = wid / NCB;
  const int c_mf = cb * 16 + (lane & 15);
  float uf[3][D / 4], udg[3];
#pragma unroll
  for (int g = 0; g < 3; ++g) {
#pragma unroll
    for (int kk = 0; kk < D / 4; ++kk) uf[g][kk] = a.U[(size_t)(g * D + c_mf) * D + (lane >> 4) * (D / 4) + kk];
    udg[g] = a.U[(size_t)(g * D + c_mf) * D + c_mf];
  }
  const float bhr = a.bh ? a.bh[c_mf] : 0.f, bhz = a.bh ? a.bh[D + c_mf] : 0.f,
              bhn = a.bh ? a.bh[2 * D + c_mf] : 0.f;
  const int pp_ = tid / D, ci = tid - pp_ * D;   // scan layout: part, channel
  const int grid = (int)gridDim.x;
  const bool merger = blockIdx.x == 0;

  // Gate inputs of step tb*16 + 4(lane/16) + i, channel c_mf, of a tile.  The loads are
  // unconditional and unmasked: the gx region is padded by kGxPadRows rows, so the rows
  // of a tile past the end of the sequence are readable, and every value computed from
  // such a row is replaced in cell_elem (residual 0, Jacobian 1) by a select.  With no
  // branch and no select at the load, the loads stay in flight across the next block's
  // MFMAs instead of each one being waited for.
  auto load_gx = [&](float (&v)[4][3], int b, int t0, int tb) {
    const float* gxb = a.gx + (size_t)b * T * 3 * D;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int s = tb * 16 + 4 * (lane >> 4) + i;
      const float* g = gxb + (size_t)(t0 + s) * 3 * D;
#pragma unroll
      for (int q = 0; q < 3; ++q) v[i][q] = g[q * D + c_mf];
    }
  };

  if (RES)
    for (int i = tid; i < (int)XS; i += PNR_BLOCK) Xb1[i] = 0.f;
  float* Xc = Xb0;   // iterate whose residual this pass checks
  float* Xn = Xb1;   // the next iterate (resident mode)

  // Leaves the loop once a stop decision is published.  Before the fix-up of pass k the
  // decided iterate is k or k-1, both still in LDS: the resident variant writes its tile
  // of it to the caller's output.
  auto finish = [&](int k) {
    if (RES && !has_fault(ctrl)) {
      const int kd = (int)(load_dec(ctrl) >> 32) - 1;
      const float* Xr = kd == k ? Xc : Xn;
      const int seg = (int)blockIdx.x / a.B, b = (int)blockIdx.x - seg * a.B;
      const int t0 = seg * TL, Lv = min(TL, T - t0);
      for (int i = tid; i < Lv * D; i += PNR_BLOCK) {
        const int s = i / D, c = i - s * D;
        a.out[((size_t)b * T + t0 + s) * D + c] = Xr[(s + 1) * LD + c];
      }
    }
  };

  // Block 0 -- the head of the first row, which otherwise idles at its gate -- merges
  // the residual maxima of pass kk once every block has published its own, records
  // rho_kk (finish_iteration) and publishes the decision.  Returns 0 (continue), 1 (stop)
  // or 2 (fault).  Block-uniform.
  auto merge = [&](int kk, int cur_kk) -> int {
    const int m3 = kk % 3;
    const uint32_t epk = (uint32_t)kk + 1u;
    uint32_t mm = 0;
    int wst = 0;
    for (int i = tid; i < grid; i += PNR_BLOCK) {
      const uint64_t* pw = a.partials + (size_t)m3 * grid + i;
      uint64_t x = 0;
      const int w = wait_for([&]() {
        x = __hip_atomic_load(pw, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        return (uint32_t)(x >> 32) == epk;
      }, ctrl);
      if (w) wst = w;
      mm = max(mm, (uint32_t)x);
    }
    mm = wave_max_u32(mm);
    __syncthreads();
    if (tid == 0) s_flag = 0;
    __syncthreads();
    if (lane == 0) s_wmax[wid] = mm;
    if (wst) atomicMax(&s_flag, wst);
    __syncthreads();
    if (s_flag) return s_flag;
    if (tid == 0) {
      for (int w2 = 0; w2 < PNR_WAVES; ++w2) mm = max(mm, s_wmax[w2]);
      finish_iteration(ctrl, a.rho_hist, bits_to_rho(mm), kk, cur_kk, a.max_iters, a.tol);
      const int done = __hip_atomic_load(&ctrl->done, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      drain_memory_ops();   // rho, status and iters land before the decision word
      __hip_atomic_store(&ctrl->dec, ((uint64_t)epk << 32) | (uint64_t)(done ? 1 : 0), __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
      s_flag = done ? 1 : 0;
    }
    __syncthreads();
    return s_flag;
  };

  int cur = -1, prev = -1, jac = -1;
  __syncthreads();
  for (int k = 0; k <= a.max_iters; ++k) {
    const bool resid_only = k == a.max_iters;
    if (!resid_only && k % a.jac_every == 0) jac = cur;
    const int next = resid_only ? cur : next_buffer(cur, REUSE ? jac : -1, a.nbuf);
    const float* Hcur = cur >= 0 ? a.H[cur] : nullptr;
    const float* Hjac = jac >= 0 ? a.H[jac] : nullptr;
    float* Hnext = next >= 0 ? a.H[next] : nullptr;
    const bool stale = REUSE && !resid_only && jac != cur;
    const uint32_t ep = (uint32_t)k + 1u;
    const int km3 = k % 3;
    uint32_t blk_max = 0;
    bool dec_seen = k == 0;   // the decision on pass k-1 (none before pass 0)
    int stop = 0;             // 1: a stop decision ended a wait; 2: fault
    // Items go out time-segment-major (segment s of every batch row before segment
    // s+1), so a tile's predecessors have smaller item indices: they were handed out
    // earlier, and their aggregates are usually published before a successor looks back.
    for (int item = blockIdx.x; item < a.n_tiles && !stop; item += grid) {
      const bool last_item = item + grid >= a.n_tiles;
      const int seg = item / a.B, b = item - seg * a.B;
      const int tile = b * a.tiles_per_row + seg;   // slot index: row-major
      const int t0 = seg * TL, Lv = min(TL, T - t0);

      // ---- stage the iterate: rows 1..TL and the halo ----
      // Thread (part, channel) loads exactly the rows its own fix-up stored in the pass
      // before, so no other thread's global stores need to have landed.
      auto stage_own = [&](float* X, const float* H) {
#pragma unroll
        for (int j = 0; j < LP; ++j) {
          const int s2 = pp_ * LP + j;
          X[(s2 + 1) * LD + ci] = (H && s2 < Lv) ? H[((size_t)b * T + t0 + s2) * D + ci] : 0.f;
        }
      };
      if (!RES || k == 0) stage_own(Xc, RES ? nullptr : Hcur);
      if (stale) stage_own(Xj, Hjac);
      if (tid == 0) s_flag = 0;
      // The halo (the state before the tile's first step) is the tile's own: it starts
      // at zero (the initial guess) and each fix-up adds the increment that enters the
      // tile, which the look-back delivers.  No tile waits for its predecessor's states.
      float* hal = reinterpret_cast<float*>(a.slots + (size_t)a.n_tiles * 3 * SVP) + (size_t)tile * 2 * D;
      if ((!RES || k == 0) && tid < D)
        Xc[tid] = seg == 0 ? (a.h0 ? a.h0[(size_t)b * D + tid] : 0.f) : (k == 0 ? 0.f : hal[tid]);
      if (REUSE && tid < D) {
        // the halo of the refresh-point iterate, for the passes that reuse its Jacobian
        if (!resid_only && k % a.jac_every == 0) hal[D + tid] = Xc[tid];
        if (stale) Xj[tid] = hal[D + tid];
      }
      __syncthreads();

      // ---- cell on MFMA: residual and diagonal Jacobian ----
      uint32_t tmax = 0;
      // Residual and Jacobian diagonal of this lane's 4 steps of a block of 16, from the
      // block's gate products.  Branch-free (steps past the end of the sequence are
      // masked), so the compiler can interleave it with the next block's MFMAs.
      auto cell_elem = [&](int tb, const v4f (&acc)[3], const float (&gv)[4][3]) {
        v4f accj[3];
        if (stale) {
          v4f fj[D / 16];
          load_afrag<D>(Xj, LD, tb, fj);
          gates_frag<D>(fj, uf, accj);
        }
        v4f rr, jj;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int s = tb * 16 + 4 * (lane >> 4) + i;
          const bool ok = s < Lv;
          const float p = Xc[s * LD + c_mf];
          float r = sigm(gv[i][0] + acc[0][i] + bhr);
          float z = sigm(gv[i][1] + acc[1][i] + bhz);
          float ghn = acc[2][i] + bhn;
          float n = tanh_(fmaf(r, ghn, gv[i][2]));
          float res = fmaf(z, p - n, n) - Xc[(s + 1) * LD + c_mf];
          res = ok ? res : 0.f;
          rr[i] = res;
          tmax = max(tmax, abs_bits(res));
          float pj = p;
          if (stale) {
            pj = Xj[s * LD + c_mf];
            r = sigm(gv[i][0] + accj[0][i] + bhr);
            z = sigm(gv[i][1] + accj[1][i] + bhz);
            ghn = accj[2][i] + bhn;
            n = tanh_(fmaf(r, ghn, gv[i][2]));
          }
          const float omz = 1.f - z, cn = omz * (1.f - n * n);
          float jd = z + (pj - n) * z * omz * udg[1] + cn * ghn * r * (1.f - r) * udg[0] + cn * r * udg[2];
          jd = a.jac_mode == PNR_JAC_ZERO ? 0.f : jd;
          jj[i] = ok ? jd : 1.f;
        }
        const int o = c_mf * RLD + tb * 16 + 4 * (lane >> 4);
        *reinterpret_cast<v4f*>(R + o) = rr;
        *reinterpret_cast<v4f*>(Jd + o) = jj;
      };
      // Software pipeline over the blocks of 16 steps: block u's MFMAs are issued
      // before block u-1's elementwise work, which does not depend on them.  The gate
      // inputs are loaded a block ahead.  Two blocks per trip in ping-pong registers:
      // copying just-loaded gate inputs from one set to the other would make the
      // compiler wait for those loads in the middle of the elementwise work.
      {
        v4f fa[D / 16];
        v4f accA[3], accB[3];
        float gvA[4][3], gvB[4][3];
        load_afrag<D>(Xc, LD, tb0, fa);
        load_gx(gvA, b, t0, tb0);
        gates_frag<D>(fa, uf, accA);
        if (NTB > 1) load_afrag<D>(Xc, LD, tb0 + TBS, fa);
#pragma unroll
        for (int u = 1; u < NTB; u += 2) {
          load_gx(gvB, b, t0, tb0 + u * TBS);
          gates_frag<D>(fa, uf, accB);
          if (u + 1 < NTB) load_afrag<D>(Xc, LD, tb0 + (u + 1) * TBS, fa);
          cell_elem(tb0 + (u - 1) * TBS, accA, gvA);
          if (u + 1 < NTB) {
            load_gx(gvA, b, t0, tb0 + (u + 1) * TBS);
            gates_frag<D>(fa, uf, accA);
            if (u + 2 < NTB) load_afrag<D>(Xc, LD, tb0 + (u + 2) * TBS, fa);
          }
          cell_elem(tb0 + u * TBS, accB, gvB);
        }
        if (NTB & 1) cell_elem(tb0 + (NTB - 1) * TBS, accA, gvA);
      }
      blk_max = max(blk_max, tmax);
      __syncthreads();

      // ---- the block's residual maximum of this pass; the merging block decides ----
      if (last_item) {
        uint32_t m = wave_max_u32(blk_max);
        if (lane == 0) s_wmax[wid] = m;
        __syncthreads();
        if (tid == 0) {
          for (int w2 = 0; w2 < PNR_WAVES; ++w2) m = max(m, s_wmax[w2]);
          __hip_atomic_store(a.partials + (size_t)km3 * grid + blockIdx.x, ((uint64_t)ep << 32) | m,
                             __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
      }

      uint64_t* myslot = a.slots + ((size_t)tile * 3 + km3) * SVP;
      float ta = 1.f, tbv = 0.f;
      if (!resid_only) {
        // ---- scan inside the tile: part aggregates, tile total, publication ----
        float jv[LP], rv[LP];   // this (part, channel)'s J and r: all loads first
        const int po = ci * RLD + pp_ * LP;   // its steps, contiguous
#pragma unroll
        for (int j = 0; j < LP; j += 4) {
          const v4f jq = *reinterpret_cast<const v4f*>(Jd + po + j), rq = *reinterpret_cast<const v4f*>(R + po + j);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            jv[j + e] = jq[e];
            rv[j + e] = rq[e];
          }
        }
        float ea = 1.f, eb = 0.f;
#pragma unroll
        for (int j = 0; j < LP; ++j) {
          eb = fmaf(jv[j], eb, rv[j]);
          ea *= jv[j];
        }
        Sa[pp_ * D + ci] = ea;
        Sb[pp_ * D + ci] = eb;
        __syncthreads();
        if (tid < D) {
          for (int q = 0; q < P; ++q) {
            tbv = fmaf(Sa[q * D + tid], tbv, Sb[q * D + tid]);
            ta *= Sa[q * D + tid];
          }
          if (seg == 0) {
            slot_put(myslot + 2 * D + tid, ep, tbv);
          } else {
            slot_put(myslot + tid, ep, ta);
            slot_put(myslot + D + tid, ep, tbv);
          }
        }
        // Before the increment entering the tile (d_in) is known, write every step's
        // increment as d_s = L_s + M_s d_in: L and M are the chain d -> J d + r started
        // from the parts before this one, applied to (d_in = 0) and to the unit map.
        // They replace r and J in place (each element is this thread's own), so the
        // fix-up after the look-back is one independent FMA per element.
        {
          float ma = 1.f, lb = 0.f;
          for (int q = 0; q < pp_; ++q) {
            lb = fmaf(Sa[q * D + ci], lb, Sb[q * D + ci]);
            ma *= Sa[q * D + ci];
          }
#pragma unroll
          for (int j = 0; j < LP; j += 4) {
            v4f lq, mq;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              lb = fmaf(jv[j + e], lb, rv[j + e]);
              ma *= jv[j + e];
              lq[e] = lb;
              mq[e] = ma;
            }
            *reinterpret_cast<v4f*>(R + po + j) = lq;
            *reinterpret_cast<v4f*>(Jd + po + j) = mq;
          }
        }
        // ---- decoupled look-back over the predecessors, in registers ----
        if (seg > 0) {
          int w = 0;
          const float dl = lookback_regs<D, mfd_lookback_per_thread(DM), mfd_lookback_chunks(DM)>(
              a.slots, tile, seg, km3, ep, Agg, ctrl, w);
          if (w) {
            stop = w;
            break;
          }
          if (tid < D) {
            Din[tid] = dl;
            slot_put(myslot + 2 * D + tid, ep, fmaf(ta, dl, tbv));
          }
        } else if (tid < D) {
          Din[tid] = 0.f;
        }
      }

      if (resid_only) continue;

      // ---- the decision on pass k-1 guards the first overwrite of iterate k-1 ----
      if (!dec_seen && merger) {
        const int w = merge(k - 1, prev);
        if (w) {
          stop = w;
          break;
        }
        dec_seen = true;
      }
      if (!dec_seen) {
        if (tid == 0) {
          uint64_t d = 0;
          const int w = wait_for([&]() {
            d = load_dec(ctrl);
            return (uint32_t)(d >> 32) >= (uint32_t)k;
          }, ctrl);
          s_flag = w ? w : (int)(d & 1ull);
        }
        __syncthreads();
        if (s_flag) {
          stop = s_flag;
          break;
        }
        dec_seen = true;
      }
      __syncthreads();
      // ---- fix-up: s <- s + L + M d_in, element by element ----
      {
        const float din = Din[ci];
        if (tid < D) {   // the next iterate's halo
          const float h = seg == 0 ? (a.h0 ? a.h0[(size_t)b * D + tid] : 0.f) : Xc[tid] + Din[tid];
          if (RES) Xn[tid] = h;
          else hal[tid] = h;
        }
        float xv[LP], lv[LP], mv[LP];
        const int po = ci * RLD + pp_ * LP;
#pragma unroll
        for (int j = 0; j < LP; j += 4) {
          const v4f lq = *reinterpret_cast<const v4f*>(R + po + j), mq = *reinterpret_cast<const v4f*>(Jd + po + j);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            lv[j + e] = lq[e];
            mv[j + e] = mq[e];
          }
        }
#pragma unroll
        for (int j = 0; j < LP; ++j) xv[j] = Xc[(pp_ * LP + j + 1) * LD + ci];
        // (rows past the end of the sequence are written too in LDS, where they are never
        // read as states; only real steps go to the state buffer)
        float* hn = Hnext + ((size_t)b * T + t0 + pp_ * LP) * D + ci;
#pragma unroll
        for (int j = 0; j < LP; ++j) {
          const float v = xv[j] + fmaf(mv[j], din, lv[j]);
          if (RES) Xn[(pp_ * LP + j + 1) * LD + ci] = v;
          else if (pp_ * LP + j < Lv) hn[(size_t)j * D] = v;
        }
      }
      __syncthreads();
    }
    if (stop == 0 && resid_only && merger) {
      // the last pass (no fix-up, so no gate): the decisions on passes M-1 and M
      if (!dec_seen) stop = merge(k - 1, prev);
      if (!stop) stop = merge(k, cur);
    }
    if (stop == 0 && resid_only) {
      // the last pass: wait for its (stopping) decision
      if (tid == 0) {
        const int w = wait_for([&]() { return (uint32_t)(load_dec(ctrl) >> 32) >= (uint32_t)(k + 1); }, ctrl);
        s_flag = w == 2 ? 2 : 1;
      }
      __syncthreads();
      stop = s_flag;
    }
    if (stop) {
      finish(k);
      return;
    }
    prev = cur;
    cur = next;
    if (RES) {
      float* t = Xc;
      Xc = Xn;
      Xn = t;
    }
  }
}

// =====================================================================================
// Dense 16x16 Jacobian.  LDS: Bh[48] | X[65 LD] | Xj (reuse) | R, Z, Al, Be, Ga [64][16] |
// Pagg[8][336] | Wm[4][336] | Xm[2][336] | Tot[336] | Win[W][288] | Din[16].
constexpr int kF = 16;
constexpr int kFAgg = kF * kF + kF;      // aggregate values: M (row-major) then v
constexpr int kFSlot = kFAgg + kF;       // slot values: aggregate, then prefix
constexpr int kFWin = 16;
// Aggregates staged for MFMA operand reads: the rows of M at a stride of kFL floats, then
// v.  With that stride a row's 4-float run (a b128 read) and a column's 4 entries fall on
// distinct banks for the 64 lanes.
constexpr int kFL = kF + 4;
constexpr int kFMat = kF * kFL + kF;
__host__ __device__ inline size_t mff_lds_floats(int reuse) {
  const int LD = kF + 4;
  return (size_t)3 * kF + (size_t)(kTL + 1) * LD * (reuse ? 2 : 1) + (size_t)5 * kTL * kF +
         (size_t)(kFParts + 4 + 2 + 1) * kFMat + (size_t)kFWin * kFSlot + kF;
}

// 16x16 operands of v_mfma_f32_16x16x4f32 with k split as 4q + i over the four issues:
// lane (q, m) holds A[m][4q+i] (an A fragment) and B[4q+i][m] (a B fragment), and the
// accumulator of A B holds (A B)[4q+i][m] -- the B fragment of the product.
template <int LDM = kFL>
__device__ __forceinline__ v4f ld_arow(const float* S, int m, int q) {
  return *reinterpret_cast<const v4f*>(S + m * LDM + 4 * q);
}
__device__ __forceinline__ v4f ld_bcol(const float* S, int m, int q) {
  v4f b;
#pragma unroll
  for (int i = 0; i < 4; ++i) b[i] = S[(4 * q + i) * kFL + m];
  return b;
}
__device__ __forceinline__ void st_acc(float* S, v4f c, int m, int q) {
#pragma unroll
  for (int i = 0; i < 4; ++i) S[(4 * q + i) * kFL + m] = c[i];
}
__device__ __forceinline__ v4f mm16(v4f a, v4f b, v4f c) {
#pragma unroll
  for (int i = 0; i < 4; ++i) c = mfma4(a[i], b[i], c);
  return c;
}
// (A v)[m] in every lane of row m, from A's fragment and v in LDS
__device__ __forceinline__ float mv_rows(v4f a, const float* v, int q) {
  const v4f x = *reinterpret_cast<const v4f*>(v + 4 * q);
  float s = fmaf(a[0], x[0], fmaf(a[1], x[1], fmaf(a[2], x[2], a[3] * x[3])));
  s += __shfl_xor(s, 16);
  s += __shfl_xor(s, 32);
  return s;
}
// d <- M d + v for a staged aggregate (rows at stride LDM, then v), with d in column 0 of a
// B fragment (lane (q, 0) holds d[4q+i], every other lane zeros); the result has the same form
template <int LDM>
__device__ __forceinline__ v4f mv_col0(const float* S, v4f d, int m, int q) {
  v4f c;
#pragma unroll
  for (int i = 0; i < 4; ++i) c[i] = m == 0 ? S[kF * LDM + 4 * q + i] : 0.f;
  return mm16(ld_arow<LDM>(S, m, q), d, c);
}

// Entry J_t[row][col] from the factors of `row` and U_g[row][col] (g = r, z, n).
__device__ __forceinline__ float jac_entry(float z, float al, float be, float ga, float ur, float uz, float un,
                                           bool diag) {
  return fmaf(al, uz, fmaf(be, ur, ga * un)) + (diag ? z : 0.f);
}

// two waves per SIMD (two 4-wave blocks per CU, as its LDS allows): the register budget is 256
__global__ void __launch_bounds__(PNR_BLOCK, 2) dense_full_mfma_kernel(DenseLoopArgs<float> a) {
  extern __shared__ __align__(16) float lds[];
  Ctrl* ctrl = a.ctrl;
  constexpr int D = kF, LD = kF + 4;
  const int tid = threadIdx.x, lane = tid & 63, wid = __builtin_amdgcn_readfirstlane(tid >> 6);
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
  float* Pagg = Ga + kTL * D;           // part aggregates
  float* Wm = Pagg + kFParts * kFMat;   // products of part pairs
  float* Xm = Wm + 4 * kFMat;           // products of those pairs
  float* Tot = Xm + 2 * kFMat;          // the tile total
  float* Win = Tot + kFMat;
  float* Din = Win + kFWin * kFSlot;

  for (int i = tid; i < 3 * D; i += PNR_BLOCK) Bh[i] = a.bh ? a.bh[i] : 0.f;
  // U in registers: MFMA B fragments for the recurrent product, and the entries each
  // lane needs to form J^T (aggregate pass) and J (fix-up pass) operands
  // (the Jacobian's entries come from a.Uj when a low-rank approximation is in use)
  float uf[3][D / 4], ubT[3][4], ubN[3][4];
  const float* Ujm = a.Uj ? a.Uj : a.U;
#pragma unroll
  for (int g = 0; g < 3; ++g) {
#pragma unroll
    for (int kk = 0; kk < D / 4; ++kk) uf[g][kk] = a.U[(size_t)(g * D + m) * D + 4 * kk + q];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      ubT[g][i] = Ujm[(size_t)(g * D + 4 * q + i) * D + m];   // U_g[4q+i][m]
      ubN[g][i] = Ujm[(size_t)(g * D + m) * D + 4 * q + i];   // U_g[m][4q+i]
    }
  }
  __syncthreads();
  const float bhr = Bh[m], bhz = Bh[D + m], bhn = Bh[2 * D + m];

  int cur = -1, jac = -1;
  uint32_t gen = 0;   // generation of the next grid barrier
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
      uint64_t* myslot = a.slots + (size_t)tile * kFSlot;
      const int t0 = seg * kTL, Lv = min(kTL, T - t0);
      const float* gxb = a.gx + (size_t)b * T * 3 * D;
      stage_rows(X, Hcur, a.h0, b, t0, T, D, LD);
      if (stale) stage_rows(Xj, Hjac, a.h0, b, t0, T, D, LD);
      __syncthreads();

      // ---- cell on MFMA: residual and the Jacobian factors; wave w owns step block w ----
      uint32_t tmax = 0;
      {
        const int tb = wid;
        // unconditional loads (the gx region is padded by kGxPadRows rows); steps past
        // the end of the sequence never read their values
        float gxv[4][3];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int s = tb * 16 + 4 * q + i;
          const float* g = gxb + (size_t)(t0 + s) * 3 * D;
#pragma unroll
          for (int gg = 0; gg < 3; ++gg) gxv[i][gg] = g[gg * D + m];
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
#pragma unroll 4
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
        float* Pa = Pagg + pa * kFMat;
        float* Pb = Pagg + pb * kFMat;
        *reinterpret_cast<v4f*>(Pa + m * kFL + 4 * q) = xa;
        *reinterpret_cast<v4f*>(Pb + m * kFL + 4 * q) = xb;
        if (q == 0) {
          Pa[kF * kFL + m] = va;
          Pb[kF * kFL + m] = vb;
        }
        // ---- tile total as a pairwise tree on MFMA ----
        // level 1, in-wave (the part rows were written by this wave): W = M_b M_a
        const v4f zero4 = {0.f, 0.f, 0.f, 0.f};
        v4f w4 = mm16(xb, ld_bcol(Pa, m, q), zero4);
        float vw = mv_rows(xb, Pa + kF * kFL, q) + vb;
        float* Ww = Wm + wid * kFMat;
        st_acc(Ww, w4, m, q);
        if (q == 0) Ww[kF * kFL + m] = vw;
        __syncthreads();
        // level 2: waves 0 and 2 form X_0 = W_1 W_0 and X_1 = W_3 W_2 (B: their own W)
        if (wid == 0 || wid == 2) {
          const float* Wl = Wm + (wid + 1) * kFMat;
          const v4f al = ld_arow(Wl, m, q);
          w4 = mm16(al, w4, zero4);
          vw = mv_rows(al, Ww + kF * kFL, q) + Wl[kF * kFL + m];
          float* Xd = Xm + (wid >> 1) * kFMat;
          st_acc(Xd, w4, m, q);
          if (q == 0) Xd[kF * kFL + m] = vw;
        }
        __syncthreads();
        // level 3: wave 0 forms the tile total T = X_1 X_0 and publishes it
        if (wid == 0) {
          const float* X1 = Xm + kFMat;
          const v4f al = ld_arow(X1, m, q);
          const v4f t4 = mm16(al, w4, zero4);
          const float vt = mv_rows(al, Xm + kF * kFL, q) + X1[kF * kFL + m];
          st_acc(Tot, t4, m, q);
          if (q == 0) Tot[kF * kFL + m] = vt;
          if (seg == 0) {
            if (q == 0) {
              slot_put(myslot + kFAgg + m, ep, vt);
              Din[m] = 0.f;
            }
          } else {
#pragma unroll
            for (int i = 0; i < 4; ++i) slot_put(myslot + (4 * q + i) * kF + m, ep, t4[i]);
            if (q == 0) slot_put(myslot + kF * kF + m, ep, vt);
          }
        }
      }
      if (seg > 0) {
        // ---- decoupled look-back: wave 0 applies the aggregates after the nearest
        // published prefix, as a chain of MFMA matrix-vector products (d in column 0) ----
        uint32_t spins = 0;
        while (true) {
          const int pw = window_read<(kFWin * kFSlot + PNR_BLOCK - 1) / PNR_BLOCK>(a.slots, tile, min(seg, kFWin),
                                                                                kFSlot, kFAgg, ep, Win);
          if (pw >= 0) {
            if (wid == 0) {
              v4f d;
#pragma unroll
              for (int i = 0; i < 4; ++i) d[i] = m == 0 ? Win[pw * kFSlot + kFAgg + 4 * q + i] : 0.f;
              for (int w = pw - 1; w >= 0; --w) d = mv_col0<kF>(Win + w * kFSlot, d, m, q);
              const v4f e = mv_col0<kFL>(Tot, d, m, q);
              if (m == 0) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                  Din[4 * q + i] = d[i];
                  slot_put(myslot + kFAgg + 4 * q + i, ep, e[i]);
                }
              }
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

      // ---- fix-up on MFMA: d <- J_t d + r_t with d in column 0; s <- s + d ----
      {
        // the increments entering this wave's parts, from the one entering the tile:
        // Pin[2w] = (W_{w-1} .. W_0)(Din) through the tree's products, Pin[2w+1] = part_2w(Pin[2w])
        const int pa = 2 * wid, pb = 2 * wid + 1;
        v4f xa, xb;
#pragma unroll
        for (int i = 0; i < 4; ++i) xa[i] = m == 0 ? Din[4 * q + i] : 0.f;
        if (wid == 1) xa = mv_col0<kFL>(Wm, xa, m, q);
        if (wid >= 2) xa = mv_col0<kFL>(Xm, xa, m, q);
        if (wid == 3) xa = mv_col0<kFL>(Wm + 2 * kFMat, xa, m, q);
        xb = mv_col0<kFL>(Pagg + pa * kFMat, xa, m, q);
#pragma unroll 4
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
          // the new states go into the staged rows (row s + 1 holds step t0 + s): no global
          // store or wait inside the chain
          if (m == 0) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              X[(sa + 1) * LD + 4 * q + i] += xa[i];
              X[(sb + 1) * LD + 4 * q + i] += xb[i];
            }
          }
        }
      }
      __syncthreads();
      // the tile's new states, 16 threads to a row (coalesced), the last step's coherently
      // (the next tile's halo)
#pragma unroll
      for (int j = 0; j < kTL * kF / PNR_BLOCK; ++j) {
        const int idx = tid + j * PNR_BLOCK, s_ = idx >> 4, c_ = idx & 15;
        if (s_ < Lv) {
          float* o = Hnext + ((size_t)b * T + t0 + s_) * D + c_;
          const float v = X[(s_ + 1) * LD + c_];
          if (s_ == kTL - 1) coherent_store(o, v);
          else *o = v;
        }
      }
      __syncthreads();   // the rows are read before the next tile stages its own
    }
    if (end_pass(a, blk_max, k, cur, gen) || has_fault(ctrl)) break;
    cur = next;
  }
}

// =====================================================================================
int dense_mfma_supported(int D, int full, int is_f64) {
  if (is_f64) return 0;
  return full ? D == kF : (D == 16 || D == 32 || D == 64);
}
int dense_mfma_tile_len() { return kTL; }
int dense_mfma_slot_words(int D, int full) { return full ? kFSlot : 10 * D; }

static int block_occupancy(const void* fn, size_t lds) { return cached_occupancy(fn, lds); }

// Launch of a persistent loop kernel: at most the co-resident grid, at most one block
// per tile.
static hipError_t persistent_launch(const void* fn, const DenseLoopArgs<float>& a, size_t lds, int num_cu, hipStream_t st) {
  const int v = block_occupancy(fn, lds);
  if (v < 1) return hipErrorInvalidConfiguration;
  long g = (long)v * num_cu;
  if (g > kMaxGrid) g = kMaxGrid;
  if (g > a.n_tiles) g = a.n_tiles;
  if (g < 1) g = 1;
  void* args[] = {const_cast<DenseLoopArgs<float>*>(&a)};
  return launch_persistent(fn, (int)g, lds, args, st);
}

template <int DM>
static const void* diag_kernel(int res_tile, bool reuse) {
  if (res_tile == 128) return DM == 64 ? (const void*)dense_diag_mfma_kernel<64, 128, true, false> : nullptr;
  if (res_tile) return (const void*)dense_diag_mfma_kernel<DM, kTL, true, false>;
  return reuse ? (const void*)dense_diag_mfma_kernel<DM, kTL, false, true>
               : (const void*)dense_diag_mfma_kernel<DM, kTL, false, false>;
}
static const void* diag_kernel_for(int D, int res_tile, bool reuse) {
  if (D == 16) return diag_kernel<16>(res_tile, reuse);
  if (D == 32) return diag_kernel<32>(res_tile, reuse);
  return diag_kernel<64>(res_tile, reuse);
}

// PNR_DENSE_RESIDENT: "0" never, "64" / "128" only that tile length (tests and tuning).
int dense_mfma_resident_tile(int D, int full, int B, int T, int reuse, int num_cu) {
  if (full || reuse || !dense_mfma_supported(D, 0, 0) || B < 1 || T < 1) return 0;
  const char* env = getenv("PNR_DENSE_RESIDENT");
  const int only = env ? atoi(env) : -1;
  if (only == 0) return 0;
  for (int tl : {64, 128}) {
    if ((only > 0 && tl != only) || (tl == 128 && D != 64)) continue;
    const long tiles = (long)B * ((T + tl - 1) / tl);
    const int v = block_occupancy(diag_kernel_for(D, tl, false), mfd_lds_floats(D, tl, 0, 1) * 4);
    if (v >= 1 && tiles <= kMaxGrid && (long)v * num_cu >= tiles) return tl;
  }
  return 0;
}

hipError_t launch_dense_mfma(const DenseLoopArgs<float>& a, int full, int num_cu, hipStream_t st) {
  const bool reuse = a.nbuf > 2;
  if (full) return persistent_launch((const void*)dense_full_mfma_kernel, a, mff_lds_floats(reuse) * 4, num_cu, st);
  const bool res = a.out != nullptr;
  const bool dreuse = a.jac_every > 1;
  if (a.nbuf != (dreuse ? 3 : 2)) return hipErrorInvalidValue;
  if (res && (dreuse || !(a.L == kTL || (a.L == 128 && a.D == 64)))) return hipErrorInvalidValue;
  if (!res && a.L != kTL) return hipErrorInvalidValue;
  const void* fn = diag_kernel_for(a.D, res ? a.L : 0, dreuse);
  const size_t lds = mfd_lds_floats(a.D, a.L, dreuse, res) * 4;
  if (a.x && lds < (size_t)a.L * 68 * 4) return hipErrorInvalidValue;   // room to stage the projection
  // the resident variant needs one co-resident block per tile
  if (res && (long)block_occupancy(fn, lds) * num_cu < a.n_tiles) return hipErrorInvalidValue;
  return persistent_launch(fn, a, lds, num_cu, st);
}

}  // namespace pnr
