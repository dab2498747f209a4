// Backward pass of the GRU with a dense recurrent matrix U (gates r, z, n).
//
// Gradients through the evaluated sequence (ParaRNN overview, "Newton's Iteration": the
// block lower-triangular system is solved by backward as well as forward substitution;
// training through the parallel evaluation, "Parallelizing non-linear sequential models
// over the sequence length", abstract).  With g_t = dL/dh_t the adjoint is the linear
// system
//     lam_t = g_t + J_{t+1}^T lam_{t+1},   lam_T = g_T,
// whose Jacobians are dense (U couples the channels).  It is solved by the quasi-Newton
// idea of "Towards Scalable and Stable Parallelization of Nonlinear RNNs" (abstract; the
// summary's "Measured effects": the diagonal approximation also in the backward pass),
// applied to this linear system: with R(lam) its residual and d_t = diag(J_t),
//     delta_t = d_{t+1} delta_{t+1} + R_t     (a diagonal scan run backwards in time)
//     lam    <- lam + delta,
// repeated until max |R| is small.  The fixed point is the exact adjoint; the dense
// product J^T lam = z * lam + U^T dgh(lam) of each residual is one MFMA GEMM.
//
// Per step and channel the forward quantities enter through six factors of the gates
// (computed once from Gx, Gh = U h_{t-1} + b_h and h_{t-1}):
//     z,  d = diag(J),  f_z = (h_{t-1} - n) z (1 - z),  f_n = (1 - z)(1 - n^2),  r,
//     f_r = f_n * gh_n * r (1 - r)
// so that for an adjoint lam the pre-activation gradients are (f_r lam, f_z lam, f_n lam)
// for the input part and (f_r lam, f_z lam, f_n r lam) for the recurrent part.
#include "common.h"
#include "kernels.h"

namespace pnr {

// hprev[b][t] = h[b][t-1], hprev[b][0] = h0[b] (or 0)
__global__ void __launch_bounds__(256) gru_shift_states_kernel(const float* __restrict__ h,
                                                               const float* __restrict__ h0,
                                                               float* __restrict__ hprev, int B, int T, int D) {
  const size_t n = (size_t)B * T * D;
  for (size_t e = (size_t)blockIdx.x * blockDim.x + threadIdx.x; e < n; e += (size_t)gridDim.x * blockDim.x) {
    const size_t bt = e / D;
    const int i = (int)(e - bt * D);
    const int t = (int)(bt % T);
    const size_t b = bt / T;
    hprev[e] = t > 0 ? h[e - D] : (h0 ? h0[b * D + i] : 0.f);
  }
}

__global__ void __launch_bounds__(256) gru_bwd_factors_kernel(const float* __restrict__ gx,
                                                              const float* __restrict__ gh,
                                                              const float* __restrict__ hprev,
                                                              const float* __restrict__ U, float* __restrict__ F,
                                                              size_t n, int D) {
  for (size_t e = (size_t)blockIdx.x * blockDim.x + threadIdx.x; e < n; e += (size_t)gridDim.x * blockDim.x) {
    const size_t bt = e / D;
    const int i = (int)(e - bt * D);
    const float* gxr = gx + bt * 3 * D;
    const float* ghr = gh + bt * 3 * D;
    const float r = sigm(gxr[i] + ghr[i]);
    const float z = sigm(gxr[D + i] + ghr[D + i]);
    const float ghn = ghr[2 * D + i];
    const float nn = tanh_(fmaf(r, ghn, gxr[2 * D + i]));
    const float p = hprev[e];
    const float fz = (p - nn) * z * (1.f - z);
    const float fn = (1.f - z) * (1.f - nn * nn);
    const float fr = fn * ghn * r * (1.f - r);
    const float dj = z + fz * U[(size_t)(D + i) * D + i] + fn * r * U[(size_t)(2 * D + i) * D + i] +
                     fr * U[(size_t)i * D + i];
    F[e] = z;
    F[n + e] = dj;
    F[2 * n + e] = fz;
    F[3 * n + e] = fn;
    F[4 * n + e] = r;
    F[5 * n + e] = fr;
  }
}

// dgh[bt] = (f_r lam, f_z lam, f_n r lam); dgx[bt] = (f_r lam, f_z lam, f_n lam) when asked
__global__ void __launch_bounds__(256) gru_bwd_gates_kernel(const float* __restrict__ F, const float* __restrict__ lam,
                                                            float* __restrict__ dgh, float* __restrict__ dgx,
                                                            size_t n, int D) {
  for (size_t e = (size_t)blockIdx.x * blockDim.x + threadIdx.x; e < n; e += (size_t)gridDim.x * blockDim.x) {
    const size_t bt = e / D;
    const int i = (int)(e - bt * D);
    const float l = lam[e];
    const float ar = F[5 * n + e] * l, az = F[2 * n + e] * l, an = F[3 * n + e] * l;
    float* o = dgh + bt * 3 * D;
    o[i] = ar;
    o[D + i] = az;
    o[2 * D + i] = an * F[4 * n + e];
    if (dgx) {
      float* q = dgx + bt * 3 * D;
      q[i] = ar;
      q[D + i] = az;
      q[2 * D + i] = an;
    }
  }
}

// ---- refinement step as a chunked scan in the [B][T][D] layout ----
// delta_t = a_t delta_{t+1} + R_t run backwards in time, with
//   R_t = g_t + z_{t+1} lam_{t+1} + v_{t+1} - lam_t,  a_t = d_{t+1}   (t+1 terms 0 at T-1),
// over chunks of kChunk steps: one wave per chunk, one lane per channel (D <= 64).
// Pass 1 composes each chunk's map delta_{end} -> delta_{start} (and max |R|); pass 2
// walks the chunks of each channel; pass 3 re-walks each chunk from its carry, writes
// lam + delta into the other adjoint buffer and the recurrent-gate gradients of it.
constexpr int kChunk = 16;
constexpr int kBatch = 8;   // steps whose loads are issued together

struct StepIn {   // per-step inputs of one lane
  float g, lam, z, v, d;
};
__device__ __forceinline__ StepIn load_step(const float* g, const float* lam, const float* F, const float* v,
                                            size_t n, size_t e) {
  return StepIn{g[e], lam[e], F[e], v[e], F[n + e]};
}

template <bool APPLY>
__global__ void __launch_bounds__(256) gru_bwd_chunk_kernel(const float* __restrict__ F,
                                                            const float* __restrict__ lam,
                                                            const float* __restrict__ v,
                                                            const float* __restrict__ g, float2* __restrict__ agg,
                                                            const float* __restrict__ carry,
                                                            float* __restrict__ lam_new, float* __restrict__ dgh,
                                                            uint32_t* __restrict__ rmax, int T, int D, int nch) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int b = blockIdx.y, c = blockIdx.x * 4 + w;
  const size_t n = (size_t)gridDim.y * T * D;
  __shared__ uint32_t swmax[4];
  uint32_t m = 0;
  if (c < nch && lane < D) {
    const int t0 = c * kChunk, t1 = min(T, t0 + kChunk);
    const size_t base = (size_t)b * T * D + lane;
    // the step after the chunk (t1): its lam, z, v, d enter R and a of step t1 - 1
    StepIn nx{0.f, 0.f, 0.f, 0.f, 0.f};
    if (t1 < T) nx = load_step(g, lam, F, v, n, base + (size_t)t1 * D);
    float P = 1.f, Q = 0.f;                          // pass 1: delta_t = P delta_{t1} + Q
    float dl = APPLY ? carry[((size_t)b * nch + c) * D + lane] : 0.f;   // pass 3: delta at t1
    for (int tb = t1 - 1; tb >= t0; tb -= kBatch) {
      // loads of kBatch steps first (indices clamped into the chunk, results masked)
      StepIn in[kBatch];
      float fg[kBatch][4];   // pass 3: the gate factors f_r, f_z, f_n, r
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        const size_t e = base + (size_t)max(tb - u, t0) * D;
        in[u] = load_step(g, lam, F, v, n, e);
        if constexpr (APPLY) {
          fg[u][0] = F[5 * n + e];
          fg[u][1] = F[2 * n + e];
          fg[u][2] = F[3 * n + e];
          fg[u][3] = F[4 * n + e];
        }
      }
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        const int t = tb - u;
        if (t < t0) break;
        const StepIn& cu = in[u];
        const float R = cu.g + fmaf(nx.z, nx.lam, nx.v) - cu.lam;
        const float a = nx.d;
        m = max(m, __float_as_uint(fabsf(R)));
        if constexpr (APPLY) {
          const size_t e = base + (size_t)t * D;
          dl = fmaf(a, dl, R);
          const float l = cu.lam + dl;
          lam_new[e] = l;
          const size_t bt = (size_t)b * T + t;
          float* o = dgh + bt * 3 * D;
          o[lane] = fg[u][0] * l;
          o[D + lane] = fg[u][1] * l;
          o[2 * D + lane] = fg[u][2] * l * fg[u][3];
        } else {
          P *= a;
          Q = fmaf(a, Q, R);
        }
        nx = cu;
      }
    }
    if constexpr (!APPLY) agg[((size_t)b * nch + c) * D + lane] = make_float2(P, Q);
  }
  if constexpr (!APPLY) {
    for (int off = 32; off >= 1; off >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, off, 64));
    if (lane == 0) swmax[w] = m;
    __syncthreads();
    if (threadIdx.x == 0) atomicMax(rmax, max(max(swmax[0], swmax[1]), max(swmax[2], swmax[3])));
  }
}

// carry[b][c][i] = delta at the first step after chunk c (0 after the last chunk).  One
// 64-thread block per (channel, b); lane l takes chunk nch - 1 - (g0 + l), so lane order is
// reverse time, and an inclusive Hillis-Steele scan of the chunk maps through LDS gives
// each lane's carry from the group's.
__global__ void __launch_bounds__(64) gru_bwd_chunk_carry_kernel(const float2* __restrict__ agg,
                                                                 float* __restrict__ carry, int D, int nch) {
  __shared__ float sp[64], sq[64];
  const int i = blockIdx.x, b = blockIdx.y, lane = threadIdx.x;
  float x = 0.f;
  for (int g0 = 0; g0 < nch; g0 += 64) {
    const int c = nch - 1 - (g0 + lane);
    float P = 1.f, Q = 0.f;
    if (c >= 0) {
      const float2 pq = agg[((size_t)b * nch + c) * D + i];
      P = pq.x;
      Q = pq.y;
    }
    for (int off = 1; off < 64; off <<= 1) {
      sp[lane] = P;
      sq[lane] = Q;
      __syncthreads();
      const float pp = lane >= off ? sp[lane - off] : 1.f, pq = lane >= off ? sq[lane - off] : 0.f;
      __syncthreads();
      Q = fmaf(P, pq, Q);
      P *= pp;
    }
    sp[lane] = P;
    sq[lane] = Q;
    __syncthreads();
    const float xin = lane == 0 ? x : fmaf(sp[lane - 1], x, sq[lane - 1]);
    if (c >= 0) carry[((size_t)b * nch + c) * D + i] = xin;
    x = fmaf(sp[63], x, sq[63]);
    __syncthreads();
  }
}

// dh0[b][i] = z[b][0][i] lam[b][0][i] + v[b][0][i]  (J_0^T lam_0)
__global__ void __launch_bounds__(256) gru_bwd_dh0_kernel(const float* __restrict__ F, const float* __restrict__ lam,
                                                          const float* __restrict__ v, float* __restrict__ dh0, int B,
                                                          int T, int D) {
  const int e = blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= B * D) return;
  const int b = e / D, i = e - b * D;
  const size_t s = (size_t)b * T * D + i;
  dh0[e] = v ? fmaf(F[s], lam[s], v[s]) : F[s] * lam[s];
}

// part[s][r] = sum of row r of M over column segment s (segments of ceil(cols / S))
__global__ void __launch_bounds__(256) row_sum_kernel(const float* __restrict__ M, size_t cols, size_t seg,
                                                      float* __restrict__ part) {
  __shared__ float sw[4];
  const size_t r = blockIdx.x, s = blockIdx.y;
  const float* row = M + r * cols;
  const size_t c0 = s * seg, c1 = c0 + seg < cols ? c0 + seg : cols;
  float acc = 0.f;
  for (size_t c = c0 + threadIdx.x; c < c1; c += blockDim.x) acc += row[c];
  for (int off = 32; off >= 1; off >>= 1) acc += __shfl_xor(acc, off, 64);
  if ((threadIdx.x & 63) == 0) sw[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) part[s * gridDim.x + r] = (sw[0] + sw[1]) + (sw[2] + sw[3]);
}

// out[j] = sum_s part[s][j]
__global__ void __launch_bounds__(256) sum_slices_kernel(const float* __restrict__ part, int S, size_t n,
                                                         float* __restrict__ out) {
  for (size_t j = (size_t)blockIdx.x * blockDim.x + threadIdx.x; j < n; j += (size_t)gridDim.x * blockDim.x) {
    float acc = 0.f;
    for (int z = 0; z < S; ++z) acc += part[(size_t)z * n + j];
    out[j] = acc;
  }
}

namespace {
unsigned elementwise_blocks(size_t n) {
  size_t b = (n + 255) / 256;
  if (b > 8192) b = 8192;
  return (unsigned)(b < 1 ? 1 : b);
}
}  // namespace

hipError_t launch_gru_shift_states(const float* h, const float* h0, float* hprev, int B, int T, int D,
                                   hipStream_t st) {
  hipLaunchKernelGGL(gru_shift_states_kernel, dim3(elementwise_blocks((size_t)B * T * D)), dim3(256), 0, st, h, h0,
                     hprev, B, T, D);
  return hipGetLastError();
}

hipError_t launch_gru_bwd_factors(const float* gx, const float* gh, const float* hprev, const float* U, float* F,
                                  size_t n, int D, hipStream_t st) {
  hipLaunchKernelGGL(gru_bwd_factors_kernel, dim3(elementwise_blocks(n)), dim3(256), 0, st, gx, gh, hprev, U, F, n,
                     D);
  return hipGetLastError();
}

hipError_t launch_gru_bwd_gates(const float* F, const float* lam, float* dgh, float* dgx, size_t n, int D,
                                hipStream_t st) {
  hipLaunchKernelGGL(gru_bwd_gates_kernel, dim3(elementwise_blocks(n)), dim3(256), 0, st, F, lam, dgh, dgx, n, D);
  return hipGetLastError();
}

hipError_t launch_gru_bwd_refine(const float* F, const float* lam, const float* v, const float* g, float* lam_new,
                                 float* dgh, float2* agg, float* carry, uint32_t* rmax, int B, int T, int D,
                                 hipStream_t st) {
  if (D > 64) return hipErrorInvalidValue;
  const int nch = (T + kChunk - 1) / kChunk;
  dim3 grid((nch + 3) / 4, B);
  hipLaunchKernelGGL(gru_bwd_chunk_kernel<false>, grid, dim3(256), 0, st, F, lam, v, g, agg, nullptr, nullptr,
                     nullptr, rmax, T, D, nch);
  hipLaunchKernelGGL(gru_bwd_chunk_carry_kernel, dim3(D, B), dim3(64), 0, st, agg, carry, D, nch);
  hipLaunchKernelGGL(gru_bwd_chunk_kernel<true>, grid, dim3(256), 0, st, F, lam, v, g, agg, carry, lam_new, dgh,
                     nullptr, T, D, nch);
  return hipGetLastError();
}

int gru_bwd_chunks(int T) { return (T + kChunk - 1) / kChunk; }

hipError_t launch_gru_bwd_dh0(const float* F, const float* lam, const float* v, float* dh0, int B, int T, int D,
                              hipStream_t st) {
  hipLaunchKernelGGL(gru_bwd_dh0_kernel, dim3((B * D + 255) / 256), dim3(256), 0, st, F, lam, v, dh0, B, T, D);
  return hipGetLastError();
}

hipError_t launch_sum_slices(const float* part, int S, size_t n, float* out, hipStream_t st) {
  hipLaunchKernelGGL(sum_slices_kernel, dim3(elementwise_blocks(n)), dim3(256), 0, st, part, S, n, out);
  return hipGetLastError();
}

// C = A B^T with a long K and a small M x N: the K range is cut into slices, each slice's
// product goes to its own partial [M][N] (one batched launch, plus one for a shorter last
// slice), and the partials are summed.  A [M][K] (lda), B [N][K] (ldb), fp32.
hipError_t launch_gemm_split_k(const float* A, int lda, const float* Bm, int ldb, float* C, int M, int N, int K,
                               float* part, int max_slices, hipStream_t st) {
  int kk = (K + max_slices - 1) / max_slices;
  kk = (kk + 31) / 32 * 32;
  const int full = K / kk, rest = K - full * kk;
  const size_t mn = (size_t)M * N;
  if (full > 0) {
    GemmArgs g{A, Bm, nullptr, part, M, N, kk, (long long)kk, (long long)kk, (long long)mn, lda, ldb, N, full, 0};
    hipError_t e = launch_gemm(PNR_F32, PNR_F32, g, st);
    if (e != hipSuccess) return e;
  }
  if (rest > 0) {
    GemmArgs g{A + (size_t)full * kk, Bm + (size_t)full * kk, nullptr, part + (size_t)full * mn, M, N, rest,
               0, 0, 0, lda, ldb, N, 1, 0};
    hipError_t e = launch_gemm(PNR_F32, PNR_F32, g, st);
    if (e != hipSuccess) return e;
  }
  return launch_sum_slices(part, full + (rest > 0), mn, C, st);
}

hipError_t launch_row_sum(const float* M, int rows, size_t cols, float* out, float* part, hipStream_t st) {
  if (rows <= 0 || !out) return hipSuccess;
  constexpr int S = 32;   // column segments per row
  const size_t seg = (cols + S - 1) / S;
  hipLaunchKernelGGL(row_sum_kernel, dim3(rows, S), dim3(256), 0, st, M, cols, seg, part);
  return launch_sum_slices(part, S, rows, out, st);
}


// ---- the whole refinement loop in one persistent, co-resident grid ----
// Iteration k on the adjoint lam_k (with v_k = U^T dgh(lam_k)):
//   A. each wave, for its fixed chunks: R and the chunk's map delta_{end} -> delta_{start}
//      (as pass 1 above), and max |R| into this iteration's word;
//   grid barrier;
//   B. the waves of a block take one (b, channel) row's chunk maps in groups of 64 (lanes
//      = chunks, reverse time), scan them with lane shuffles and exchange the group totals
//      through LDS: each chunk's carry.  Meanwhile thread 0 reads the residual word;
//   grid barrier; every block then takes the same decision (stop when rho_k <= tol_rel
//      rho_0, on a non-finite rho, or after max_iters updates) and block 0 records it, so
//      the adjoint returned is exactly the one whose residual passed;
//   C. each wave, for its chunks: lam_{k+1} = lam_k + delta from the carry (as pass 3),
//      and v_{k+1} = U^T dgh(lam_{k+1}) for steps t0+1 .. t1 of the chunk [t0, t1) -- the
//      steps whose v the chunk's residuals read, t1 (the first step of the next chunk)
//      included.  The chunk keeps lam_{k+1} at t1 too, so pass A of the next iteration
//      reads nothing another wave wrote and no third barrier is needed.
// Chunk maps and carries cross blocks: written and read with agent-scope atomics (the
// grid barrier orders only those).  Everything else a wave reads it wrote itself.
// v: the 16 staged dgh rows times [U_r; U_z; U_n] on fp32 MFMA (16x16x4, four 16-channel
// column tiles, 48 k-steps over the 3 x 64 padded rows), the k index split across lane
// groups (k = 48 (l / 16) + kk in k-step kk), so a lane's A operands are 48 consecutive
// floats of its row and its B operands for one k-step one 16-byte vector.
constexpr int kLoopWaves = 8;
constexpr int kDgLd = 3 * 64 + 4;   // staged row stride: 16 rows of 16-byte reads hit 64 banks
typedef float v4f_t __attribute__((ext_vector_type(4)));

// RES: every chunk has a wave of its own (B * nch <= waves of the grid).  The chunk's
// per-step constants (g, z, d, f_r, f_z, f_n r), the adjoint and v then stay in the wave's
// registers for the whole launch (v comes back from the MFMA layout through the staging
// rows), and each iteration only stores the new adjoint; every register array is assigned
// in full (rows past a ragged end on clamped, finite inputs, only their effects masked).
// Otherwise a wave loops over its chunks and reads them from the workspace planes.
template <bool RES>
__global__ void __launch_bounds__(64 * kLoopWaves, 1) gru_bwd_loop_kernel(BwdLoopArgs a) {
  static_assert(kChunk == 16, "a chunk is one 16-row MFMA tile");
  // One pool, the operand table first (every read of it a base register plus an immediate
  // offset below 64 KiB):
  //  ufb[kk][l][nt] = U_g[j][16 nt + l % 16], g * 64 + j = 48 (l / 16) + kk (zero past D);
  //  then per wave the staged dgh rows [16][kDgLd].
  __shared__ __align__(16) float pool[48 * 64 * 4 + kLoopWaves * kChunk * kDgLd];
  __shared__ uint32_t s_wmax[kLoopWaves];
  __shared__ float2 s_tot[kLoopWaves];
  __shared__ uint32_t s_rb[2];
  float* const ufb = pool;
  // the wave index is uniform across the wave: saying so keeps every chunk index and base
  // address derived from it in scalar registers
  const int lane = threadIdx.x & 63, wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), tid = threadIdx.x;
  const int D = a.D, T = a.T, nch = a.nch;
  const size_t n = (size_t)a.B * T * D;
  const bool act = lane < D;
  Ctrl* ctrl = a.ctrl;
  for (int idx = tid; idx < 48 * 64 * 4; idx += 64 * kLoopWaves) {
    const int kk = idx >> 8, l = (idx >> 2) & 63, nt = idx & 3;
    const int K = 48 * (l >> 4) + kk, g = K >> 6, j = K & 63, ch = 16 * nt + (l & 15);
    ufb[idx] = (j < D && ch < D) ? a.U[(size_t)(g * D + j) * D + ch] : 0.f;
  }
  __syncthreads();
  const int gw = blockIdx.x * kLoopWaves + wid, nw = gridDim.x * kLoopWaves;
  const int ntask = a.B * nch, nrow = a.B * D;
  // carry scans: groups of 64 chunks per row, waves per row (a power of two up to 8)
  const int ngr = (nch + 63) / 64;
  const int wpr = ngr >= 8 ? 8 : ngr > 2 ? 4 : ngr;
  const int rpb = kLoopWaves / wpr;
  float* const dgw = pool + 48 * 64 * 4 + wid * (kChunk * kDgLd);
  const int m16 = lane & 15, q4 = lane >> 4;
  // RES: the wave's chunk (a wave past the last chunk repeats it with its effects masked)
  const int rtask = min(gw, ntask - 1);
  const bool rlive = gw < ntask && act;
  const int ln = act ? lane : 0;   // the channel whose addresses a lane uses
  const int rb_ = rtask / nch, rc_ = rtask - rb_ * nch;
  const int rt0 = rc_ * kChunk, rt1 = min(T, rt0 + kChunk), rlen = rt1 - rt0;
  const bool rtail = rt1 < T;
  const size_t rbase = (size_t)rb_ * T * D + ln;
  float cg[kChunk], cz[kChunk], cd[kChunk], cfr[kChunk], cfz[kChunk], cfnr[kChunk], lv[kChunk], vr[kChunk];
  float bz = 0.f, bd = 0.f, bfr = 0.f, bfz = 0.f, bfnr = 0.f;   // constants at the step after the chunk
  float blam = 0.f, bv = 0.f;                                   // lam_k and v_k there
  if constexpr (RES) {
#pragma unroll
    for (int u = 0; u < kChunk; ++u) {
      const size_t e = rbase + (size_t)min(rt0 + u, rt1 - 1) * D;
      cg[u] = a.g[e];
      cz[u] = a.F[e];
      cd[u] = a.F[n + e];
      cfz[u] = a.F[2 * n + e];
      cfnr[u] = a.F[3 * n + e] * a.F[4 * n + e];
      cfr[u] = a.F[5 * n + e];
      lv[u] = 0.f;   // lam_0 = 0, v_0 = U^T dgh(0) = 0
      vr[u] = 0.f;
    }
    if (rtail) {
      const size_t e = rbase + (size_t)rt1 * D;
      bz = a.F[e];
      bd = a.F[n + e];
      bfz = a.F[2 * n + e];
      bfnr = a.F[3 * n + e] * a.F[4 * n + e];
      bfr = a.F[5 * n + e];
    }
  }
  int cur = 0;
  uint32_t gen = 0;   // generation of the next grid barrier
  for (int k = 0; k <= a.max_iters; ++k) {
    const float* lam = a.lam[cur];
    const float* vv = a.v[cur];
    // ---- A: residual and chunk maps ----
    uint32_t m = 0;
    if constexpr (RES) {
      float nlam = blam, nv = bv, nz = bz, nd = bd;   // the step after the current one
      float P = 1.f, Q = 0.f;
      uint32_t mloc = 0;
#pragma unroll
      for (int u = kChunk - 1; u >= 0; --u) {
        const bool in = u < rlen;
        const float R = cg[u] + fmaf(nz, nlam, nv) - lv[u];
        mloc = in ? max(mloc, abs_bits(R)) : mloc;
        const float Pn = P * nd, Qn = fmaf(nd, Q, R);
        P = in ? Pn : P;
        Q = in ? Qn : Q;
        nlam = in ? lv[u] : nlam;
        nv = in ? vr[u] : nv;
        nz = in ? cz[u] : nz;
        nd = in ? cd[u] : nd;
      }
      if (rlive) {
        m = mloc;
        float* ag = a.agg + (((size_t)rb_ * D + lane) * nch + rc_) * 2;
        coherent_store(ag, P);
        coherent_store(ag + 1, Q);
      }
    }
    for (int task = RES ? ntask : gw; task < ntask; task += nw) {   // (none with RES)
      const int b = task / nch, c = task - b * nch;
      const int t0 = c * kChunk, t1 = min(T, t0 + kChunk);
      const size_t base = (size_t)b * T * D + lane;
      if (!act) continue;
      // every load of the chunk first (indices clamped into it), then the recurrence
      StepIn in[kChunk];
#pragma unroll
      for (int u = 0; u < kChunk; ++u) in[u] = load_step(a.g, lam, a.F, vv, n, base + (size_t)min(t0 + u, t1 - 1) * D);
      float nlam = 0.f, nv = 0.f, nz = 0.f, nd = 0.f;   // the step after the current one
      if (t1 < T) {
        const size_t e = base + (size_t)t1 * D;
        nlam = a.bnd[(size_t)task * D + lane];
        nv = vv[e];
        nz = a.F[e];
        nd = a.F[n + e];
      }
      float P = 1.f, Q = 0.f;
#pragma unroll
      for (int u = kChunk - 1; u >= 0; --u) {
        if (t0 + u < t1) {
          const float R = in[u].g + fmaf(nz, nlam, nv) - in[u].lam;
          m = max(m, abs_bits(R));
          P *= nd;
          Q = fmaf(nd, Q, R);
          nlam = in[u].lam; nv = in[u].v; nz = in[u].z; nd = in[u].d;
        }
      }
      float* ag = a.agg + (((size_t)b * D + lane) * nch + c) * 2;
      coherent_store(ag, P);
      coherent_store(ag + 1, Q);
    }
    m = wave_max_u32(m);
    if (lane == 0) s_wmax[wid] = m;
    __syncthreads();
    if (tid == 0) {
      uint32_t bm = s_wmax[0];
      for (int w = 1; w < kLoopWaves; ++w) bm = max(bm, s_wmax[w]);
      if (bm) __hip_atomic_fetch_max(&a.rmax[k], bm, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    if (!grid_sync(ctrl, gen)) break;
    // the residual words are read here and the decision taken after B, so that their round
    // trip overlaps B (whose writes are harmless when the loop stops)
    uint32_t rb0 = 0, rbk = 0;
    if (tid == 0) {
      rb0 = __hip_atomic_load(&a.rmax[0], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      rbk = __hip_atomic_load(&a.rmax[k], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }

    // ---- B: carries (delta at the first step after each chunk), lane order = reverse time ----
    for (int r0 = blockIdx.x * rpb; r0 < nrow; r0 += gridDim.x * rpb) {
      const int row = r0 + wid / wpr, sub = wid % wpr;
      const bool live = row < nrow;
      const int b = live ? row / D : 0, i = live ? row - b * D : 0;
      const float* ag = a.agg + ((size_t)b * D + i) * nch * 2;
      float x = 0.f;   // delta after the row's last chunk
      for (int g0 = 0; g0 < ngr; g0 += wpr) {
        const int c = nch - 1 - ((g0 + sub) * 64 + lane);
        float p_ = 1.f, q_ = 0.f;
        if (live && c >= 0) {
          p_ = coherent_load(ag + (size_t)c * 2);
          q_ = coherent_load(ag + (size_t)c * 2 + 1);
        }
        const Aff1 f = wave_inclusive_scan(Aff1{p_, q_}, aff_identity1());
        if (lane == 63) s_tot[wid] = make_float2(f.a, f.b);
        __syncthreads();
        float xg = x;   // after this wave's group
        for (int s2 = wid - sub; s2 < wid; ++s2) xg = fmaf(s_tot[s2].x, xg, s_tot[s2].y);
        const Aff1 before = aff_wave_shr1(f, aff_identity1());
        const float xin = fmaf(before.a, xg, before.b);
        if (live && c >= 0) coherent_store(a.carry + ((size_t)b * nch + c) * D + i, xin);
        for (int s2 = wid - sub; s2 < wid - sub + wpr; ++s2) x = fmaf(s_tot[s2].x, x, s_tot[s2].y);
        __syncthreads();   // the totals are read before the next round writes them
      }
    }
    if (tid == 0) {
      s_rb[0] = rb0;
      s_rb[1] = rbk;
    }
    if (!grid_sync(ctrl, gen)) break;   // (its closing block-wide sync publishes s_rb)
    {
      const double rho = bits_to_rho(s_rb[1]), rho0 = bits_to_rho(s_rb[0]);
      const double tol = a.tol_rel * rho0;
      if (blockIdx.x == 0 && tid == 0) finish_iteration(ctrl, a.hist, rho, k, cur, a.max_iters, tol);
      if (!(rho < __builtin_inf()) || rho <= tol || k >= a.max_iters) break;
    }

    // ---- C: the update and the next v ----
    float* lam_n = a.lam[cur ^ 1];
    float* v_n = a.v[cur ^ 1];
    if constexpr (RES) {
      const float dl0 = coherent_load(a.carry + (size_t)rtask * D + ln);   // delta at t1
      const float lb = blam + dl0;                                         // lam_{k+1} at t1
      // staged row r is dgh at step t0 + 1 + r; row 15 the step after the chunk
      dgw[15 * kDgLd + lane] = act && rtail ? bfr * lb : 0.f;
      dgw[15 * kDgLd + 64 + lane] = act && rtail ? bfz * lb : 0.f;
      dgw[15 * kDgLd + 128 + lane] = act && rtail ? bfnr * lb : 0.f;
      float dl = dl0, nlam = blam, nv = bv, nz = bz, nd = bd;
#pragma unroll
      for (int u = kChunk - 1; u >= 0; --u) {
        const bool in = u < rlen;
        const float R = cg[u] + fmaf(nz, nlam, nv) - lv[u];
        const float dn = fmaf(nd, dl, R);
        dl = in ? dn : dl;
        const float l = lv[u] + dl;
        nlam = in ? lv[u] : nlam;
        nv = in ? vr[u] : nv;
        nz = in ? cz[u] : nz;
        nd = in ? cd[u] : nd;
        lv[u] = l;
        if (u >= 1) {
          const bool st = act && in;
          dgw[(u - 1) * kDgLd + lane] = st ? cfr[u] * l : 0.f;
          dgw[(u - 1) * kDgLd + 64 + lane] = st ? cfz[u] * l : 0.f;
          dgw[(u - 1) * kDgLd + 128 + lane] = st ? cfnr[u] * l : 0.f;
        }
      }
      if (rlive) {
#pragma unroll
        for (int u = 0; u < kChunk; ++u)
          if (u < rlen) lam_n[rbase + (size_t)(rt0 + u) * D] = lv[u];
      }
      blam = lb;
      __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0): the rows are read by every lane
      __builtin_amdgcn_wave_barrier();
      v4f_t acc[4];
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) acc[nt] = v4f_t{0.f, 0.f, 0.f, 0.f};
      const float4* arow = reinterpret_cast<const float4*>(dgw + m16 * kDgLd + 48 * q4);
      const float4* ub = reinterpret_cast<const float4*>(ufb) + lane;
      float4 bcur = ub[0], bnxt = bcur, acur = arow[0], anxt = acur;
#pragma unroll
      for (int kk = 0; kk < 48; ++kk) {
        if (kk + 1 < 48) bnxt = ub[(kk + 1) * 64];
        if ((kk & 3) == 0 && kk + 4 < 48) anxt = arow[(kk >> 2) + 1];
        const float aval = (kk & 3) == 0 ? acur.x : (kk & 3) == 1 ? acur.y : (kk & 3) == 2 ? acur.z : acur.w;
        acc[0] = __builtin_amdgcn_mfma_f32_16x16x4f32(aval, bcur.x, acc[0], 0, 0, 0);
        acc[1] = __builtin_amdgcn_mfma_f32_16x16x4f32(aval, bcur.y, acc[1], 0, 0, 0);
        acc[2] = __builtin_amdgcn_mfma_f32_16x16x4f32(aval, bcur.z, acc[2], 0, 0, 0);
        acc[3] = __builtin_amdgcn_mfma_f32_16x16x4f32(aval, bcur.w, acc[3], 0, 0, 0);
        bcur = bnxt;
        if ((kk & 3) == 3) acur = anxt;
      }
      // V back to lane = channel through the staging rows: row r (step t0 + 1 + r) of
      // channel 16 nt + l % 16 sits in lane l's acc[nt][r - 4 (l / 16)]
      __builtin_amdgcn_s_waitcnt(0xC07F);   // the MFMA operands are read before the rows are reused
      __builtin_amdgcn_wave_barrier();
#pragma unroll
      for (int nt = 0; nt < 4; ++nt)
#pragma unroll
        for (int i = 0; i < 4; ++i) dgw[(4 * q4 + i) * kDgLd + 16 * nt + m16] = acc[nt][i];
      __builtin_amdgcn_s_waitcnt(0xC07F);
      __builtin_amdgcn_wave_barrier();
#pragma unroll
      for (int u = 1; u < kChunk; ++u) vr[u] = dgw[(u - 1) * kDgLd + lane];
      bv = rtail ? dgw[15 * kDgLd + lane] : 0.f;
      __builtin_amdgcn_s_waitcnt(0xC07F);   // read before the next iteration stages its rows
      __builtin_amdgcn_wave_barrier();
    }
    for (int task = RES ? ntask : gw; task < ntask; task += nw) {   // (none with RES)
      const int b = task / nch, c = task - b * nch;
      const int t0 = c * kChunk, t1 = min(T, t0 + kChunk), len = t1 - t0;
      const size_t base = (size_t)b * T * D + lane;
      const bool tail = t1 < T;   // the step after the chunk exists
      // Staged row r holds dgh at step t0 + 1 + r: rows 0 .. len - 2 from the walk, row 15
      // the step after the chunk (zero without one), and in a short last chunk the rows
      // between are zero.
      if (len < kChunk) {
#pragma unroll
        for (int r = 0; r < kChunk; ++r)
          if (r >= len - 1) {
            dgw[r * kDgLd + lane] = 0.f;
            dgw[r * kDgLd + 64 + lane] = 0.f;
            dgw[r * kDgLd + 128 + lane] = 0.f;
          }
      }
      // The chunk in two batches of kBatch steps, latest first.  The first batch's loads
      // are issued before the carry and the boundary step's, so that they share one round
      // trip.
      float dl = 0.f, nlam = 0.f, nv = 0.f, nz = 0.f, nd = 0.f, lb = 0.f;
      for (int h = kChunk / kBatch - 1; h >= 0; --h) {
        const int u0 = h * kBatch;
        StepIn in[kBatch];
        float fg[kBatch][4];   // the gate factors f_r, f_z, f_n, r
        if (act) {
#pragma unroll
          for (int u = 0; u < kBatch; ++u) {
            const size_t e = base + (size_t)min(t0 + u0 + u, t1 - 1) * D;
            in[u] = load_step(a.g, lam, a.F, vv, n, e);
            fg[u][0] = a.F[5 * n + e];
            fg[u][1] = a.F[2 * n + e];
            fg[u][2] = a.F[3 * n + e];
            fg[u][3] = a.F[4 * n + e];
          }
        }
        if (h == kChunk / kBatch - 1) {
          float ft[4] = {0.f, 0.f, 0.f, 0.f};
          if (act) {
            dl = coherent_load(a.carry + (size_t)task * D + lane);   // delta at t1
            if (tail) {
              const size_t e = base + (size_t)t1 * D;
              nlam = a.bnd[(size_t)task * D + lane];
              nv = vv[e];
              nz = a.F[e];
              nd = a.F[n + e];
              ft[0] = a.F[5 * n + e];
              ft[1] = a.F[2 * n + e];
              ft[2] = a.F[3 * n + e];
              ft[3] = a.F[4 * n + e];
            }
          }
          lb = nlam + dl;   // lam_{k+1} at t1
          if (tail) {
            dgw[15 * kDgLd + lane] = act ? ft[0] * lb : 0.f;
            dgw[15 * kDgLd + 64 + lane] = act ? ft[1] * lb : 0.f;
            dgw[15 * kDgLd + 128 + lane] = act ? ft[2] * lb * ft[3] : 0.f;
          }
        }
#pragma unroll
        for (int u = kBatch - 1; u >= 0; --u) {
          const int t = t0 + u0 + u;
          if (t < t1) {
            float l = 0.f;
            if (act) {
              const float R = in[u].g + fmaf(nz, nlam, nv) - in[u].lam;
              dl = fmaf(nd, dl, R);
              l = in[u].lam + dl;
              lam_n[base + (size_t)t * D] = l;
              nlam = in[u].lam; nv = in[u].v; nz = in[u].z; nd = in[u].d;
            }
            const int r = u0 + u - 1;   // the staged row of step t
            if (r >= 0) {
              dgw[r * kDgLd + lane] = act ? fg[u][0] * l : 0.f;
              dgw[r * kDgLd + 64 + lane] = act ? fg[u][1] * l : 0.f;
              dgw[r * kDgLd + 128 + lane] = act ? fg[u][2] * l * fg[u][3] : 0.f;
            }
          }
        }
      }
      if (act && tail) a.bnd[(size_t)task * D + lane] = lb;
      // the rows just written are read back by every lane of this wave
      __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
      __builtin_amdgcn_wave_barrier();
      // lane l ends with V[row 4 (l / 16) + i][channel 16 nt + l % 16]
      v4f_t acc[4];
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) acc[nt] = v4f_t{0.f, 0.f, 0.f, 0.f};
      float4 av[12];
      const float4* arow = reinterpret_cast<const float4*>(dgw + m16 * kDgLd + 48 * q4);
#pragma unroll
      for (int j = 0; j < 12; ++j) av[j] = arow[j];
      const float4* ub = reinterpret_cast<const float4*>(ufb) + lane;
      float4 bcur = ub[0], bnxt = bcur;
#pragma unroll
      for (int kk = 0; kk < 48; ++kk) {
        if (kk + 1 < 48) bnxt = ub[(kk + 1) * 64];
        const float4 a4 = av[kk >> 2];
        const float aval = (kk & 3) == 0 ? a4.x : (kk & 3) == 1 ? a4.y : (kk & 3) == 2 ? a4.z : a4.w;
        acc[0] = __builtin_amdgcn_mfma_f32_16x16x4f32(aval, bcur.x, acc[0], 0, 0, 0);
        acc[1] = __builtin_amdgcn_mfma_f32_16x16x4f32(aval, bcur.y, acc[1], 0, 0, 0);
        acc[2] = __builtin_amdgcn_mfma_f32_16x16x4f32(aval, bcur.z, acc[2], 0, 0, 0);
        acc[3] = __builtin_amdgcn_mfma_f32_16x16x4f32(aval, bcur.w, acc[3], 0, 0, 0);
        bcur = bnxt;
      }
      // row r is step t0 + 1 + r: rows 0 .. len - 2 inside the chunk, row 15 the step after it
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        const int ch = 16 * nt + m16;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = 4 * q4 + i;
          if (ch < D && (r < len - 1 || (r == 15 && tail))) v_n[((size_t)b * T + t0 + 1 + r) * D + ch] = acc[nt][i];
        }
      }
      // the staging rows are rewritten by this wave's next chunk only after these reads
      __builtin_amdgcn_s_waitcnt(0xC07F);
      __builtin_amdgcn_wave_barrier();
    }
    cur ^= 1;
  }
}

hipError_t launch_gru_bwd_loop(const BwdLoopArgs& a, int num_cu, hipStream_t st) {
  if (a.D > 64) return hipErrorInvalidValue;
  constexpr int threads = 64 * kLoopWaves;
  const int per_cu = min(cached_occupancy((const void*)gru_bwd_loop_kernel<true>, 0, threads),
                         cached_occupancy((const void*)gru_bwd_loop_kernel<false>, 0, threads));
  if (per_cu < 1) return hipErrorInvalidConfiguration;
  long g = (long)per_cu * num_cu;
  if (g > kMaxGrid) g = kMaxGrid;
  const long work = ((long)a.B * a.nch + kLoopWaves - 1) / kLoopWaves;
  const bool res = work <= g;   // a wave per chunk
  if (g > work) g = work;
  if (g < 1) g = 1;
  void* args[] = {const_cast<BwdLoopArgs*>(&a)};
  const void* fn = res ? (const void*)gru_bwd_loop_kernel<true> : (const void*)gru_bwd_loop_kernel<false>;
  return launch_persistent(fn, (int)g, 0, args, st, threads);
}

}  // namespace pnr
