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
constexpr int kChunk = 32;
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
  dh0[e] = fmaf(F[s], lam[s], v[s]);
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

}  // namespace pnr
