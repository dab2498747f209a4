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

// Residual of the adjoint system and the reversed, transposed inputs of the diagonal
// scan, through a 32 (t) x 32 (channel) LDS tile of batch element b:
//   R_t = g_t + z_{t+1} lam_{t+1} + v_{t+1} - lam_t,   a_t = d_{t+1}   (0 past the end)
//   Ar[b*D + i][T-1-t] = a_t,  br[b*D + i][T-1-t] = R_t;  rmax = max |R| (as bits).
__global__ void __launch_bounds__(256) gru_bwd_resid_kernel(const float* __restrict__ F, const float* __restrict__ lam,
                                                            const float* __restrict__ v, const float* __restrict__ g,
                                                            float* __restrict__ Ar, float* __restrict__ br,
                                                            uint32_t* __restrict__ rmax, int T, int D) {
  __shared__ float sR[32][33], sA[32][33];
  __shared__ uint32_t swmax[4];
  const size_t n = (size_t)gridDim.z * T * D;
  const int b = blockIdx.z, t0 = blockIdx.x * 32, i0 = blockIdx.y * 32;
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;   // 32 x 8
  uint32_t m = 0;
  for (int k = ty; k < 32; k += 8) {
    const int t = t0 + k, i = i0 + tx;
    float R = 0.f, a = 0.f;
    if (t < T && i < D) {
      const size_t e = ((size_t)b * T + t) * D + i;
      R = g[e] - lam[e];
      if (t + 1 < T) {
        const size_t e1 = e + D;
        R += fmaf(F[e1], lam[e1], v[e1]);
        a = F[n + e1];
      }
      m = max(m, __float_as_uint(fabsf(R)));
    }
    sR[k][tx] = R;
    sA[k][tx] = a;
  }
  __syncthreads();
  for (int k = ty; k < 32; k += 8) {
    const int i = i0 + k, t = t0 + tx;
    if (t < T && i < D) {
      const size_t o = ((size_t)b * D + i) * T + (T - 1 - t);
      Ar[o] = sA[tx][k];
      br[o] = sR[tx][k];
    }
  }
  // block max of |R|, then one atomic per block
  for (int off = 32; off >= 1; off >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, off, 64));
  if ((threadIdx.x & 63) == 0) swmax[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    m = max(max(swmax[0], swmax[1]), max(swmax[2], swmax[3]));
    atomicMax(rmax, m);
  }
}

// lam[b][t][i] += dr[b*D + i][T-1-t], and the recurrent-gate gradients of the new lam
// (dgh as in gru_bwd_gates_kernel) for the next residual
__global__ void __launch_bounds__(256) gru_bwd_update_kernel(const float* __restrict__ dr, float* __restrict__ lam,
                                                             const float* __restrict__ F, float* __restrict__ dgh,
                                                             int T, int D) {
  __shared__ float s[32][33];
  const size_t n = (size_t)gridDim.z * T * D;
  const int b = blockIdx.z, t0 = blockIdx.x * 32, i0 = blockIdx.y * 32;
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;
  for (int k = ty; k < 32; k += 8) {
    const int i = i0 + k, t = t0 + tx;
    s[k][tx] = (t < T && i < D) ? dr[((size_t)b * D + i) * T + (T - 1 - t)] : 0.f;
  }
  __syncthreads();
  for (int k = ty; k < 32; k += 8) {
    const int t = t0 + k, i = i0 + tx;
    if (t < T && i < D) {
      const size_t bt = (size_t)b * T + t, e = bt * D + i;
      const float l = lam[e] + s[tx][k];
      lam[e] = l;
      float* o = dgh + bt * 3 * D;
      o[i] = F[5 * n + e] * l;
      o[D + i] = F[2 * n + e] * l;
      o[2 * D + i] = F[3 * n + e] * l * F[4 * n + e];
    }
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

// out[r] = sum_c M[r][c]: one block per row
__global__ void __launch_bounds__(256) row_sum_kernel(const float* __restrict__ M, size_t cols, float* __restrict__ out) {
  __shared__ float sw[4];
  const float* row = M + (size_t)blockIdx.x * cols;
  float s = 0.f;
  for (size_t c = threadIdx.x; c < cols; c += blockDim.x) s += row[c];
  for (int off = 32; off >= 1; off >>= 1) s += __shfl_xor(s, off, 64);
  if ((threadIdx.x & 63) == 0) sw[threadIdx.x >> 6] = s;
  __syncthreads();
  if (threadIdx.x == 0) out[blockIdx.x] = (sw[0] + sw[1]) + (sw[2] + sw[3]);
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

hipError_t launch_gru_bwd_resid(const float* F, const float* lam, const float* v, const float* g, float* Ar,
                                float* br, uint32_t* rmax, int B, int T, int D, hipStream_t st) {
  dim3 grid((T + 31) / 32, (D + 31) / 32, B);
  hipLaunchKernelGGL(gru_bwd_resid_kernel, grid, dim3(256), 0, st, F, lam, v, g, Ar, br, rmax, T, D);
  return hipGetLastError();
}

hipError_t launch_gru_bwd_update(const float* dr, float* lam, const float* F, float* dgh, int B, int T, int D,
                                 hipStream_t st) {
  dim3 grid((T + 31) / 32, (D + 31) / 32, B);
  hipLaunchKernelGGL(gru_bwd_update_kernel, grid, dim3(256), 0, st, dr, lam, F, dgh, T, D);
  return hipGetLastError();
}

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

hipError_t launch_row_sum(const float* M, int rows, size_t cols, float* out, hipStream_t st) {
  if (rows <= 0 || !out) return hipSuccess;
  hipLaunchKernelGGL(row_sum_kernel, dim3(rows), dim3(256), 0, st, M, cols, out);
  return hipGetLastError();
}

}  // namespace pnr
