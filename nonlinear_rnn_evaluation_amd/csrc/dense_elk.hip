// Damped (Levenberg-Marquardt) step for the GRU with a dense recurrent matrix U, with the
// diagonal Jacobian: quasi-ELK ("Towards Scalable and Stable Parallelization of Nonlinear
// RNNs", abstract and the summary's "Approach": a trust region whose linear-Gaussian MAP
// solve is a Kalman filter and smoother; with the diagonal Jacobian, quasi-ELK).
//
// One iteration on the iterate H [B][T][D]:
//   1. gh = h_{t-1} U^T + b_h for every step: one MFMA GEMM (the channels couple only here);
//   2. the cell: residual R_t = f(h_{t-1}, x_t) - h_t and J_t = diag(df/dh) (quasi), max |R|;
//   3. per channel the scalar filter P- = J^2 P + 1, m- = J m + R, P = P- / (1 + lam P-),
//      m = m- / (1 + lam P-) -- a forward scan of 3x3 maps in homogeneous coordinates --
//      and from it the smoother's gain and offset in new-iterate space,
//        G_t = P_t J_{t+1} / P-_{t+1},  e_t = m_t + h_t - G_t (m-_{t+1} + h_{t+1})
//      (G = 0, e = m + h at the last step);
//   4. the smoother h'_t = G_t h'_{t+1} + e_t, a backward affine scan, writes the next
//      iterate.
// The scans run over chunks of kEChunk steps in the [B][T][D] layout: one wave per chunk,
// one lane per channel (D <= 64); each scan is an aggregate pass, a carry pass along the
// chunks of each channel, and an apply pass.
#include "common.h"
#include "kernels.h"

namespace pnr {

constexpr int kEChunk = 32;
constexpr int kEBatch = 8;   // steps whose loads are issued together

int elk_dense_chunks(int T) { return (T + kEChunk - 1) / kEChunk; }

// Residual and quasi Jacobian at the iterate (H == nullptr: the zero guess).  A block
// covers 4 steps (rows of B*T) x 64 channels (D <= 64).
__global__ void __launch_bounds__(256) gru_elk_cell_kernel(const float* __restrict__ gx, const float* __restrict__ gh,
                                                           const float* __restrict__ hprev,
                                                           const float* __restrict__ H, const float* __restrict__ U,
                                                           float* __restrict__ R, float* __restrict__ J,
                                                           uint32_t* __restrict__ rmax, size_t rows, int D) {
  __shared__ uint32_t swmax[4];
  const int i = threadIdx.x & 63, w = threadIdx.x >> 6;
  uint32_t m = 0;
  // rows walked grid-stride, so that one atomic per block stays cheap
  for (size_t bt = (size_t)blockIdx.x * 4 + w; bt < rows && i < D; bt += (size_t)gridDim.x * 4) {
    const size_t e = bt * D + i;
    const float* gxr = gx + bt * 3 * D;
    const float* ghr = gh + bt * 3 * D;
    const float r = sigm(gxr[i] + ghr[i]);
    const float z = sigm(gxr[D + i] + ghr[D + i]);
    const float ghn = ghr[2 * D + i];
    const float nn = tanh_(fmaf(r, ghn, gxr[2 * D + i]));
    const float p = hprev[e];
    const float res = fmaf(z, p - nn, nn) - (H ? H[e] : 0.f);
    const float fz = (p - nn) * z * (1.f - z);
    const float fn = (1.f - z) * (1.f - nn * nn);
    J[e] = z + fz * U[(size_t)(D + i) * D + i] + fn * r * U[(size_t)(2 * D + i) * D + i] +
           fn * ghn * r * (1.f - r) * U[(size_t)i * D + i];
    R[e] = res;
    m = max(m, __float_as_uint(fabsf(res)));
  }
  for (int off = 32; off >= 1; off >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, off, 64));
  if (i == 0) swmax[w] = m;
  __syncthreads();
  if (threadIdx.x == 0) atomicMax(rmax, max(max(swmax[0], swmax[1]), max(swmax[2], swmax[3])));
}

__device__ __forceinline__ Flt filter_step(float j, float r, float lam) {
  const float j2 = j * j;
  return Flt{j2, 1.f, lam * j2, 1.f + lam, 0.f, r, j};
}

// Filter: APPLY = false composes each chunk's maps into agg[b][c][7][D]; APPLY = true
// walks the chunk from its carry (u, n with v = 1: carry[b][c][2][D]) and writes the
// smoother's gain and offset per step.
template <bool APPLY>
__global__ void __launch_bounds__(256) gru_elk_filter_kernel(const float* __restrict__ J, const float* __restrict__ R,
                                                             const float* __restrict__ H, float lam,
                                                             float* __restrict__ agg, const float* __restrict__ carry,
                                                             float* __restrict__ Gc, float* __restrict__ Ec, int T,
                                                             int D, int nch) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int b = blockIdx.y, c = blockIdx.x * 4 + w;
  if (c >= nch || lane >= D) return;
  const int t0 = c * kEChunk, t1 = min(T, t0 + kEChunk);
  const size_t base = (size_t)b * T * D + lane;
  const size_t cb = ((size_t)b * nch + c);
  if constexpr (!APPLY) {
    Flt a = flt_identity();
    for (int tb = t0; tb < t1; tb += kEBatch) {
      float jv[kEBatch], rv[kEBatch];
#pragma unroll
      for (int u = 0; u < kEBatch; ++u) {
        const size_t e = base + (size_t)min(tb + u, t1 - 1) * D;
        jv[u] = J[e];
        rv[u] = R[e];
      }
#pragma unroll
      for (int u = 0; u < kEBatch; ++u)
        if (tb + u < t1) a = compose(filter_step(jv[u], rv[u], lam), a);
    }
    float* o = agg + cb * 7 * D + lane;
    o[0] = a.a; o[D] = a.b; o[2 * D] = a.c; o[3 * D] = a.d; o[4 * D] = a.e; o[5 * D] = a.f; o[6 * D] = a.g;
  } else {
    V3 x{carry[cb * 2 * D + lane], 1.f, carry[cb * 2 * D + D + lane]};
    // this step's J, R, h and the next step's (for the coefficients)
    float jc = J[base + (size_t)t0 * D], rc = R[base + (size_t)t0 * D], hc = H ? H[base + (size_t)t0 * D] : 0.f;
    for (int tb = t0; tb < t1; tb += kEBatch) {
      float jn[kEBatch], rn[kEBatch], hn[kEBatch];
#pragma unroll
      for (int u = 0; u < kEBatch; ++u) {
        const size_t e = base + (size_t)min(tb + u + 1, T - 1) * D;
        jn[u] = J[e];
        rn[u] = R[e];
        hn[u] = H ? H[e] : 0.f;
      }
#pragma unroll
      for (int u = 0; u < kEBatch; ++u) {
        const int t = tb + u;
        if (t >= t1) break;
        x = normalized(apply(filter_step(jc, rc, lam), x));
        const float P = x.u, m = x.n;
        float G = 0.f, e = m + hc;
        if (t + 1 < T) {
          G = P * jn[u] * fast_rcp(fmaf(jn[u] * jn[u], P, 1.f));
          e = (m + hc) - G * (fmaf(jn[u], m, rn[u]) + hn[u]);
        }
        const size_t o = base + (size_t)t * D;
        Gc[o] = G;
        Ec[o] = e;
        jc = jn[u];
        rc = rn[u];
        hc = hn[u];
      }
    }
  }
}

// Filter carry along the chunks of one channel (one 64-thread block per (channel, b)):
// the state (u, 1, n) entering each chunk.  Lanes take 64 chunks at a time; an inclusive
// Hillis-Steele scan of their maps through LDS (lane order = time) gives each lane's
// entering state from the group's.
__global__ void __launch_bounds__(64) gru_elk_filter_carry_kernel(const float* __restrict__ agg,
                                                                  float* __restrict__ carry, int D, int nch) {
  __shared__ Flt sm[64];
  const int i = blockIdx.x, b = blockIdx.y, lane = threadIdx.x;
  V3 x{0.f, 1.f, 0.f};   // entering the group
  for (int g0 = 0; g0 < nch; g0 += 64) {
    const int c = g0 + lane;
    Flt F = flt_identity();
    if (c < nch) {
      const float* a = agg + ((size_t)b * nch + c) * 7 * D + i;
      F = Flt{a[0], a[D], a[2 * D], a[3 * D], a[4 * D], a[5 * D], a[6 * D]};
    }
    for (int off = 1; off < 64; off <<= 1) {
      sm[lane] = F;
      __syncthreads();
      const Flt prev = lane >= off ? sm[lane - off] : flt_identity();
      __syncthreads();
      F = compose(F, prev);
    }
    sm[lane] = F;
    __syncthreads();
    const V3 xin = lane == 0 ? x : normalized(apply(sm[lane - 1], x));
    if (c < nch) {
      const size_t cb = (size_t)b * nch + c;
      carry[cb * 2 * D + i] = xin.u;
      carry[cb * 2 * D + D + i] = xin.n;
    }
    x = normalized(apply(sm[63], x));
    __syncthreads();
  }
}

// Smoother h'_t = G_t h'_{t+1} + e_t, backwards: APPLY = false composes each chunk's map
// h'_{end} -> h'_{start} into agg2[b][c][2][D]; APPLY = true writes h' from the carry.
template <bool APPLY>
__global__ void __launch_bounds__(256) gru_elk_smooth_kernel(const float* __restrict__ Gc, const float* __restrict__ Ec,
                                                             float* __restrict__ agg2, const float* __restrict__ carry2,
                                                             float* __restrict__ Hn, int T, int D, int nch) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int b = blockIdx.y, c = blockIdx.x * 4 + w;
  if (c >= nch || lane >= D) return;
  const int t0 = c * kEChunk, t1 = min(T, t0 + kEChunk);
  const size_t base = (size_t)b * T * D + lane;
  const size_t cb = ((size_t)b * nch + c);
  float P = 1.f, Q = 0.f, x = APPLY ? carry2[cb * D + lane] : 0.f;
  for (int tb = t1 - 1; tb >= t0; tb -= kEBatch) {
    float gv[kEBatch], ev[kEBatch];
#pragma unroll
    for (int u = 0; u < kEBatch; ++u) {
      const size_t e = base + (size_t)max(tb - u, t0) * D;
      gv[u] = Gc[e];
      ev[u] = Ec[e];
    }
#pragma unroll
    for (int u = 0; u < kEBatch; ++u) {
      const int t = tb - u;
      if (t < t0) break;
      if constexpr (APPLY) {
        x = fmaf(gv[u], x, ev[u]);
        Hn[base + (size_t)t * D] = x;
      } else {
        P *= gv[u];
        Q = fmaf(gv[u], Q, ev[u]);
      }
    }
  }
  if constexpr (!APPLY) {
    agg2[cb * 2 * D + lane] = P;
    agg2[cb * 2 * D + D + lane] = Q;
  }
}

// Smoother carry along the chunks of one channel, backwards in time: lane l takes chunk
// nch - 1 - (g0 + l), so lane order is reverse time and the same lane scan applies.
__global__ void __launch_bounds__(64) gru_elk_smooth_carry_kernel(const float* __restrict__ agg2,
                                                                  float* __restrict__ carry2, int D, int nch) {
  __shared__ float sp[64], sq[64];
  const int i = blockIdx.x, b = blockIdx.y, lane = threadIdx.x;
  float x = 0.f;   // h' at the step after the group (none after the last chunk)
  for (int g0 = 0; g0 < nch; g0 += 64) {
    const int c = nch - 1 - (g0 + lane);
    float P = 1.f, Q = 0.f;
    if (c >= 0) {
      const size_t cb = (size_t)b * nch + c;
      P = agg2[cb * 2 * D + i];
      Q = agg2[cb * 2 * D + D + i];
    }
    for (int off = 1; off < 64; off <<= 1) {
      sp[lane] = P;
      sq[lane] = Q;
      __syncthreads();
      const float pp = lane >= off ? sp[lane - off] : 1.f, pq = lane >= off ? sq[lane - off] : 0.f;
      __syncthreads();
      Q = fmaf(P, pq, Q);   // (P, Q) o (pp, pq)
      P *= pp;
    }
    sp[lane] = P;
    sq[lane] = Q;
    __syncthreads();
    const float xin = lane == 0 ? x : fmaf(sp[lane - 1], x, sq[lane - 1]);
    if (c >= 0) carry2[((size_t)b * nch + c) * D + i] = xin;
    x = fmaf(sp[63], x, sq[63]);
    __syncthreads();
  }
}

hipError_t launch_gru_elk_cell(const float* gx, const float* gh, const float* hprev, const float* H, const float* U,
                               float* R, float* J, uint32_t* rmax, size_t n, int D, hipStream_t st) {
  if (D > 64) return hipErrorInvalidValue;
  const size_t rows = n / D;
  size_t blocks = (rows + 3) / 4;
  if (blocks > 1024) blocks = 1024;
  hipLaunchKernelGGL(gru_elk_cell_kernel, dim3((unsigned)blocks), dim3(256), 0, st, gx, gh, hprev, H, U, R, J, rmax,
                     rows, D);
  return hipGetLastError();
}

hipError_t launch_gru_elk_step(const float* J, const float* R, const float* H, float lam, float* agg, float* carry,
                               float* Gc, float* Ec, float* agg2, float* carry2, float* Hn, int B, int T, int D,
                               hipStream_t st) {
  if (D > 64) return hipErrorInvalidValue;
  const int nch = elk_dense_chunks(T);
  dim3 grid((nch + 3) / 4, B);
  hipLaunchKernelGGL(gru_elk_filter_kernel<false>, grid, dim3(256), 0, st, J, R, H, lam, agg, nullptr, nullptr,
                     nullptr, T, D, nch);
  hipLaunchKernelGGL(gru_elk_filter_carry_kernel, dim3(D, B), dim3(64), 0, st, agg, carry, D, nch);
  hipLaunchKernelGGL(gru_elk_filter_kernel<true>, grid, dim3(256), 0, st, J, R, H, lam, agg, carry, Gc, Ec, T, D,
                     nch);
  hipLaunchKernelGGL(gru_elk_smooth_kernel<false>, grid, dim3(256), 0, st, Gc, Ec, agg2, nullptr, nullptr, T, D, nch);
  hipLaunchKernelGGL(gru_elk_smooth_carry_kernel, dim3(D, B), dim3(64), 0, st, agg2, carry2, D, nch);
  hipLaunchKernelGGL(gru_elk_smooth_kernel<true>, grid, dim3(256), 0, st, Gc, Ec, agg2, carry2, Hn, T, D, nch);
  return hipGetLastError();
}

}  // namespace pnr
