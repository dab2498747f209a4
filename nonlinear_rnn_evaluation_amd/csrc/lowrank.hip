// Low-rank approximation of the dense GRU's Jacobian factors (ParaRNN overview page,
// "Technical Implementation / Newton's Iteration": approximate-Newton strategies, among
// them low-rank approximations of the Jacobian; the page gives no form).
//
// The exact Jacobian is J_t = diag(z) + diag(al) U_z + diag(be) U_r + diag(ga) U_n.  Here
// each gate block U_g (D x D) is replaced, in the Jacobian only, by its best rank-r
// approximation with its own diagonal restored:
//     U~_g = U_g V_r V_r^T       (V_r: the r leading right singular vectors of U_g)
//     U^_g = U~_g - diag(U~_g) + diag(U_g)
// U_g V_r V_r^T is the truncated singular value decomposition (Eckart-Young).  V_r is
// taken from the eigenvectors of the Gram matrix U_g^T U_g, found by the cyclic Jacobi
// eigenvalue method (Golub & Van Loan, "Matrix Computations", the symmetric Schur
// rotation), with the round-robin ordering of disjoint pairs so that every rotation of a
// round runs in parallel.  One 64-lane block per gate block; D <= 32.  r >= D copies U.
#include "common.h"
#include "kernels.h"

namespace pnr {

constexpr int kLrMaxD = 32;
constexpr int kLrSweeps = 30;

template <typename Tt> __device__ __forceinline__ Tt lr_sqrt(Tt v);
template <> __device__ __forceinline__ float lr_sqrt(float v) { return sqrtf(v); }
template <> __device__ __forceinline__ double lr_sqrt(double v) { return sqrt(v); }
template <typename Tt> __device__ __forceinline__ Tt lr_eps();
template <> __device__ __forceinline__ float lr_eps() { return 1e-7f; }
template <> __device__ __forceinline__ double lr_eps() { return 1e-15; }

template <typename Tt>
__global__ void __launch_bounds__(64) lowrank_kernel(const Tt* __restrict__ U, Tt* __restrict__ Uh, int D, int rank) {
  __shared__ Tt A[kLrMaxD][kLrMaxD + 1];   // the gate block
  __shared__ Tt Gm[kLrMaxD][kLrMaxD + 1];  // Gram matrix, rotated towards diagonal form
  __shared__ Tt V[kLrMaxD][kLrMaxD + 1];   // accumulated rotations: eigenvectors in columns
  __shared__ Tt P[kLrMaxD][kLrMaxD + 1];   // projector V_r V_r^T
  __shared__ Tt rc[kLrMaxD / 2], rs[kLrMaxD / 2];
  __shared__ int rp[kLrMaxD / 2], rq[kLrMaxD / 2];
  __shared__ int keep[kLrMaxD];
  __shared__ int s_done;
  const int g = blockIdx.x, tid = threadIdx.x, nt = blockDim.x;
  const Tt* src = U + (size_t)g * D * D;
  Tt* dst = Uh + (size_t)g * D * D;
  if (rank >= D) {
    for (int i = tid; i < D * D; i += nt) dst[i] = src[i];
    return;
  }
  for (int i = tid; i < D * D; i += nt) A[i / D][i % D] = src[i];
  __syncthreads();
  for (int i = tid; i < D * D; i += nt) {
    const int r = i / D, c = i % D;
    Tt s = 0;
    for (int k = 0; k < D; ++k) s += A[k][r] * A[k][c];
    Gm[r][c] = s;
    V[r][c] = r == c ? Tt(1) : Tt(0);
  }
  __syncthreads();
  // cyclic Jacobi, round-robin pairs: players 0..m-1 on a circle plus the fixed player m
  const int Dp = D + (D & 1), m = Dp - 1, npair = Dp / 2;
  for (int sweep = 0; sweep < kLrSweeps && rank > 0; ++sweep) {
    for (int round = 0; round < m; ++round) {
      if (tid < npair) {
        int p = tid == 0 ? round : (round + tid) % m;
        int q = tid == 0 ? m : (round - tid + m) % m;
        if (p > q) { const int t = p; p = q; q = t; }
        Tt c = 1, s = 0;
        if (q < D) {
          const Tt gpq = Gm[p][q];
          if (gpq != Tt(0)) {
            // symmetric Schur rotation: zero Gm[p][q] of J^T Gm J, J = [[c, s], [-s, c]]
            const Tt tau = (Gm[q][q] - Gm[p][p]) / (Tt(2) * gpq);
            const Tt t = (tau >= Tt(0) ? Tt(1) : Tt(-1)) / (fabs(tau) + lr_sqrt(Tt(1) + tau * tau));
            c = Tt(1) / lr_sqrt(Tt(1) + t * t);
            s = t * c;
          }
        }
        rp[tid] = p; rq[tid] = q < D ? q : p; rc[tid] = c; rs[tid] = q < D ? s : Tt(0);
      }
      __syncthreads();
      // columns: Gm <- Gm J, V <- V J
      for (int i = tid; i < npair * D; i += nt) {
        const int k = i / D, r = i - k * D;
        const int p = rp[k], q = rq[k];
        if (p == q) continue;
        const Tt c = rc[k], s = rs[k];
        const Tt gp = Gm[r][p], gq = Gm[r][q];
        Gm[r][p] = c * gp - s * gq; Gm[r][q] = s * gp + c * gq;
        const Tt vp = V[r][p], vq = V[r][q];
        V[r][p] = c * vp - s * vq; V[r][q] = s * vp + c * vq;
      }
      __syncthreads();
      // rows: Gm <- J^T Gm
      for (int i = tid; i < npair * D; i += nt) {
        const int k = i / D, col = i - k * D;
        const int p = rp[k], q = rq[k];
        if (p == q) continue;
        const Tt c = rc[k], s = rs[k];
        const Tt gp = Gm[p][col], gq = Gm[q][col];
        Gm[p][col] = c * gp - s * gq; Gm[q][col] = s * gp + c * gq;
      }
      __syncthreads();
    }
    // converged when the off-diagonal mass is negligible next to the diagonal
    if (tid == 0) {
      Tt off = 0, on = 0;
      for (int r = 0; r < D; ++r)
        for (int c = 0; c < D; ++c) (r == c ? on : off) += Gm[r][c] * Gm[r][c];
      s_done = off <= lr_eps<Tt>() * lr_eps<Tt>() * on;
    }
    __syncthreads();
    if (s_done) break;
  }
  // the r largest eigenvalues of the Gram matrix (ties by index)
  for (int i = tid; i < D; i += nt) {
    int above = 0;
    for (int j = 0; j < D; ++j) above += Gm[j][j] > Gm[i][i] || (Gm[j][j] == Gm[i][i] && j < i);
    keep[i] = above < rank;
  }
  __syncthreads();
  for (int i = tid; i < D * D; i += nt) {
    const int r = i / D, c = i % D;
    Tt s = 0;
    for (int k = 0; k < D; ++k)
      if (keep[k]) s += V[r][k] * V[c][k];
    P[r][c] = s;
  }
  __syncthreads();
  for (int i = tid; i < D * D; i += nt) {
    const int r = i / D, c = i % D;
    Tt s = 0;
    for (int k = 0; k < D; ++k) s += A[r][k] * P[k][c];
    dst[i] = r == c ? A[r][r] : s;
  }
}

template <typename Tt>
hipError_t launch_lowrank_matrix(const Tt* U, Tt* Uh, int D, int rank, hipStream_t st) {
  if (D > kLrMaxD) return hipErrorInvalidValue;
  hipLaunchKernelGGL(lowrank_kernel<Tt>, dim3(3), dim3(64), 0, st, U, Uh, D, rank);
  return hipGetLastError();
}
template hipError_t launch_lowrank_matrix<float>(const float*, float*, int, int, hipStream_t);
template hipError_t launch_lowrank_matrix<double>(const double*, double*, int, int, hipStream_t);

}  // namespace pnr
