// ELK proper for the LSTM with elementwise recurrent weights: the damped (Levenberg-
// Marquardt) Newton step with the exact 2x2 Jacobian block of every channel ("Towards
// Scalable and Stable Parallelization of Nonlinear RNNs", abstract and the summary's
// "Approach": a trust region whose linear-Gaussian MAP solve is a Kalman filter and
// smoother, computed in parallel).
//
// Per channel the step D (2 components: c and h) minimises
//   sum_t |D_t - J_t D_{t-1} - r_t|^2 + lam sum_t |D_t|^2,     D_0 = 0,
// the smoothed mean of the state-space model D_t = J_t D_{t-1} + r_t + w_t (w ~ N(0, I)),
// 0 = D_t + v_t (v ~ N(0, I / lam)).  With 2x2 covariances the scalar kernel's homogeneous
// form would need J^{-1}; the filter is instead one associative scan of the filtering
// elements of Sarkka and Garcia-Fernandez ("Temporal Parallelization of Bayesian
// Smoothers", IEEE TAC 2021): per step (A, b, C, eta, Jm), here with H = I, Q = I,
// R = I / lam and a = 1 / (1 + lam):
//   A = a J,  b = a r,  C = a I,  eta = -lam a J^T r,  Jm = lam a J^T J
// (at the first step J counts as 0: D_0 = 0 is known exactly), combined by
//   M = (I + C_i Jm_j)^{-1}
//   A_ij = A_j M A_i,  b_ij = A_j M (b_i + C_i eta_j) + b_j,  C_ij = A_j M C_i A_j^T + C_j,
//   eta_ij = A_i^T M^T (eta_j - Jm_j b_i) + eta_i,  Jm_ij = A_i^T M^T Jm_j A_i + Jm_i
// (i earlier, j later; I + C Jm is invertible since C and Jm are positive semidefinite).
// A prefix from the first step has A = 0, and its (b, C) is the filtered mean m_t and
// covariance P_t.  The RTS smoother, rewritten in new-iterate space as in the scalar
// kernel,
//   h'_t = G_t h'_{t+1} + e_t,  G_t = P_t J_{t+1}^T (J_{t+1} P_t J_{t+1}^T + I)^{-1},
//   e_t = m_t + h_t - G_t (J_{t+1} m_t + r_{t+1} + h_{t+1})    (G = 0, e = m + h at the end)
// is one affine scan of 2x2 maps run backwards in time.  One block walks a whole row
// (channel), forward then backward; the forward sweep stores G (4 planes) and e (2).
#include "common.h"
#include "diag_cell.h"
#include "kernels.h"

namespace pnr {

struct KElem {   // filtering element: A (2x2), b, C (symmetric), eta, Jm (symmetric)
  float a00, a01, a10, a11, b0, b1, c00, c01, c11, e0, e1, j00, j01, j11;
};
struct KState {  // filtered mean and covariance after a step
  float m0, m1, p00, p01, p11;
};

// later o earlier, in the scan's compose(later, earlier) convention
__device__ __forceinline__ KElem compose(const KElem& j, const KElem& i) {
  // M = (I + C_i Jm_j)^{-1}
  const float x00 = 1.f + i.c00 * j.j00 + i.c01 * j.j01, x01 = i.c00 * j.j01 + i.c01 * j.j11;
  const float x10 = i.c01 * j.j00 + i.c11 * j.j01, x11 = 1.f + i.c01 * j.j01 + i.c11 * j.j11;
  const float id = 1.f / (x00 * x11 - x01 * x10);
  const float m00 = x11 * id, m01 = -x01 * id, m10 = -x10 * id, m11 = x00 * id;
  // AM = A_j M
  const float am00 = j.a00 * m00 + j.a01 * m10, am01 = j.a00 * m01 + j.a01 * m11;
  const float am10 = j.a10 * m00 + j.a11 * m10, am11 = j.a10 * m01 + j.a11 * m11;
  KElem o;
  o.a00 = am00 * i.a00 + am01 * i.a10; o.a01 = am00 * i.a01 + am01 * i.a11;
  o.a10 = am10 * i.a00 + am11 * i.a10; o.a11 = am10 * i.a01 + am11 * i.a11;
  const float v0 = i.b0 + i.c00 * j.e0 + i.c01 * j.e1, v1 = i.b1 + i.c01 * j.e0 + i.c11 * j.e1;
  o.b0 = am00 * v0 + am01 * v1 + j.b0;
  o.b1 = am10 * v0 + am11 * v1 + j.b1;
  // C_ij = (AM C_i) A_j^T + C_j
  const float w00 = am00 * i.c00 + am01 * i.c01, w01 = am00 * i.c01 + am01 * i.c11;
  const float w10 = am10 * i.c00 + am11 * i.c01, w11 = am10 * i.c01 + am11 * i.c11;
  o.c00 = w00 * j.a00 + w01 * j.a01 + j.c00;
  o.c01 = w00 * j.a10 + w01 * j.a11 + j.c01;
  o.c11 = w10 * j.a10 + w11 * j.a11 + j.c11;
  // eta_ij = A_i^T M^T (eta_j - Jm_j b_i) + eta_i
  const float y0 = j.e0 - (j.j00 * i.b0 + j.j01 * i.b1), y1 = j.e1 - (j.j01 * i.b0 + j.j11 * i.b1);
  const float z0 = m00 * y0 + m10 * y1, z1 = m01 * y0 + m11 * y1;
  o.e0 = i.a00 * z0 + i.a10 * z1 + i.e0;
  o.e1 = i.a01 * z0 + i.a11 * z1 + i.e1;
  // Jm_ij = A_i^T (M^T Jm_j) A_i + Jm_i
  const float n00 = m00 * j.j00 + m10 * j.j01, n01 = m00 * j.j01 + m10 * j.j11;
  const float n10 = m01 * j.j00 + m11 * j.j01, n11 = m01 * j.j01 + m11 * j.j11;
  const float q00 = n00 * i.a00 + n01 * i.a10, q01 = n00 * i.a01 + n01 * i.a11;
  const float q10 = n10 * i.a00 + n11 * i.a10, q11 = n10 * i.a01 + n11 * i.a11;
  o.j00 = i.a00 * q00 + i.a10 * q10 + i.j00;
  o.j01 = i.a00 * q01 + i.a10 * q11 + i.j01;
  o.j11 = i.a01 * q01 + i.a11 * q11 + i.j11;
  return o;
}

// a filter state pushed through an element: the state as the element with A = 0
__device__ __forceinline__ KState push(const KState& s, const KElem& j) {
  const float x00 = 1.f + s.p00 * j.j00 + s.p01 * j.j01, x01 = s.p00 * j.j01 + s.p01 * j.j11;
  const float x10 = s.p01 * j.j00 + s.p11 * j.j01, x11 = 1.f + s.p01 * j.j01 + s.p11 * j.j11;
  const float id = 1.f / (x00 * x11 - x01 * x10);
  const float m00 = x11 * id, m01 = -x01 * id, m10 = -x10 * id, m11 = x00 * id;
  const float am00 = j.a00 * m00 + j.a01 * m10, am01 = j.a00 * m01 + j.a01 * m11;
  const float am10 = j.a10 * m00 + j.a11 * m10, am11 = j.a10 * m01 + j.a11 * m11;
  const float v0 = s.m0 + s.p00 * j.e0 + s.p01 * j.e1, v1 = s.m1 + s.p01 * j.e0 + s.p11 * j.e1;
  const float w00 = am00 * s.p00 + am01 * s.p01, w01 = am00 * s.p01 + am01 * s.p11;
  const float w10 = am10 * s.p00 + am11 * s.p01, w11 = am10 * s.p01 + am11 * s.p11;
  return KState{am00 * v0 + am01 * v1 + j.b0, am10 * v0 + am11 * v1 + j.b1,
                w00 * j.a00 + w01 * j.a01 + j.c00, w00 * j.a10 + w01 * j.a11 + j.c01,
                w10 * j.a10 + w11 * j.a11 + j.c11};
}

template <>
__device__ __forceinline__ KElem select_aff(bool take, const KElem& a, const KElem& b) {
  return KElem{take ? a.a00 : b.a00, take ? a.a01 : b.a01, take ? a.a10 : b.a10, take ? a.a11 : b.a11,
               take ? a.b0 : b.b0,   take ? a.b1 : b.b1,   take ? a.c00 : b.c00, take ? a.c01 : b.c01,
               take ? a.c11 : b.c11, take ? a.e0 : b.e0,   take ? a.e1 : b.e1,   take ? a.j00 : b.j00,
               take ? a.j01 : b.j01, take ? a.j11 : b.j11};
}
__device__ __forceinline__ KElem shfl_row_shr_aff(const KElem& v, const KElem& id, int s) {
  KElem o;
#define PNR_DPP14(C)                                                                              \
  o.a00 = dpp_f<C>(id.a00, v.a00); o.a01 = dpp_f<C>(id.a01, v.a01); o.a10 = dpp_f<C>(id.a10, v.a10); \
  o.a11 = dpp_f<C>(id.a11, v.a11); o.b0 = dpp_f<C>(id.b0, v.b0);    o.b1 = dpp_f<C>(id.b1, v.b1);    \
  o.c00 = dpp_f<C>(id.c00, v.c00); o.c01 = dpp_f<C>(id.c01, v.c01); o.c11 = dpp_f<C>(id.c11, v.c11); \
  o.e0 = dpp_f<C>(id.e0, v.e0);    o.e1 = dpp_f<C>(id.e1, v.e1);    o.j00 = dpp_f<C>(id.j00, v.j00); \
  o.j01 = dpp_f<C>(id.j01, v.j01); o.j11 = dpp_f<C>(id.j11, v.j11);
  switch (s) {
    case 1: PNR_DPP14(0x111) break;
    case 2: PNR_DPP14(0x112) break;
    case 4: PNR_DPP14(0x114) break;
    default: PNR_DPP14(0x118) break;
  }
#undef PNR_DPP14
  return o;
}
__device__ __forceinline__ KElem readlane_aff(const KElem& v, int l) {
  return KElem{readlane_f(v.a00, l), readlane_f(v.a01, l), readlane_f(v.a10, l), readlane_f(v.a11, l),
               readlane_f(v.b0, l),  readlane_f(v.b1, l),  readlane_f(v.c00, l), readlane_f(v.c01, l),
               readlane_f(v.c11, l), readlane_f(v.e0, l),  readlane_f(v.e1, l),  readlane_f(v.j00, l),
               readlane_f(v.j01, l), readlane_f(v.j11, l)};
}
__device__ __forceinline__ KElem kelem_identity() {
  return KElem{1.f, 0.f, 0.f, 1.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
}
__device__ __forceinline__ KState wave_shr1(const KState& x, const KState& lane0) {
  return KState{wave_shr1(x.m0, lane0.m0), wave_shr1(x.m1, lane0.m1), wave_shr1(x.p00, lane0.p00),
                wave_shr1(x.p01, lane0.p01), wave_shr1(x.p11, lane0.p11)};
}

// the element of one step (Jacobian J, residual r; J counts as 0 at the row's first step)
__device__ __forceinline__ KElem kelem_step(const Aff2& J, float r0, float r1, float lam, bool first) {
  const float al = 1.f / (1.f + lam), la = lam * al;
  if (first) return KElem{0.f, 0.f, 0.f, 0.f, al * r0, al * r1, al, 0.f, al, 0.f, 0.f, 0.f, 0.f, 0.f};
  return KElem{al * J.a00, al * J.a01, al * J.a10, al * J.a11, al * r0, al * r1, al, 0.f, al,
               -la * (J.a00 * r0 + J.a10 * r1), -la * (J.a01 * r0 + J.a11 * r1),
               la * (J.a00 * J.a00 + J.a10 * J.a10), la * (J.a00 * J.a01 + J.a10 * J.a11),
               la * (J.a01 * J.a01 + J.a11 * J.a11)};
}

// one plain filter step: predict with (J, r) (nothing to predict from at the row's first
// step), then the pseudo-observation 0 with noise I / lam
__device__ __forceinline__ KState kfilter_step(const KState& s, const Aff2& J, float r0, float r1, float lam,
                                               bool first) {
  float pm00, pm01, pm11, mm0, mm1;
  if (first) {
    pm00 = 1.f; pm01 = 0.f; pm11 = 1.f; mm0 = r0; mm1 = r1;
  } else {
    // J P J^T + I
    const float t00 = J.a00 * s.p00 + J.a01 * s.p01, t01 = J.a00 * s.p01 + J.a01 * s.p11;
    const float t10 = J.a10 * s.p00 + J.a11 * s.p01, t11 = J.a10 * s.p01 + J.a11 * s.p11;
    pm00 = t00 * J.a00 + t01 * J.a01 + 1.f;
    pm01 = t00 * J.a10 + t01 * J.a11;
    pm11 = t10 * J.a10 + t11 * J.a11 + 1.f;
    mm0 = J.a00 * s.m0 + J.a01 * s.m1 + r0;
    mm1 = J.a10 * s.m0 + J.a11 * s.m1 + r1;
  }
  // (I + lam P-)^{-1}
  const float q00 = 1.f + lam * pm00, q01 = lam * pm01, q11 = 1.f + lam * pm11;
  const float id = 1.f / (q00 * q11 - q01 * q01);
  const float i00 = q11 * id, i01 = -q01 * id, i11 = q00 * id;
  return KState{i00 * mm0 + i01 * mm1, i01 * mm0 + i11 * mm1, i00 * pm00 + i01 * pm01,
                0.5f * ((i00 * pm01 + i01 * pm11) + (i01 * pm00 + i11 * pm01)), i01 * pm01 + i11 * pm11};
}

// smoother coefficients of a step from its filtered state s and state (c, h), and the next
// step's Jacobian Jn, residual (rn0, rn1) and state (cn, hn); last: the row's last step
__device__ __forceinline__ void kcoeffs(const KState& s, float c, float h, const Aff2& Jn, float rn0, float rn1,
                                        float cn, float hn, bool last, float* G, float* e) {
  if (last) {
    G[0] = G[1] = G[2] = G[3] = 0.f;
    e[0] = s.m0 + c;
    e[1] = s.m1 + h;
    return;
  }
  // Pn = Jn P Jn^T + I, K = P Jn^T, G = K Pn^{-1}
  const float k00 = s.p00 * Jn.a00 + s.p01 * Jn.a01, k01 = s.p00 * Jn.a10 + s.p01 * Jn.a11;
  const float k10 = s.p01 * Jn.a00 + s.p11 * Jn.a01, k11 = s.p01 * Jn.a10 + s.p11 * Jn.a11;
  const float n00 = Jn.a00 * k00 + Jn.a01 * k10 + 1.f, n01 = Jn.a00 * k01 + Jn.a01 * k11;
  const float n11 = Jn.a10 * k01 + Jn.a11 * k11 + 1.f;
  const float id = 1.f / (n00 * n11 - n01 * n01);
  const float i00 = n11 * id, i01 = -n01 * id, i11 = n00 * id;
  G[0] = k00 * i00 + k01 * i01; G[1] = k00 * i01 + k01 * i11;
  G[2] = k10 * i00 + k11 * i01; G[3] = k10 * i01 + k11 * i11;
  const float y0 = Jn.a00 * s.m0 + Jn.a01 * s.m1 + rn0 + cn, y1 = Jn.a10 * s.m0 + Jn.a11 * s.m1 + rn1 + hn;
  e[0] = s.m0 + c - (G[0] * y0 + G[1] * y1);
  e[1] = s.m1 + h - (G[2] * y0 + G[3] * y1);
}

struct Elk2Shared {
  KElem ftot[PNR_WAVES];
  Aff2 btot[PNR_WAVES];
  float nj[PNR_WAVES][4], nr[PNR_WAVES][2], ns[PNR_WAVES][2];   // each wave's first step: J, r, (c, h)
  KState fcarry;     // filter state after the previous tile's last step
  float bcarry[2];   // new iterate (c, h) at the step after the tile (backward sweep)
};

// Forward sweep over one tile: cell, residual, exact 2x2 Jacobian, filter; stores G, e.
template <int N>
__device__ __forceinline__ void elk2_forward_tile(const ElkArgs& a, Elk2Shared& sh, int b, int d, int seg,
                                                  const float* Hcur, bool resid_only, uint32_t& blk_max) {
  using C = DiagCell<PNR_CELL_LSTM_DIAG>;
  constexpr int TILE = PNR_BLOCK * N;
  const int tid = threadIdx.x, wid = tid >> 6, lane = tid & 63;
  const int D = a.D, T = a.T, S = 2 * D;
  const bool vec = (T & 3) == 0;
  const int tb = seg * TILE + tid * N;
  const C::Par q = C::load_par(a.u, a.bh, D, d);
  const size_t coff = ((size_t)b * S + d) * T, hoff = ((size_t)b * S + D + d) * T;
  float g[4][N], c[N], h[N];
#pragma unroll
  for (int gg = 0; gg < 4; ++gg) load_n(a.gx + ((size_t)(b * 4 + gg) * D + d) * T, tb, T, vec, N, g[gg]);
  if (!Hcur) {
#pragma unroll
    for (int i = 0; i < N; ++i) { c[i] = 0.f; h[i] = 0.f; }
  } else {
    load_n(Hcur + coff, tb, T, vec, N, c);
    load_n(Hcur + hoff, tb, T, vec, N, h);
  }
  // the state before the thread's first step: the previous lane's last one (DPP); lane 0 of
  // each wave loads it (this block wrote it, or it is h0 / the zero guess)
  float cp0 = 0.f, hp0 = 0.f;
  if (lane == 0) {
    if (tb == 0) {
      cp0 = a.h0 ? a.h0[(size_t)b * S + d] : 0.f;
      hp0 = a.h0 ? a.h0[(size_t)b * S + D + d] : 0.f;
    } else if (Hcur && tb <= T) {
      cp0 = Hcur[coff + tb - 1];
      hp0 = Hcur[hoff + tb - 1];
    }
  }
  cp0 = wave_shr1(c[N - 1], cp0);
  hp0 = wave_shr1(h[N - 1], hp0);
  Aff2 J[N];
  float r0[N], r1[N];
  uint32_t tmax = 0;
#pragma unroll
  for (int i = 0; i < N; ++i) {
    float gi[4] = {g[0][i], g[1][i], g[2][i], g[3][i]};
    J[i] = aff_identity2();
    C::eval(q, gi, i == 0 ? cp0 : c[i - 1], i == 0 ? hp0 : h[i - 1], c[i], h[i], PNR_JAC_FULL, true, r0[i], r1[i],
            J[i]);
    if (tb + i >= T) { r0[i] = 0.f; r1[i] = 0.f; }
    tmax = max(tmax, max(abs_bits(r0[i]), abs_bits(r1[i])));
  }
  blk_max = max(blk_max, tmax);
  if (resid_only) return;   // uniform over the block
  const float lam = a.lam;
  // ---- filter scan: thread-serial, wave (DPP), block (LDS), carry ----
  KElem agg = kelem_step(J[0], r0[0], r1[0], lam, tb == 0);
#pragma unroll
  for (int i = 1; i < N; ++i)
    if (tb + i < T) agg = compose(kelem_step(J[i], r0[i], r1[i], lam, false), agg);
  const KElem incl = wave_inclusive_scan(agg, kelem_identity());
  if (lane == 63) sh.ftot[wid] = incl;
  if (lane == 0) {
    sh.nj[wid][0] = J[0].a00; sh.nj[wid][1] = J[0].a01; sh.nj[wid][2] = J[0].a10; sh.nj[wid][3] = J[0].a11;
    sh.nr[wid][0] = r0[0]; sh.nr[wid][1] = r1[0];
    sh.ns[wid][0] = c[0]; sh.ns[wid][1] = h[0];
  }
  __syncthreads();
  const int lim = (tid == PNR_BLOCK - 1 && tb + N < T) ? tb + N - 1 : T;
  KState xw = sh.fcarry;   // filter state entering this wave's first step
  // the previous tile's last step: filtered state = the carry, state = (cp0, hp0)
  float dG[4] = {0.f, 0.f, 0.f, 0.f}, dE[2] = {0.f, 0.f};
  if (tid == 0 && seg > 0) kcoeffs(xw, cp0, hp0, J[0], r0[0], r1[0], c[0], h[0], false, dG, dE);
  for (int w = 0; w < wid; ++w) xw = push(xw, sh.ftot[w]);
  KState x = wave_shr1(push(xw, incl), xw);   // entering this thread's first step
  KState xs[N];
#pragma unroll
  for (int i = 0; i < N; ++i) {
    x = kfilter_step(x, J[i], r0[i], r1[i], lam, tb + i == 0);
    xs[i] = x;
  }
  // the step after the thread's last one: the next lane's first; lane 63 takes the next
  // wave's first from LDS
  Aff2 Jn = aff_identity2();
  Jn.a00 = shfl_down_f(J[0].a00, 1); Jn.a01 = shfl_down_f(J[0].a01, 1);
  Jn.a10 = shfl_down_f(J[0].a10, 1); Jn.a11 = shfl_down_f(J[0].a11, 1);
  float rn0 = shfl_down_f(r0[0], 1), rn1 = shfl_down_f(r1[0], 1);
  float cn = shfl_down_f(c[0], 1), hn = shfl_down_f(h[0], 1);
  if (lane == 63 && wid + 1 < PNR_WAVES) {
    Jn.a00 = sh.nj[wid + 1][0]; Jn.a01 = sh.nj[wid + 1][1]; Jn.a10 = sh.nj[wid + 1][2]; Jn.a11 = sh.nj[wid + 1][3];
    rn0 = sh.nr[wid + 1][0]; rn1 = sh.nr[wid + 1][1];
    cn = sh.ns[wid + 1][0]; hn = sh.ns[wid + 1][1];
  }
  float Gv[4][N], Ev[2][N];
#pragma unroll
  for (int i = 0; i < N; ++i) {
    float Gi[4], Ei[2];
    if (i + 1 < N)
      kcoeffs(xs[i], c[i], h[i], J[i + 1], r0[i + 1], r1[i + 1], c[i + 1], h[i + 1], tb + i + 1 >= T, Gi, Ei);
    else
      kcoeffs(xs[i], c[i], h[i], Jn, rn0, rn1, cn, hn, tb + N >= T, Gi, Ei);
#pragma unroll
    for (int qq = 0; qq < 4; ++qq) Gv[qq][i] = Gi[qq];
    Ev[0][i] = Ei[0];
    Ev[1][i] = Ei[1];
  }
#pragma unroll
  for (int qq = 0; qq < 4; ++qq) {
    float* row = a.Gs + ((size_t)(b * 4 + qq) * D + d) * T;
    store_n(row, tb, lim, vec, N, Gv[qq]);
    if (tid == 0 && seg > 0) row[tb - 1] = dG[qq];
  }
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    float* row = a.Es + ((size_t)(b * 2 + k) * D + d) * T;
    store_n(row, tb, lim, vec, N, Ev[k]);
    if (tid == 0 && seg > 0) row[tb - 1] = dE[k];
  }
  __syncthreads();   // everyone has read ftot, nj / nr / ns and fcarry
  if (tid == PNR_BLOCK - 1) sh.fcarry = xs[N - 1];   // the next tile's carry
  __syncthreads();
}

// Backward sweep over one tile: h'_t = G_t h'_{t+1} + e_t.  Thread t takes the run of N
// steps that starts at step (PNR_BLOCK - 1 - t) * N of the tile and walks it backwards.
template <int N>
__device__ __forceinline__ void elk2_backward_tile(const ElkArgs& a, Elk2Shared& sh, int b, int d, int seg,
                                                   float* Hnext) {
  constexpr int TILE = PNR_BLOCK * N;
  const int tid = threadIdx.x, wid = tid >> 6, lane = tid & 63;
  const int D = a.D, T = a.T, S = 2 * D;
  const bool vec = (T & 3) == 0;
  const int tb = seg * TILE + (PNR_BLOCK - 1 - tid) * N;
  float Gv[4][N], Ev[2][N];
#pragma unroll
  for (int qq = 0; qq < 4; ++qq) load_n(a.Gs + ((size_t)(b * 4 + qq) * D + d) * T, tb, T, vec, N, Gv[qq]);
#pragma unroll
  for (int k = 0; k < 2; ++k) load_n(a.Es + ((size_t)(b * 2 + k) * D + d) * T, tb, T, vec, N, Ev[k]);
  // latest step first
  Aff2 e[N];
#pragma unroll
  for (int i = 0; i < N; ++i)
    e[N - 1 - i] = tb + i < T ? Aff2{Gv[0][i], Gv[1][i], Gv[2][i], Gv[3][i], Ev[0][i], Ev[1][i]} : aff_identity2();
  Aff2 agg = e[0];
#pragma unroll
  for (int i = 1; i < N; ++i) agg = compose(e[i], agg);
  const Aff2 incl = wave_inclusive_scan(agg, aff_identity2());
  if (lane == 63) sh.btot[wid] = incl;
  __syncthreads();
  float2 hw = make_float2(sh.bcarry[0], sh.bcarry[1]);   // new iterate after this wave's runs
  for (int w = 0; w < wid; ++w) hw = apply(sh.btot[w], hw);
  float2 hl = wave_shr1(apply(incl, hw), hw);
  float oc[N], oh[N];
#pragma unroll
  for (int i = 0; i < N; ++i) {
    hl = apply(e[i], hl);   // step tb + N - 1 - i
    oc[N - 1 - i] = hl.x;
    oh[N - 1 - i] = hl.y;
  }
  store_n(Hnext + ((size_t)b * S + d) * T, tb, T, vec, N, oc);
  store_n(Hnext + ((size_t)b * S + D + d) * T, tb, T, vec, N, oh);
  __syncthreads();
  if (tid == PNR_BLOCK - 1) {   // the tile's first step
    sh.bcarry[0] = hl.x;
    sh.bcarry[1] = hl.y;
  }
  __syncthreads();
}

template <int N>
__global__ void __launch_bounds__(PNR_BLOCK, 2) elk2_lstm_kernel(ElkArgs a) {
  __shared__ Elk2Shared sh;
  __shared__ uint32_t s_wmax[PNR_WAVES];
  Ctrl* ctrl = a.ctrl;
  const int tid = threadIdx.x, wid = tid >> 6, lane = tid & 63;
  int cur = -1;
  for (int k = 0; k <= a.max_iters; ++k) {
    const bool resid_only = k == a.max_iters;
    const int next = resid_only ? cur : (cur == 0 ? 1 : 0);
    const float* Hcur = cur >= 0 ? a.H[cur] : nullptr;
    float* Hnext = a.H[next < 0 ? 0 : next];
    uint32_t blk_max = 0;
    for (int row = blockIdx.x; row < a.n_rows; row += gridDim.x) {
      const int b = row / a.D, d = row - b * a.D;
      if (tid == 0) sh.fcarry = KState{0.f, 0.f, 0.f, 0.f, 0.f};
      __syncthreads();
      for (int seg = 0; seg < a.tiles_per_row; ++seg)
        elk2_forward_tile<N>(a, sh, b, d, seg, Hcur, resid_only, blk_max);
      if (resid_only) continue;
      if (tid == 0) { sh.bcarry[0] = 0.f; sh.bcarry[1] = 0.f; }
      __syncthreads();
      for (int seg = a.tiles_per_row - 1; seg >= 0; --seg) elk2_backward_tile<N>(a, sh, b, d, seg, Hnext);
      if (__syncthreads_or(has_fault(ctrl))) break;   // the same decision in every wave
    }
    blk_max = wave_max_u32(blk_max);
    if (lane == 0) s_wmax[wid] = blk_max;
    __syncthreads();
    if (tid == 0) {
      uint32_t m = s_wmax[0];
      for (int w = 1; w < PNR_WAVES; ++w) m = max(m, s_wmax[w]);
      __hip_atomic_store(&a.partials[blockIdx.x], m, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    grid_barrier(ctrl, [&]() {
      uint32_t m = 0;
      for (int i = tid; i < (int)gridDim.x; i += PNR_BLOCK)
        m = max(m, __hip_atomic_load(&a.partials[i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
      m = wave_max_u32(m);
      __syncthreads();
      if (lane == 0) s_wmax[wid] = m;
      __syncthreads();
      if (tid == 0) {
        for (int w = 0; w < PNR_WAVES; ++w) m = max(m, s_wmax[w]);
        finish_iteration(ctrl, a.rho_hist, bits_to_rho(m), k, cur, a.max_iters, a.tol);
      }
    });
    if (__hip_atomic_load(&ctrl->done, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) || has_fault(ctrl)) break;
    cur = next;
  }
}

constexpr int kElk2N = 4;

hipError_t launch_elk2_lstm(const ElkArgs& a, int num_cu, hipStream_t st) {
  const void* fn = (const void*)elk2_lstm_kernel<kElk2N>;
  const int per_cu = cached_occupancy(fn, 0);
  if (per_cu < 1) return hipErrorInvalidConfiguration;
  long g = (long)per_cu * num_cu;
  if (g > kMaxGrid) g = kMaxGrid;
  if (g > a.n_rows) g = a.n_rows;
  if (g < 1) g = 1;
  void* args[] = {const_cast<ElkArgs*>(&a)};
  return launch_persistent(fn, (int)g, 0, args, st);
}

}  // namespace pnr
