// Cells with elementwise recurrent weights (GRU_DIAG, LSTM_DIAG) and the per-thread helpers
// the kernels that stream their time-contiguous rows share: the cell, its residual and
// exact Jacobian (diagonal for the GRU, one 2x2 block per channel for the LSTM), float4
// row loads and stores, and lane shifts of scan values.
#pragma once

#include "common.h"

namespace pnr {

template <int CELL> struct DiagCell;

// ---- GRU with elementwise recurrent weights: state h, gates (r, z, n) ----------------
template <> struct DiagCell<PNR_CELL_GRU_DIAG> {
  static constexpr int G = 3, SP = 1;        // gates, state planes per channel
  static constexpr int AGG_WORDS = 2, PRE_WORDS = 1;
  using E = Aff1;
  struct Par { float ur, uz, un, br, bz, bn; };
  struct Vec { float v0; };                  // one state component
  __device__ static Par load_par(const float* u, const float* bh, int D, int d) {
    Par p;
    p.ur = u[d]; p.uz = u[D + d]; p.un = u[2 * D + d];
    p.br = bh ? bh[d] : 0.f; p.bz = bh ? bh[D + d] : 0.f; p.bn = bh ? bh[2 * D + d] : 0.f;
    return p;
  }
  // residual at (prev p, current h) and, when want_j, the Jacobian there
  __device__ static void eval(const Par& q, const float* g, float p, float h, int jmode,
                              bool want_j, float& res, float& ja) {
    float ghr = fmaf(q.ur, p, q.br), ghz = fmaf(q.uz, p, q.bz), ghn = fmaf(q.un, p, q.bn);
    float r = sigm(g[0] + ghr), z = sigm(g[1] + ghz);
    float n = tanh_(fmaf(r, ghn, g[2]));
    float f = fmaf(z, p - n, n);
    res = f - h;
    if (want_j) {
      if (jmode == PNR_JAC_ZERO) {
        ja = 0.f;
      } else {
        float omz = 1.f - z;
        float cn = omz * (1.f - n * n);
        ja = z + (p - n) * z * omz * q.uz + cn * r * fmaf(ghn * (1.f - r), q.ur, q.un);
      }
    }
  }
  __device__ static float jac_only(const Par& q, const float* g, float p, int jmode) {
    float res, ja;
    eval(q, g, p, 0.f, jmode, true, res, ja);
    return ja;
  }
};

// ---- LSTM with elementwise recurrent weights: state (c, h), gates (i, f, o, g) ------
template <> struct DiagCell<PNR_CELL_LSTM_DIAG> {
  static constexpr int G = 4, SP = 2;
  static constexpr int AGG_WORDS = 6, PRE_WORDS = 2;
  using E = Aff2;
  struct Par { float ui, uf, uo, ug, bi, bf, bo, bg; };
  __device__ static Par load_par(const float* u, const float* bh, int D, int d) {
    Par p;
    p.ui = u[d]; p.uf = u[D + d]; p.uo = u[2 * D + d]; p.ug = u[3 * D + d];
    p.bi = bh ? bh[d] : 0.f; p.bf = bh ? bh[D + d] : 0.f;
    p.bo = bh ? bh[2 * D + d] : 0.f; p.bg = bh ? bh[3 * D + d] : 0.f;
    return p;
  }
  __device__ static void eval(const Par& q, const float* gx, float cp, float hp, float c, float h,
                              int jmode, bool want_j, float& rc, float& rh, Aff2& J) {
    float i = sigm(gx[0] + fmaf(q.ui, hp, q.bi));
    float f = sigm(gx[1] + fmaf(q.uf, hp, q.bf));
    float o = sigm(gx[2] + fmaf(q.uo, hp, q.bo));
    float g = tanh_(gx[3] + fmaf(q.ug, hp, q.bg));
    float cn = fmaf(f, cp, i * g);
    float tau = tanh_(cn);
    rc = cn - c;
    rh = o * tau - h;
    if (want_j) {
      if (jmode == PNR_JAC_ZERO) {
        J = Aff2{0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
      } else {
        // c' = f c + i g:  dc'/dc = f,  dc'/dh = kappa
        float kappa = cp * f * (1.f - f) * q.uf + g * i * (1.f - i) * q.ui + i * (1.f - g * g) * q.ug;
        // h' = o tanh(c'):  dh'/dc = o (1 - tau^2) f,  dh'/dh = tau o (1-o) u_o + o (1 - tau^2) kappa
        float dt = o * (1.f - tau * tau);
        J.a00 = f;
        J.a11 = fmaf(tau * o * (1.f - o), q.uo, dt * kappa);
        if (jmode == PNR_JAC_DIAG) {
          J.a01 = 0.f; J.a10 = 0.f;
        } else {
          J.a01 = kappa; J.a10 = dt * f;
        }
      }
    }
  }
};

// ---------------------------------------------------------------------------------
typedef float f4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ void load_n(const float* __restrict__ row, int tb, int T, bool vec,
                                       int N, float* out) {
  if (vec && tb + N <= T) {
    const f4_t* p = reinterpret_cast<const f4_t*>(row + tb);
    for (int v = 0; v < N / 4; ++v) {
      f4_t x = __builtin_nontemporal_load(p + v);
      out[4 * v] = x[0]; out[4 * v + 1] = x[1]; out[4 * v + 2] = x[2]; out[4 * v + 3] = x[3];
    }
  } else {
    for (int i = 0; i < N; ++i) out[i] = (tb + i < T) ? row[tb + i] : 0.f;
  }
}
__device__ __forceinline__ void store_n(float* __restrict__ row, int tb, int T, bool vec, int N,
                                        const float* in) {
  if (vec && tb + N <= T) {
    f4_t* p = reinterpret_cast<f4_t*>(row + tb);
    for (int v = 0; v < N / 4; ++v) {
      f4_t x = {in[4 * v], in[4 * v + 1], in[4 * v + 2], in[4 * v + 3]};
      __builtin_nontemporal_store(x, p + v);
    }
  } else {
    for (int i = 0; i < N; ++i)
      if (tb + i < T) row[tb + i] = in[i];
  }
}

// The bounded iteration's projection of one new state component: NaN keeps the current
// value, anything else is clipped to [-lim, lim] (infinities included).
__device__ __forceinline__ float project_state(float v, float cur, float lim) {
  return v != v ? cur : fminf(fmaxf(v, -lim), lim);
}

// Apply an affine map to a state increment.
__device__ __forceinline__ float apply(const Aff1& e, float d) { return fmaf(e.a, d, e.b); }
__device__ __forceinline__ float2 apply(const Aff2& e, float2 d) {
  return make_float2(fmaf(e.a00, d.x, fmaf(e.a01, d.y, e.b0)), fmaf(e.a10, d.x, fmaf(e.a11, d.y, e.b1)));
}


template <class E> struct DeltaOf;
template <> struct DeltaOf<Aff1> { using T = float; __device__ static float zero() { return 0.f; } };
template <> struct DeltaOf<Aff2> { using T = float2; __device__ static float2 zero() { return make_float2(0.f, 0.f); } };

template <class E> __device__ __forceinline__ E identity_of();
template <> __device__ __forceinline__ Aff1 identity_of<Aff1>() { return aff_identity1(); }
template <> __device__ __forceinline__ Aff2 identity_of<Aff2>() { return aff_identity2(); }

__device__ __forceinline__ float wave_shr1(float v, float lane0) { return dpp_f<0x138>(lane0, v); }
__device__ __forceinline__ float2 wave_shr1(float2 v, float2 lane0) {
  return make_float2(dpp_f<0x138>(lane0.x, v.x), dpp_f<0x138>(lane0.y, v.y));
}

__device__ __forceinline__ float shfl_down_f(float v, int off) { return __shfl_down(v, off, 64); }
__device__ __forceinline__ Aff1 shfl_down_e(const Aff1& v, int off) {
  return Aff1{shfl_down_f(v.a, off), shfl_down_f(v.b, off)};
}
__device__ __forceinline__ Aff2 shfl_down_e(const Aff2& v, int off) {
  return Aff2{shfl_down_f(v.a00, off), shfl_down_f(v.a01, off), shfl_down_f(v.a10, off),
              shfl_down_f(v.a11, off), shfl_down_f(v.b0, off), shfl_down_f(v.b1, off)};
}
__device__ __forceinline__ float readlane_d(float v, int l) { return readlane_f(v, l); }
__device__ __forceinline__ float2 readlane_d(float2 v, int l) {
  return make_float2(readlane_f(v.x, l), readlane_f(v.y, l));
}


}  // namespace pnr
