// Shared device/host definitions for libpnr (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/pnr.h"

#define PNR_BLOCK 256          // threads per block for every iteration kernel (4 waves)
#define PNR_WAVES (PNR_BLOCK / 64)
#define PNR_MAX_ITERS 4096     // residual history capacity

namespace pnr {

// ---------------------------------------------------------------------------------
// Control block written only on the device during a call; read back once at the end.
constexpr int kBarGroups = 32;   // first-level arrival counters of the grid barrier

struct Ctrl {
  int32_t done;        // 1 once the loop has decided (converged, non-finite, or exhausted)
  int32_t status;      // pnr_status
  int32_t iters;       // Newton updates applied to the returned iterate
  int32_t result_buf;  // index of the state buffer holding the result (-1 = the zero guess)
  double rho;          // residual of the returned iterate
  uint32_t ticket;     // dynamic tile counter (standalone scan)
  int32_t fault;       // a bounded device wait ran out (1 = look-back, 2 = barrier)
  int32_t refresh;     // adaptive Jacobian refresh: 1 if the next pass takes a new Jacobian
  int32_t jac_pass;    // adaptive Jacobian refresh: the last pass that took one
  uint32_t pad0[22];
  // Grid barrier.  Every counter sits on a 256-byte line of its own: blocks arrive on
  // one of kBarGroups group counters, the last of each group on the top counter, and
  // all blocks poll the generation word.
  uint32_t bar_top;
  uint32_t pad1[63];
  uint32_t bar_gen;
  uint32_t pad2[63];
  struct { uint32_t count; uint32_t pad[63]; } bar_group[kBarGroups];
  // Barrier-free loops: the decision on iteration k, tagged (k + 1) << 32 | flags
  // (bit 0: stop).  Written by the merging block, polled by the others.
  uint64_t dec;
  uint32_t pad3[62];
};

// Bound on every device-side wait (polls of a look-back slot or of the grid barrier).
// With the back-off below a full count is a few seconds: far above any
// legitimate wait, and it guarantees that every wave reaches the end of the kernel.
constexpr uint32_t kSpinLimit = 1u << 22;

// Sleep between polls of a shared word, growing from ~64 to ~2048 clocks, so that
// thousands of waiting waves do not saturate the memory side with polls.
__device__ __forceinline__ void backoff(uint32_t spins) {
  if (spins < 8) __builtin_amdgcn_s_sleep(1);
  else if (spins < 64) __builtin_amdgcn_s_sleep(8);
  else __builtin_amdgcn_s_sleep(32);
}

__device__ __forceinline__ void record_fault(Ctrl* c, int code) {
  __hip_atomic_store(&c->fault, code, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// One 16-byte global -> LDS load per lane (global_load_lds_dwordx4): lane l writes bytes
// 16l..16l+15 after the wave-uniform LDS address `dst`.  Counted by vmcnt.
__device__ __forceinline__ void lds_load16(const float* src, float* dst) {
  __builtin_amdgcn_global_load_lds(src, dst, 16, 0, 0);
}

__device__ __forceinline__ bool has_fault(const Ctrl* c) {
  return __hip_atomic_load(&c->fault, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0;
}

// Wait until every memory operation this thread issued has completed.  Atomic (agent
// scope) operations complete at the device's coherence point, so an atomic issued after
// this wait is ordered after them for every observer -- without the L2 write-back and
// invalidate that an agent-scope fence costs on a multi-XCD device.
__device__ __forceinline__ void drain_memory_ops() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// Grid-wide barrier for a persistent, co-resident grid whose blocks exchange data only
// through agent-scope atomics (look-back slots, residual partials, the control block)
// and whose other global data is private to a block across the barrier.  Arrival is
// two-level (a group counter, then the top counter for the last of each group); the
// last block to arrive runs `merge` -- the "final block" of the residual reduction --
// then resets the counters and bumps the generation that the others poll.  The wait is
// bounded (kSpinLimit) and records a fault instead of hanging.
template <class Merge>
__device__ __forceinline__ void grid_barrier(Ctrl* c, Merge merge) {
  __shared__ int s_last;
  __shared__ uint32_t s_gen;
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t gen = __hip_atomic_load(&c->bar_gen, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    drain_memory_ops();
    const uint32_t g = blockIdx.x % kBarGroups;
    const uint32_t members = (gridDim.x - g + kBarGroups - 1) / kBarGroups;
    int last = 0;
    const uint32_t prev = atomicAdd(&c->bar_group[g].count, 1u);
    if (prev == members - 1) {
      __hip_atomic_store(&c->bar_group[g].count, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      drain_memory_ops();
      const uint32_t groups = gridDim.x < (unsigned)kBarGroups ? gridDim.x : (unsigned)kBarGroups;
      const uint32_t top = atomicAdd(&c->bar_top, 1u);
      last = top == groups - 1;
    }
    s_last = last;
    s_gen = gen;
  }
  __syncthreads();
  if (s_last) {
    merge();
    __syncthreads();
    if (threadIdx.x == 0) {
      __hip_atomic_store(&c->bar_top, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      drain_memory_ops();
      __hip_atomic_store(&c->bar_gen, s_gen + 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  } else if (threadIdx.x == 0) {
    uint32_t spins = 0;
    while (__hip_atomic_load(&c->bar_gen, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == s_gen) {
      backoff(spins);
      if (++spins > kSpinLimit) {
        record_fault(c, 2);
        break;
      }
    }
  }
  __syncthreads();
}

// Lean grid-wide barrier for loops that take their decisions without a merging block.
// Two-level arrival on agent-scope counters as in grid_barrier, but the counters only
// ever grow: barrier n (counted from 0 in this launch; the control block is zero at
// launch and every block passes the same barriers in order) is complete at a group
// counter of members * (n + 1) and a top counter of groups * (n + 1), so nothing is reset
// and no store needs draining on the way.  `gen` is the caller's count of barriers passed.
// Each arrival is issued after the block's own stores have completed, and the value an
// atomic returns shows every earlier arrival performed, so the block that completes the
// top counter knows every block's data is visible before it publishes generation n + 1.
// Returns false when this block's wait ran out (the fault is recorded); such a block
// leaves the loop and the others give up at the next barrier, so every wave ends.
__device__ __forceinline__ bool grid_sync(Ctrl* c, uint32_t& gen) {
  __shared__ int s_ok;
  __syncthreads();
  if (threadIdx.x == 0) {
    drain_memory_ops();
    const uint32_t g = blockIdx.x % kBarGroups;
    const uint32_t members = (gridDim.x - g + kBarGroups - 1) / kBarGroups;
    const uint32_t groups = gridDim.x < (unsigned)kBarGroups ? gridDim.x : (unsigned)kBarGroups;
    bool released = false;
    if (atomicAdd(&c->bar_group[g].count, 1u) == members * (gen + 1u) - 1u) {
      if (atomicAdd(&c->bar_top, 1u) == groups * (gen + 1u) - 1u) {
        __hip_atomic_store(&c->bar_gen, gen + 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        released = true;
      }
    }
    int ok = 1;
    if (!released) {
      uint32_t spins = 0;
      while (__hip_atomic_load(&c->bar_gen, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == gen) {
        backoff(spins);
        if (++spins > kSpinLimit) {
          record_fault(c, 2);
          ok = 0;
          break;
        }
      }
    }
    s_ok = ok;
  }
  ++gen;
  __syncthreads();
  return s_ok != 0;
}

// Coherent (agent-scope) scalar load of data another block may have written during this
// kernel, e.g. the last state of the preceding tile.
__device__ __forceinline__ float coherent_load(const float* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ double coherent_load(const double* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void coherent_store(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void coherent_store(double* p, double v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ---------------------------------------------------------------------------------
// Elementwise math.  sigmoid(a) = 1 / (1 + e^-a); tanh(a) = 2 sigmoid(2a) - 1.  fp32
// uses the hardware exp2/rcp (a few ulp; far below the fp32 conditioning floor of the
// recurrences), fp64 uses the device math library.
__device__ __forceinline__ float fast_exp(float a) { return __expf(a); }
// v_rcp_f32 (1 ulp); rcp(+inf) = 0 gives the saturated ends of both functions
__device__ __forceinline__ float fast_rcp(float a) { return __builtin_amdgcn_rcpf(a); }
__device__ __forceinline__ float sigm(float a) { return fast_rcp(1.0f + fast_exp(-a)); }
__device__ __forceinline__ float tanh_(float a) {
  return 1.0f - 2.0f * fast_rcp(1.0f + fast_exp(2.0f * a));
}
__device__ __forceinline__ double sigm(double a) { return 1.0 / (1.0 + exp(-a)); }
__device__ __forceinline__ double tanh_(double a) { return tanh(a); }

// |r| as ordered unsigned bits: for non-negative floats the bit patterns order like the
// values, and every NaN pattern sorts above +inf, so an integer max keeps NaN.
__device__ __forceinline__ uint32_t abs_bits(float r) { return __float_as_uint(r) & 0x7fffffffu; }
__device__ __forceinline__ uint64_t abs_bits(double r) {
  return (uint64_t)__double_as_longlong(r) & 0x7fffffffffffffffull;
}
__host__ __device__ inline double bits_to_rho(uint32_t b) {
  if (b >= 0x7f800000u) return __builtin_inf();
  union { uint32_t u; float f; } c; c.u = b; return (double)c.f;
}
__host__ __device__ inline double bits_to_rho64(uint64_t b) {
  if (b >= 0x7ff0000000000000ull) return __builtin_inf();
  union { uint64_t u; double f; } c; c.u = b; return c.f;
}

// ---------------------------------------------------------------------------------
// Cross-lane helpers (wave64).  DPP row_shr:n moves a value n lanes up inside each row
// of 16 lanes; lanes with no source keep `old`.
template <int CTRL>
__device__ __forceinline__ float dpp_f(float old, float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(old), __float_as_int(v), CTRL,
                                                    0xF, 0xF, false));
}
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u(uint32_t old, uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp((int)old, (int)v, CTRL, 0xF, 0xF, false);
}
__device__ __forceinline__ float readlane_f(float v, int lane) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), lane));
}
__device__ __forceinline__ uint32_t lane_id() { return __lane_id(); }

// max over the 64 lanes (all lanes get the result)
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = max(v, dpp_u<0x111>(0u, v));   // row_shr:1
  v = max(v, dpp_u<0x112>(0u, v));   // row_shr:2
  v = max(v, dpp_u<0x114>(0u, v));   // row_shr:4
  v = max(v, dpp_u<0x118>(0u, v));   // row_shr:8
  uint32_t r0 = (uint32_t)__builtin_amdgcn_readlane((int)v, 15);
  uint32_t r1 = (uint32_t)__builtin_amdgcn_readlane((int)v, 31);
  uint32_t r2 = (uint32_t)__builtin_amdgcn_readlane((int)v, 47);
  uint32_t r3 = (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
  return max(max(r0, r1), max(r2, r3));
}

// ---------------------------------------------------------------------------------
// Affine maps d -> A d + b.  compose(later, earlier) = later o earlier.
struct Aff1 {  // one channel (diagonal Jacobian)
  float a, b;
};
__device__ __forceinline__ Aff1 compose(const Aff1& l, const Aff1& e) {
  return Aff1{l.a * e.a, fmaf(l.a, e.b, l.b)};
}
__device__ __forceinline__ Aff1 aff_identity1() { return Aff1{1.0f, 0.0f}; }

struct Aff2 {  // one channel of the (c, h) LSTM state: 2x2 block
  float a00, a01, a10, a11, b0, b1;
};
__device__ __forceinline__ Aff2 compose(const Aff2& l, const Aff2& e) {
  Aff2 r;
  r.a00 = fmaf(l.a00, e.a00, l.a01 * e.a10);
  r.a01 = fmaf(l.a00, e.a01, l.a01 * e.a11);
  r.a10 = fmaf(l.a10, e.a00, l.a11 * e.a10);
  r.a11 = fmaf(l.a10, e.a01, l.a11 * e.a11);
  r.b0 = fmaf(l.a00, e.b0, fmaf(l.a01, e.b1, l.b0));
  r.b1 = fmaf(l.a10, e.b0, fmaf(l.a11, e.b1, l.b1));
  return r;
}
__device__ __forceinline__ Aff2 aff_identity2() { return Aff2{1.f, 0.f, 0.f, 1.f, 0.f, 0.f}; }

// The damped step's Kalman filter in homogeneous coordinates (u, v, n), P = u / v and
// m = n / v: one step is the linear map [[a b 0][c d 0][e f g]] (7 numbers).
// compose(later, earlier) = later o earlier, rescaled by the largest 2x2 entry (a
// positive factor changes neither P nor m).
struct Flt {
  float a, b, c, d, e, f, g;
};
__device__ __forceinline__ Flt compose(const Flt& l, const Flt& x) {
  Flt o;
  o.a = fmaf(l.a, x.a, l.b * x.c);
  o.b = fmaf(l.a, x.b, l.b * x.d);
  o.c = fmaf(l.c, x.a, l.d * x.c);
  o.d = fmaf(l.c, x.b, l.d * x.d);
  o.e = fmaf(l.e, x.a, fmaf(l.f, x.c, l.g * x.e));
  o.f = fmaf(l.e, x.b, fmaf(l.f, x.d, l.g * x.f));
  o.g = l.g * x.g;
  // a positive rescaling changes neither P = u / v nor m = n / v: keep the entries near 1
  const float s = fast_rcp(fmaxf(fmaxf(fabsf(o.a), fabsf(o.b)), fmaxf(fabsf(o.c), fabsf(o.d))));
  o.a *= s; o.b *= s; o.c *= s; o.d *= s; o.e *= s; o.f *= s; o.g *= s;
  return o;
}
__device__ __forceinline__ Flt flt_identity() { return Flt{1.f, 0.f, 0.f, 1.f, 0.f, 0.f, 1.f}; }
struct V3 {
  float u, v, n;
};
__device__ __forceinline__ V3 apply(const Flt& F, const V3& x) {
  return V3{fmaf(F.a, x.u, F.b * x.v), fmaf(F.c, x.u, F.d * x.v), fmaf(F.e, x.u, fmaf(F.f, x.v, F.g * x.n))};
}
__device__ __forceinline__ V3 normalized(const V3& x) {
  const float s = fast_rcp(x.v);
  return V3{x.u * s, 1.f, x.n * s};
}
// Inclusive scan over the 64 lanes of a wave, in lane order (lane 0 earliest):
// after it, lane l holds e_l o e_{l-1} o ... o e_0.  Within each 16-lane row a
// Hillis-Steele pass with DPP row_shr:1,2,4,8; across rows the row totals are
// broadcast with readlane and folded in.
__device__ __forceinline__ Aff1 shfl_row_shr_aff(const Aff1& v, const Aff1& id, int s) {
  Aff1 o;
  switch (s) {
    case 1: o.a = dpp_f<0x111>(id.a, v.a); o.b = dpp_f<0x111>(id.b, v.b); break;
    case 2: o.a = dpp_f<0x112>(id.a, v.a); o.b = dpp_f<0x112>(id.b, v.b); break;
    case 4: o.a = dpp_f<0x114>(id.a, v.a); o.b = dpp_f<0x114>(id.b, v.b); break;
    default: o.a = dpp_f<0x118>(id.a, v.a); o.b = dpp_f<0x118>(id.b, v.b); break;
  }
  return o;
}
__device__ __forceinline__ Aff2 shfl_row_shr_aff(const Aff2& v, const Aff2& id, int s) {
  Aff2 o;
#define PNR_DPP6(C)                                                     \
  o.a00 = dpp_f<C>(id.a00, v.a00); o.a01 = dpp_f<C>(id.a01, v.a01);     \
  o.a10 = dpp_f<C>(id.a10, v.a10); o.a11 = dpp_f<C>(id.a11, v.a11);     \
  o.b0 = dpp_f<C>(id.b0, v.b0); o.b1 = dpp_f<C>(id.b1, v.b1);
  switch (s) {
    case 1: PNR_DPP6(0x111) break;
    case 2: PNR_DPP6(0x112) break;
    case 4: PNR_DPP6(0x114) break;
    default: PNR_DPP6(0x118) break;
  }
#undef PNR_DPP6
  return o;
}
__device__ __forceinline__ Aff1 readlane_aff(const Aff1& v, int l) {
  return Aff1{readlane_f(v.a, l), readlane_f(v.b, l)};
}
__device__ __forceinline__ Aff2 readlane_aff(const Aff2& v, int l) {
  return Aff2{readlane_f(v.a00, l), readlane_f(v.a01, l), readlane_f(v.a10, l),
              readlane_f(v.a11, l), readlane_f(v.b0, l), readlane_f(v.b1, l)};
}

// Lanes with no source lane in their row keep their value (a select, not a composition
// with the identity: with an infinite entry, inf * 0 in that product would make a NaN
// that the plain sequence of compositions never forms).
template <class E>
__device__ __forceinline__ E select_aff(bool take, const E& a, const E& b);
template <>
__device__ __forceinline__ Aff1 select_aff(bool take, const Aff1& a, const Aff1& b) {
  return Aff1{take ? a.a : b.a, take ? a.b : b.b};
}
template <>
__device__ __forceinline__ Aff2 select_aff(bool take, const Aff2& a, const Aff2& b) {
  return Aff2{take ? a.a00 : b.a00, take ? a.a01 : b.a01, take ? a.a10 : b.a10,
              take ? a.a11 : b.a11, take ? a.b0 : b.b0,   take ? a.b1 : b.b1};
}

template <>
__device__ __forceinline__ Flt select_aff(bool take, const Flt& a, const Flt& b) {
  return Flt{take ? a.a : b.a, take ? a.b : b.b, take ? a.c : b.c, take ? a.d : b.d,
             take ? a.e : b.e, take ? a.f : b.f, take ? a.g : b.g};
}

__device__ __forceinline__ Flt shfl_row_shr_aff(const Flt& v, const Flt& id, int s) {
  Flt o;
#define PNR_DPP7(C)                                                                 \
  o.a = dpp_f<C>(id.a, v.a); o.b = dpp_f<C>(id.b, v.b); o.c = dpp_f<C>(id.c, v.c); \
  o.d = dpp_f<C>(id.d, v.d); o.e = dpp_f<C>(id.e, v.e); o.f = dpp_f<C>(id.f, v.f); \
  o.g = dpp_f<C>(id.g, v.g);
  switch (s) {
    case 1: PNR_DPP7(0x111) break;
    case 2: PNR_DPP7(0x112) break;
    case 4: PNR_DPP7(0x114) break;
    default: PNR_DPP7(0x118) break;
  }
#undef PNR_DPP7
  return o;
}
__device__ __forceinline__ Flt readlane_aff(const Flt& v, int l) {
  return Flt{readlane_f(v.a, l), readlane_f(v.b, l), readlane_f(v.c, l), readlane_f(v.d, l),
             readlane_f(v.e, l), readlane_f(v.f, l), readlane_f(v.g, l)};
}
// one lane up across the whole wave (DPP wave_shr:1); lane 0 takes `lane0`
__device__ __forceinline__ Flt flt_wave_shr1(const Flt& v, const Flt& lane0) {
  return Flt{dpp_f<0x138>(lane0.a, v.a), dpp_f<0x138>(lane0.b, v.b), dpp_f<0x138>(lane0.c, v.c),
             dpp_f<0x138>(lane0.d, v.d), dpp_f<0x138>(lane0.e, v.e), dpp_f<0x138>(lane0.f, v.f),
             dpp_f<0x138>(lane0.g, v.g)};
}
__device__ __forceinline__ Aff1 aff_wave_shr1(const Aff1& v, const Aff1& lane0) {
  return Aff1{dpp_f<0x138>(lane0.a, v.a), dpp_f<0x138>(lane0.b, v.b)};
}

template <class E>
__device__ __forceinline__ E wave_inclusive_scan(E v, const E& id) {
  const int rl = (int)(lane_id() & 15);
#pragma unroll
  for (int s = 1; s <= 8; s <<= 1) v = select_aff(rl >= s, compose(v, shfl_row_shr_aff(v, id, s)), v);
  const int row = (int)(lane_id() >> 4);
  E r0 = readlane_aff(v, 15), r1 = readlane_aff(v, 31), r2 = readlane_aff(v, 47);
  E p1 = r0;
  E p2 = compose(r1, r0);
  E p3 = compose(r2, p2);
  E pre = row == 1 ? p1 : (row == 2 ? p2 : p3);
  if (row > 0) v = compose(v, pre);
  return v;
}

// ---------------------------------------------------------------------------------
// Look-back slots.  A slot word carries 32 value bits and the epoch (iteration + 1) that
// wrote it, in one 64-bit word written by a single relaxed agent-scope atomic store, so a
// reader needs no fence: a word is either from this iteration (epoch matches) or not.
__device__ __forceinline__ void slot_put(uint64_t* w, uint32_t epoch, float v) {
  uint64_t x = ((uint64_t)epoch << 32) | (uint64_t)__float_as_uint(v);
  __hip_atomic_store(w, x, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ bool slot_get(const uint64_t* w, uint32_t epoch, float& v) {
  uint64_t x = __hip_atomic_load(w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  v = __uint_as_float((uint32_t)x);
  return (uint32_t)(x >> 32) == epoch;
}

}  // namespace pnr
