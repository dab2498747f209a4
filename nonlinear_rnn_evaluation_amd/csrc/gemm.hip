// Input projection, computed once per call: gx = W x + b_x for every step.  Each step
// depends only on its input and the previous state (ParaRNN overview page, "Newton's
// Iteration"), so the input half of every gate pre-activation is one dense product over
// all steps -- a plain GEMM, done before the Newton loop.
//
//   C[z][i][j] = sum_k A[z][i][k] * Bm[z][j][k] + bias[i or j]      (fp32 or fp64 out)
//
// Both operands are K-contiguous.  bf16 inputs run on MFMA (v_mfma_f32_32x32x16_bf16,
// fp32 accumulate), fp32 inputs on fp32 MFMA; fp64 inputs use an LDS-tiled VALU kernel
// (the fp64 projections are tiny).
#include <atomic>
#include <cmath>

#include "common.h"
#include "kernels.h"

namespace pnr {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float floatx16_t;

// ---------------------------------------------------------------------------------
// bf16 MFMA GEMM.  Block tile 128 x 128, K step 32, 256 threads = 4 waves in 2 x 2,
// each wave 64 x 64 = 2 x 2 MFMA tiles of 32 x 32.  LDS double buffered; rows padded
// by 8 bf16 to spread ds_read_b128 over banks.  Registers are held to 128 so that four
// blocks share a CU (their waves hide each other's global-load latency; LDS 4 x 40 KB).
// Block order: groups of GB_GM row tiles sweep the column tiles together, so each
// column-operand tile is fetched by GB_GM blocks at about the same time (one trip from
// HBM instead of one per row tile) while the group's row tiles stay cached.
constexpr int GB_M = 128, GB_N = 128, GB_K = 32, GB_LD = GB_K + 8, GB_GM = 32;

__global__ void __launch_bounds__(256, 4) gemm_bf16_mfma(GemmArgs g) {
  __shared__ __align__(16) __bf16 As[2][GB_M * GB_LD];
  __shared__ __align__(16) __bf16 Bs[2][GB_N * GB_LD];
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int wm = wid >> 1, wn = wid & 1;
  const int z = blockIdx.z;
  const int gx = (int)gridDim.x, gy = (int)gridDim.y;
  const int lin = (int)blockIdx.y * gx + (int)blockIdx.x;
  const int grp = lin / (GB_GM * gx), loc = lin - grp * GB_GM * gx;
  const int gm = min(GB_GM, gy - grp * GB_GM);   // row tiles in this group
  const int i0 = (grp * GB_GM + loc % gm) * GB_M, j0 = (loc / gm) * GB_N;
  const __bf16* A = reinterpret_cast<const __bf16*>(g.A) + (size_t)z * g.sA;
  const __bf16* Bm = reinterpret_cast<const __bf16*>(g.Bm) + (size_t)z * g.sB;
  float* C = reinterpret_cast<float*>(g.C) + (size_t)z * g.sC;

  // global -> register staging: each thread moves 2 x 16 B of A and of B per K step
  const int lr = tid >> 2;          // 0..63
  const int lk = (tid & 3) * 8;     // 0, 8, 16, 24
  uint4 ra[2], rb[2];
  auto gload = [&](int k0) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int r = lr + 64 * h;
      const int ia = i0 + r, jb = j0 + r, kk = k0 + lk;
      uint4 va = make_uint4(0, 0, 0, 0), vb = make_uint4(0, 0, 0, 0);
      if (ia < g.M && kk < g.K) va = *reinterpret_cast<const uint4*>(A + (size_t)ia * g.lda + kk);
      if (jb < g.N && kk < g.K) vb = *reinterpret_cast<const uint4*>(Bm + (size_t)jb * g.ldb + kk);
      ra[h] = va; rb[h] = vb;
    }
  };
  auto sstore = [&](int buf) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int r = lr + 64 * h;
      *reinterpret_cast<uint4*>(&As[buf][r * GB_LD + lk]) = ra[h];
      *reinterpret_cast<uint4*>(&Bs[buf][r * GB_LD + lk]) = rb[h];
    }
  };

  floatx16_t acc[2][2];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.f;

  const int nk = (g.K + GB_K - 1) / GB_K;
  gload(0);
  sstore(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nk) gload((kt + 1) * GB_K);
#pragma unroll
    for (int ks = 0; ks < GB_K / 16; ++ks) {
      bf16x8_t fa[2], fb[2];
      const int kofs = ks * 16 + (lane >> 5) * 8;
#pragma unroll
      for (int mi = 0; mi < 2; ++mi) {
        const int r = wm * 64 + mi * 32 + (lane & 31);
        fa[mi] = *reinterpret_cast<const bf16x8_t*>(&As[buf][r * GB_LD + kofs]);
      }
#pragma unroll
      for (int ni = 0; ni < 2; ++ni) {
        const int r = wn * 64 + ni * 32 + (lane & 31);
        fb[ni] = *reinterpret_cast<const bf16x8_t*>(&Bs[buf][r * GB_LD + kofs]);
      }
#pragma unroll
      for (int mi = 0; mi < 2; ++mi)
#pragma unroll
        for (int ni = 0; ni < 2; ++ni)
          acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[mi], fb[ni], acc[mi][ni], 0, 0, 0);
    }
    if (kt + 1 < nk) sstore(buf ^ 1);
    __syncthreads();
  }

  // epilogue: lane holds column (lane & 31) and rows 8*q + 4*(lane >> 5) + e
  const float* bias = reinterpret_cast<const float*>(g.bias);
#pragma unroll
  for (int mi = 0; mi < 2; ++mi)
#pragma unroll
    for (int ni = 0; ni < 2; ++ni) {
      const int j = j0 + wn * 64 + ni * 32 + (lane & 31);
      if (j >= g.N) continue;
      const float bj = (bias && !g.bias_on_i) ? bias[j] : 0.f;
#pragma unroll
      for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int i = i0 + wm * 64 + mi * 32 + 8 * q + 4 * (lane >> 5) + e;
          if (i < g.M) {
            const float bi = (bias && g.bias_on_i) ? bias[i] : 0.f;
            __builtin_nontemporal_store(acc[mi][ni][4 * q + e] + bi + bj, &C[(size_t)i * g.ldc + j]);
          }
        }
    }
}

// ---------------------------------------------------------------------------------
// bf16 MFMA GEMM with direct global -> LDS loads (global_load_lds_dwordx4), for K a
// multiple of 32.  The block holds WM x WN waves; each wave computes (32 TM) x (32 TN) of
// C as TM x TN tiles of v_mfma_f32_32x32x16_bf16, so the block tile is (32 TM WM) x
// (32 TN WN).
//  * Long M and N (every projection and gradient product of the long workloads): 256 x 384
//    from 8 waves of 128 x 96, four LDS stages (4 x 40 KB, the whole LDS).  Per K step a
//    wave reads 4 + 3 fragments for 12 MFMAs, and the block pulls 640 operand rows for
//    256 x 384 outputs -- a fifth fewer L2 -> LDS bytes per flop than 256 x 256.
//  * Long M only: 256 x 128 (8 waves of 64 x 64, three stages); otherwise 128 x 128.
//  * Each lane's 16 B go straight from global memory into LDS (lane l of a load writes
//    bytes 16l..16l+15 of a 1 KB run), so no registers stage the tiles and no LDS store
//    instructions are issued.
//  * NS LDS stages: loads run NS-1 K steps ahead of the MFMAs, with one barrier per K
//    step.  Each stage is its own LDS array, so that the compiler can tell the stage being
//    read from the stages being loaded and waits only for the loads it needs (with one
//    array indexed by stage it waits for all).
//  * A tile row is 64 B (32 bf16) with its four 16-B chunks permuted by row bits 2-3.
//    ds_read_b128 serves 16 lanes per cycle from 64 four-byte banks (measured with the
//    bank-conflict counter); a fragment read's 16 lanes take 16 consecutive rows at one
//    chunk, and the permutation puts them on 16 distinct 16-B bank groups.
//  * Rows past M (or N) read the last row instead (their results are not stored), so
//    every load is issued unconditionally and the wait counts stay exact.
//  * The 256 x 384 and 256 x 256 kernels write C through LDS (16-row rounds through the
//    free stage arrays), so that each row of the tile leaves as one contiguous run.
//  * Block order: groups of GM row tiles sweep the column tiles together (as in
//    gemm_bf16_mfma); with 256 x 384 tiles and one block per CU, groups of 64 measured best.
//  * Measured on the 131072-step LSTM's projection (M 16384, N 131072, K 4096): 256 x 384
//    in groups of 64 15.0-15.3 ms with 4-byte stores and 14.2-14.3 ms with C through LDS,
//    against 16.4-16.6 ms for 256 x 256 with 16 waves of 64 x 64 in groups of 32; the
//    gradient products (K 131072, and M 131072) gain 6-11%.
constexpr int GD_K = 32, GD_ROW = GD_K * 2;   // bytes of one tile row

__device__ __forceinline__ int gd_swz(int row) { return (row >> 2) & 3; }

template <int WM, int WN, int TM, int TN>
struct GdCfg {
  static constexpr int BM = 32 * TM * WM, BN = 32 * TN * WN, NW = WM * WN, THREADS = 64 * NW;
  static constexpr int A_RUNS = BM / 16 / NW;   // 1 KB runs per wave and stage
  static constexpr int B_RUNS = BN / 16 / NW;
  static constexpr int LOADS = A_RUNS + B_RUNS;   // vmcnt of one stage
  // the register budget: four waves per SIMD for 64 x 64 wave tiles, two for larger ones
  static constexpr int MIN_BLOCKS = (TM * TN > 4) ? 1 : 4;
  static_assert(A_RUNS * 16 * NW == BM && B_RUNS * 16 * NW == BN, "tile rows must split into whole runs per wave");
};

template <int WM, int WN, int TM, int TN>
struct GdLoad {
  using C = GdCfg<WM, WN, TM, TN>;
  const __bf16* pa[C::A_RUNS];   // this lane's source rows
  const __bf16* pb[C::B_RUNS];
  int ka[C::A_RUNS], kb[C::B_RUNS];   // element offset of its 16-B chunk
};

// vmcnt <= n (expcnt and lgkmcnt left at their maxima), then the barrier.  n must fold
// to a constant (s_waitcnt takes an immediate); every call site passes one.
__device__ __forceinline__ void gd_wait_barrier(int n) {
  switch (n) {
    case 0: __builtin_amdgcn_s_waitcnt(0x0F70); break;
    case 1: __builtin_amdgcn_s_waitcnt(0x0F71); break;
    case 2: __builtin_amdgcn_s_waitcnt(0x0F72); break;
    case 3: __builtin_amdgcn_s_waitcnt(0x0F73); break;
    case 4: __builtin_amdgcn_s_waitcnt(0x0F74); break;
    case 5: __builtin_amdgcn_s_waitcnt(0x0F75); break;
    case 6: __builtin_amdgcn_s_waitcnt(0x0F76); break;
    case 7: __builtin_amdgcn_s_waitcnt(0x0F77); break;
    case 8: __builtin_amdgcn_s_waitcnt(0x0F78); break;
    case 9: __builtin_amdgcn_s_waitcnt(0x0F79); break;
    case 10: __builtin_amdgcn_s_waitcnt(0x0F7A); break;
    case 11: __builtin_amdgcn_s_waitcnt(0x0F7B); break;
    case 12: __builtin_amdgcn_s_waitcnt(0x0F7C); break;
    default: __builtin_amdgcn_s_waitcnt(0x0F70); break;   // waiting for all is always safe
  }
  asm volatile("s_barrier" ::: "memory");
}

// The builtins sit in plain (non-template) functions: the host pass of a kernel template
// rejects a target builtin met while instantiating it, which drops the kernel silently.
__device__ __forceinline__ int gd_uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }
__device__ __forceinline__ void gd_load(const __bf16* src, char* dst) {
  __builtin_amdgcn_global_load_lds(src, dst, 16, 0, 0);
}
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ floatx16_t gd_mfma(u32x4_t a, u32x4_t b, floatx16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b), c,
                                                 0, 0, 0);
}

template <int WM, int WN, int TM, int TN>
__device__ __forceinline__ void gd_issue(const GdLoad<WM, WN, TM, TN>& L, int k0, char* sa, char* sb, int wid) {
  using C = GdCfg<WM, WN, TM, TN>;
#pragma unroll
  for (int h = 0; h < C::A_RUNS; ++h) gd_load(L.pa[h] + k0 + L.ka[h], sa + (C::A_RUNS * wid + h) * 1024);
#pragma unroll
  for (int h = 0; h < C::B_RUNS; ++h) gd_load(L.pb[h] + k0 + L.kb[h], sb + (C::B_RUNS * wid + h) * 1024);
}

template <int TM, int TN>
__device__ __forceinline__ void gd_compute(const char* sa, const char* sb, int wm, int wn, int lane,
                                           floatx16_t (&acc)[TM][TN]) {
#pragma unroll
  for (int ks = 0; ks < GD_K / 16; ++ks) {
    const int kc = ks * 2 + (lane >> 5);
    u32x4_t fa[TM], fb[TN];
#pragma unroll
    for (int mi = 0; mi < TM; ++mi) {
      const int r = wm * 32 * TM + mi * 32 + (lane & 31);
      fa[mi] = *reinterpret_cast<const u32x4_t*>(sa + r * GD_ROW + 16 * (kc ^ gd_swz(r)));
    }
#pragma unroll
    for (int ni = 0; ni < TN; ++ni) {
      const int r = wn * 32 * TN + ni * 32 + (lane & 31);
      fb[ni] = *reinterpret_cast<const u32x4_t*>(sb + r * GD_ROW + 16 * (kc ^ gd_swz(r)));
    }
#pragma unroll
    for (int mi = 0; mi < TM; ++mi)
#pragma unroll
      for (int ni = 0; ni < TN; ++ni) acc[mi][ni] = gd_mfma(fa[mi], fb[ni], acc[mi][ni]);
  }
}

template <int WM, int WN, int TM, int TN, int NS, int GM, bool STAGED>
__global__ void __launch_bounds__((GdCfg<WM, WN, TM, TN>::THREADS), (GdCfg<WM, WN, TM, TN>::MIN_BLOCKS))
    gemm_bf16_dma(GemmArgs g) {
  using Cf = GdCfg<WM, WN, TM, TN>;
  constexpr int SA = Cf::BM * GD_ROW, SB = Cf::BN * GD_ROW;
  static_assert(NS >= 3 && NS <= 4, "three or four stages");
  __shared__ __align__(1024) char sa0[SA], sa1[SA], sa2[SA], sa3[NS > 3 ? SA : 16];
  __shared__ __align__(1024) char sb0[SB], sb1[SB], sb2[SB], sb3[NS > 3 ? SB : 16];
  // stage j is the LDS array named in slot j; every index below is a constant once the
  // loops over stages are unrolled
  char* const stA[4] = {sa0, sa1, sa2, sa3};
  char* const stB[4] = {sb0, sb1, sb2, sb3};
  // the wave index is made uniform so that each load's LDS address (taken from M0) is
  // computed once on the scalar unit, not read back from a vector register per load
  const int tid = threadIdx.x, lane = tid & 63, wid = gd_uniform(tid >> 6);
  const int wm = wid / WN, wn = wid % WN;
  const int z = blockIdx.z;
  const int gx = (int)gridDim.x, gy = (int)gridDim.y;
  const int lin = (int)blockIdx.y * gx + (int)blockIdx.x;
  const int grp = lin / (GM * gx), loc = lin - grp * GM * gx;
  const int gm = min(GM, gy - grp * GM);
  const int i0 = (grp * GM + loc % gm) * Cf::BM, j0 = (loc / gm) * Cf::BN;
  const __bf16* A = reinterpret_cast<const __bf16*>(g.A) + (size_t)z * g.sA;
  const __bf16* Bm = reinterpret_cast<const __bf16*>(g.Bm) + (size_t)z * g.sB;
  float* C = reinterpret_cast<float*>(g.C) + (size_t)z * g.sC;

  // lane l of a 1 KB run holds tile row 16 run + l/4, physical chunk l%4
  GdLoad<WM, WN, TM, TN> L;
#pragma unroll
  for (int h = 0; h < Cf::A_RUNS; ++h) {
    const int row = (Cf::A_RUNS * wid + h) * 16 + (lane >> 2);
    L.ka[h] = 8 * ((lane & 3) ^ gd_swz(row));
    L.pa[h] = A + (size_t)min(i0 + row, g.M - 1) * g.lda;
  }
#pragma unroll
  for (int h = 0; h < Cf::B_RUNS; ++h) {
    const int row = (Cf::B_RUNS * wid + h) * 16 + (lane >> 2);
    L.kb[h] = 8 * ((lane & 3) ^ gd_swz(row));
    L.pb[h] = Bm + (size_t)min(j0 + row, g.N - 1) * g.ldb;
  }

  floatx16_t acc[TM][TN];
#pragma unroll
  for (int a = 0; a < TM; ++a)
#pragma unroll
    for (int b = 0; b < TN; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.f;

  // K step t: wait for its own loads (those of the next NS-2 steps stay in flight),
  // barrier (every wave's loads of step t have landed and every wave is done reading step
  // t-1), load step t+NS-1 into step t-1's stage, multiply step t.  Every step issues its
  // loads, past the last K step too (they reload the last one, unused), so that each wait
  // is the same on every path; the stage rotation is unrolled NS times with no exit
  // inside the loop body, so that the loop head is reached with one order of pending
  // loads, and every stage index is a constant.
  constexpr int W = Cf::LOADS;
  static_assert(W * (NS - 2) <= 12, "wait count beyond the table");
  const int nk = g.K / GD_K, kmax = (nk - 1) * GD_K;
#pragma unroll
  for (int j = 0; j < NS - 1; ++j) gd_issue<WM, WN, TM, TN>(L, min(j * GD_K, kmax), stA[j], stB[j], wid);
  int t = 0;
  for (; t + NS <= nk; t += NS) {
#pragma unroll
    for (int j = 0; j < NS; ++j) {
      gd_wait_barrier(W * (NS - 2));
      gd_issue<WM, WN, TM, TN>(L, min((t + j + NS - 1) * GD_K, kmax), stA[(j + NS - 1) % NS],
                               stB[(j + NS - 1) % NS], wid);
      gd_compute<TM, TN>(stA[j], stB[j], wm, wn, lane, acc);
    }
  }
  // the last nk - t < NS steps: no more loads, so fewer stay in flight at each wait
#pragma unroll
  for (int j = 0; j < NS - 1; ++j) {
    if (t + j < nk) {
      gd_wait_barrier(W * (NS - 2 - j));
      gd_compute<TM, TN>(stA[j], stB[j], wm, wn, lane, acc);
    }
  }
  __builtin_amdgcn_s_waitcnt(0x0F70);   // no load into LDS outlives the block

  const float* bias = reinterpret_cast<const float*>(g.bias);
  if constexpr (STAGED) {
    // Epilogue through LDS, 16 tile rows per round: the waves holding those rows write
    // them into one B stage array (exactly 16 rows of BN floats), then every thread moves
    // 16 B of a row to C, so each row leaves as one contiguous run of 4 BN bytes.  Round r
    // uses stage r % NS: the barriers of the rounds in between order its reads before the
    // writes of round r + NS.
    typedef float f4 __attribute__((ext_vector_type(4)));
    char* const stg[4] = {sb0, sb1, sb2, sb3};
    const bool vec_ok = (g.ldc & 3) == 0 && (reinterpret_cast<uintptr_t>(C) & 15) == 0;
    __syncthreads();   // every wave is done reading the stages
#pragma unroll
    for (int r = 0; r < Cf::BM / 16; ++r) {
      float* Ls = reinterpret_cast<float*>(stg[r % NS]);
      // tile rows 16 r .. 16 r + 15: wave row r / (2 TM), MFMA tile (r % (2 TM)) / 2, and
      // lane groups q = 2 (r & 1) and 2 (r & 1) + 1 of it
      if (wm == r / (2 * TM)) {
        const int mi = (r % (2 * TM)) / 2;
#pragma unroll
        for (int ni = 0; ni < TN; ++ni)
#pragma unroll
          for (int qq = 0; qq < 2; ++qq)
#pragma unroll
            for (int e = 0; e < 4; ++e)
              Ls[(8 * qq + 4 * (lane >> 5) + e) * Cf::BN + wn * 32 * TN + ni * 32 + (lane & 31)] =
                  acc[mi][ni][4 * (2 * (r & 1) + qq) + e];
      }
      __syncthreads();
      constexpr int NV = 16 * Cf::BN / 4;
#pragma unroll
      for (int v = tid; v < NV; v += Cf::THREADS) {
        const int rr = v / (Cf::BN / 4), c4 = v - rr * (Cf::BN / 4);
        const int i = i0 + 16 * r + rr, j = j0 + 4 * c4;
        if (i >= g.M) continue;
        f4 x = *reinterpret_cast<const f4*>(&Ls[rr * Cf::BN + 4 * c4]);
        const float bi = (bias && g.bias_on_i) ? bias[i] : 0.f;
#pragma unroll
        for (int e = 0; e < 4; ++e) x[e] += bi + ((bias && !g.bias_on_i && j + e < g.N) ? bias[j + e] : 0.f);
        if (j + 3 < g.N && vec_ok) {
          __builtin_nontemporal_store(x, reinterpret_cast<f4*>(&C[(size_t)i * g.ldc + j]));
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (j + e < g.N) C[(size_t)i * g.ldc + j + e] = x[e];
        }
      }
    }
    return;
  }
  // epilogue: lane holds column (lane & 31) and rows 8 q + 4 (lane >> 5) + e of each tile,
  // so one store instruction writes two 128-B row segments
#pragma unroll
  for (int mi = 0; mi < TM; ++mi)
#pragma unroll
    for (int ni = 0; ni < TN; ++ni) {
      const int j = j0 + wn * 32 * TN + ni * 32 + (lane & 31);
      if (j >= g.N) continue;
      const float bj = (bias && !g.bias_on_i) ? bias[j] : 0.f;
#pragma unroll
      for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int i = i0 + wm * 32 * TM + mi * 32 + 8 * q + 4 * (lane >> 5) + e;
          if (i < g.M) {
            const float bi = (bias && g.bias_on_i) ? bias[i] : 0.f;
            __builtin_nontemporal_store(acc[mi][ni][4 * q + e] + bi + bj, &C[(size_t)i * g.ldc + j]);
          }
        }
    }
}

// ---------------------------------------------------------------------------------
// fp32 MFMA GEMM (v_mfma_f32_16x16x4f32, fp32 products and sums).  Block tile 64 x 64, K
// step 32, 4 waves in 2 x 2, each 32 x 32 = 2 x 2 MFMA tiles.  In MFMA step kk the lane
// group q = lane / 16 contributes k = 8q + kk for both operands, so a lane's operands of
// one K step are 8 consecutive floats of one LDS row (two 16-byte reads).
constexpr int GF_M = 64, GF_N = 64, GF_K = 32, GF_LD = GF_K + 4;
typedef float f32x4_t __attribute__((ext_vector_type(4)));

__global__ void __launch_bounds__(256) gemm_f32_mfma(GemmArgs g) {
  __shared__ __align__(16) float As[GF_M * GF_LD];
  __shared__ __align__(16) float Bs[GF_N * GF_LD];
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int wm = wid >> 1, wn = wid & 1, q = lane >> 4, r16 = lane & 15;
  const int z = blockIdx.z;
  const int i0 = blockIdx.y * GF_M, j0 = blockIdx.x * GF_N;
  const float* A = reinterpret_cast<const float*>(g.A) + (size_t)z * g.sA;
  const float* Bm = reinterpret_cast<const float*>(g.Bm) + (size_t)z * g.sB;
  float* C = reinterpret_cast<float*>(g.C) + (size_t)z * g.sC;
  const bool vec = (g.lda % 4) == 0 && (g.ldb % 4) == 0 && (g.sA % 4) == 0 && (g.sB % 4) == 0 &&
                   ((uintptr_t)g.A % 16) == 0 && ((uintptr_t)g.Bm % 16) == 0;

  // one operand row segment of 4 k values, zero outside the matrix
  auto load4 = [&](const float* P, int ld, int rows, int r, int k) -> f32x4_t {
    f32x4_t v = {0.f, 0.f, 0.f, 0.f};
    if (r >= rows) return v;
    const float* p = P + (size_t)r * ld + k;
    if (vec && k + 3 < g.K) return *reinterpret_cast<const f32x4_t*>(p);
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = (k + e < g.K) ? p[e] : 0.f;
    return v;
  };

  f32x4_t acc[2][2];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b) acc[a][b] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  for (int k0 = 0; k0 < g.K; k0 += GF_K) {
    f32x4_t va[2], vb[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int e = tid + 256 * h, r = e >> 3, kq = (e & 7) * 4;
      va[h] = load4(A, g.lda, g.M, i0 + r, k0 + kq);
      vb[h] = load4(Bm, g.ldb, g.N, j0 + r, k0 + kq);
    }
    __syncthreads();   // the previous step's reads are done
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int e = tid + 256 * h, r = e >> 3, kq = (e & 7) * 4;
      *reinterpret_cast<f32x4_t*>(&As[r * GF_LD + kq]) = va[h];
      *reinterpret_cast<f32x4_t*>(&Bs[r * GF_LD + kq]) = vb[h];
    }
    __syncthreads();
    f32x4_t fa[2][2], fb[2][2];
#pragma unroll
    for (int mi = 0; mi < 2; ++mi) {
      const float* pa = &As[(wm * 32 + mi * 16 + r16) * GF_LD + 8 * q];
      fa[mi][0] = *reinterpret_cast<const f32x4_t*>(pa);
      fa[mi][1] = *reinterpret_cast<const f32x4_t*>(pa + 4);
    }
#pragma unroll
    for (int ni = 0; ni < 2; ++ni) {
      const float* pb = &Bs[(wn * 32 + ni * 16 + r16) * GF_LD + 8 * q];
      fb[ni][0] = *reinterpret_cast<const f32x4_t*>(pb);
      fb[ni][1] = *reinterpret_cast<const f32x4_t*>(pb + 4);
    }
#pragma unroll
    for (int kk = 0; kk < 8; ++kk)
#pragma unroll
      for (int mi = 0; mi < 2; ++mi)
#pragma unroll
        for (int ni = 0; ni < 2; ++ni)
          acc[mi][ni] = __builtin_amdgcn_mfma_f32_16x16x4f32(fa[mi][kk >> 2][kk & 3], fb[ni][kk >> 2][kk & 3],
                                                             acc[mi][ni], 0, 0, 0);
  }

  // epilogue: lane holds rows 4q + e, column r16 of each 16 x 16 tile
  const float* bias = reinterpret_cast<const float*>(g.bias);
#pragma unroll
  for (int mi = 0; mi < 2; ++mi)
#pragma unroll
    for (int ni = 0; ni < 2; ++ni) {
      const int j = j0 + wn * 32 + ni * 16 + r16;
      if (j >= g.N) continue;
      const float bj = (bias && !g.bias_on_i) ? bias[j] : 0.f;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int i = i0 + wm * 32 + mi * 16 + 4 * q + e;
        if (i < g.M) C[(size_t)i * g.ldc + j] = acc[mi][ni][e] + bj + ((bias && g.bias_on_i) ? bias[i] : 0.f);
      }
    }
}

// ---------------------------------------------------------------------------------
// Generic LDS-tiled GEMM: 64 x 64 block tile, K step 16, 256 threads with 4 x 4 outputs.
template <typename Tin> __device__ __forceinline__ float to_acc(Tin v, float) { return (float)v; }
template <typename Tin> __device__ __forceinline__ double to_acc(Tin v, double) { return (double)v; }
__device__ __forceinline__ float to_acc(__bf16 v, float) { return (float)v; }

template <typename Tin, typename Tout>
__global__ void __launch_bounds__(256) gemm_generic(GemmArgs g) {
  __shared__ Tout As[16][64 + 1];
  __shared__ Tout Bs[16][64 + 1];
  const int tid = threadIdx.x;
  const int tx = tid & 15, ty = tid >> 4;
  const int z = blockIdx.z;
  const int i0 = blockIdx.y * 64, j0 = blockIdx.x * 64;
  const Tin* A = reinterpret_cast<const Tin*>(g.A) + (size_t)z * g.sA;
  const Tin* Bm = reinterpret_cast<const Tin*>(g.Bm) + (size_t)z * g.sB;
  Tout* C = reinterpret_cast<Tout*>(g.C) + (size_t)z * g.sC;
  Tout acc[4][4];
  for (int a = 0; a < 4; ++a)
    for (int b = 0; b < 4; ++b) acc[a][b] = Tout(0);
  for (int k0 = 0; k0 < g.K; k0 += 16) {
    for (int e = tid; e < 64 * 16; e += 256) {
      const int r = e >> 4, kk = e & 15;
      const int ia = i0 + r, jb = j0 + r, k = k0 + kk;
      As[kk][r] = (ia < g.M && k < g.K) ? to_acc(A[(size_t)ia * g.lda + k], Tout(0)) : Tout(0);
      Bs[kk][r] = (jb < g.N && k < g.K) ? to_acc(Bm[(size_t)jb * g.ldb + k], Tout(0)) : Tout(0);
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < 16; ++kk) {
      Tout av[4], bv[4];
      for (int a = 0; a < 4; ++a) av[a] = As[kk][ty * 4 + a];
      for (int b = 0; b < 4; ++b) bv[b] = Bs[kk][tx + 16 * b];
      for (int a = 0; a < 4; ++a)
        for (int b = 0; b < 4; ++b) acc[a][b] += av[a] * bv[b];
    }
    __syncthreads();
  }
  const Tout* bias = reinterpret_cast<const Tout*>(g.bias);
  for (int a = 0; a < 4; ++a) {
    const int i = i0 + ty * 4 + a;
    if (i >= g.M) continue;
    for (int b = 0; b < 4; ++b) {
      const int j = j0 + tx + 16 * b;
      if (j >= g.N) continue;
      Tout v = acc[a][b];
      if (bias) v += g.bias_on_i ? bias[i] : bias[j];
      C[(size_t)i * g.ldc + j] = v;
    }
  }
}

// Compute units of the current device (cached per device; 0 if the query fails).
static int num_cu() {
  constexpr int kMaxDev = 64;
  static std::atomic<int> cache[kMaxDev];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 0;
  if (dev < kMaxDev) {
    const int c = cache[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) n = 0;
  if (dev < kMaxDev && n > 0) cache[dev].store(n, std::memory_order_relaxed);
  return n;
}

// 256 x 384 or 256 x 256 tiles for a long product.  Both run one block per CU, so the
// time goes as (waves of blocks) x (tile area) / (rate per area); the wider tile's rate
// per area is higher by the factor measured on the long workloads' products: about 1.1
// at K = 4096 and 1.2 at K >= 16384, where its fixed costs per tile are spread over more
// K steps.  The wave count decides the rest: a product whose last wave of wide tiles is
// mostly empty (the 8192-step chunks' projections: 1408 blocks, 5.5 waves) keeps the
// 256 x 256 tiles.
static bool wide_tiles_pay(const GemmArgs& g, int ncu) {
  if (ncu <= 0) return true;
  const double b3 = (double)((g.M + 255) / 256) * ((g.N + 383) / 384) * g.batch;
  const double b2 = (double)((g.M + 255) / 256) * ((g.N + 255) / 256) * g.batch;
  const double eff = g.K >= 16384 ? 1.2 : 1.1;
  const double c3 = std::ceil(b3 / ncu) * 1.5 / eff, c2 = std::ceil(b2 / ncu);
  return c3 < c2;
}

hipError_t launch_gemm(int in_dtype, int out_dtype, const GemmArgs& g, hipStream_t st) {
  if (g.M <= 0 || g.N <= 0 || g.batch <= 0) return hipSuccess;
  if (in_dtype == PNR_BF16 && out_dtype == PNR_F32 && (g.K % 8) == 0 && (g.lda % 8) == 0 &&
      (g.ldb % 8) == 0 && (g.sA % 8) == 0 && (g.sB % 8) == 0) {
    const bool aligned = ((uintptr_t)g.A % 16) == 0 && ((uintptr_t)g.Bm % 16) == 0;
    if ((g.K % GD_K) == 0 && aligned) {
      if (g.M >= 1024 && g.N >= 1024) {   // 256 x 384 or 256 x 256 once both sides fill several
        using C3 = GdCfg<2, 4, 4, 3>;
        using C2 = GdCfg<4, 4, 2, 2>;
        if (wide_tiles_pay(g, num_cu())) {
          dim3 grid((g.N + C3::BN - 1) / C3::BN, (g.M + C3::BM - 1) / C3::BM, g.batch);
          hipLaunchKernelGGL((gemm_bf16_dma<2, 4, 4, 3, 4, 64, true>), grid, dim3(C3::THREADS), 0, st, g);
        } else {
          dim3 grid((g.N + C2::BN - 1) / C2::BN, (g.M + C2::BM - 1) / C2::BM, g.batch);
          hipLaunchKernelGGL((gemm_bf16_dma<4, 4, 2, 2, 4, GB_GM, true>), grid, dim3(C2::THREADS), 0, st, g);
        }
      } else if (g.M >= 1024) {
        using Cf = GdCfg<4, 2, 2, 2>;
        dim3 grid((g.N + Cf::BN - 1) / Cf::BN, (g.M + Cf::BM - 1) / Cf::BM, g.batch);
        hipLaunchKernelGGL((gemm_bf16_dma<4, 2, 2, 2, 3, GB_GM, false>), grid, dim3(Cf::THREADS), 0, st, g);
      } else {
        using Cf = GdCfg<2, 2, 2, 2>;
        dim3 grid((g.N + Cf::BN - 1) / Cf::BN, (g.M + Cf::BM - 1) / Cf::BM, g.batch);
        hipLaunchKernelGGL((gemm_bf16_dma<2, 2, 2, 2, 3, GB_GM, false>), grid, dim3(Cf::THREADS), 0, st, g);
      }
      return hipGetLastError();
    }
    dim3 grid((g.N + GB_N - 1) / GB_N, (g.M + GB_M - 1) / GB_M, g.batch);
    hipLaunchKernelGGL(gemm_bf16_mfma, grid, dim3(256), 0, st, g);
    return hipGetLastError();
  }
  dim3 grid((g.N + 63) / 64, (g.M + 63) / 64, g.batch);
  if (in_dtype == PNR_BF16 && out_dtype == PNR_F32)
    hipLaunchKernelGGL((gemm_generic<__bf16, float>), grid, dim3(256), 0, st, g);
  else if (in_dtype == PNR_F32 && out_dtype == PNR_F32)
    hipLaunchKernelGGL(gemm_f32_mfma, grid, dim3(256), 0, st, g);
  else if (in_dtype == PNR_F64 && out_dtype == PNR_F64)
    hipLaunchKernelGGL((gemm_generic<double, double>), grid, dim3(256), 0, st, g);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace pnr
