// Small kernels around the Newton loop: per-call initialisation of the control block
// and look-back slots, and the conversion of the returned iterate to the caller's
// [B, T, S] layout.
#include <cstdlib>
#include <mutex>

#include "common.h"
#include "kernels.h"

namespace pnr {

int cached_occupancy(const void* fn, size_t lds, int threads) {
  struct Entry { const void* fn; size_t lds; int threads, dev, v; };
  static Entry cache[64];
  static int n = 0;
  static std::mutex mu;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  std::lock_guard<std::mutex> lock(mu);
  for (int i = 0; i < n; ++i)
    if (cache[i].fn == fn && cache[i].lds == lds && cache[i].threads == threads && cache[i].dev == dev)
      return cache[i].v;
  int v = 0;
  if (lds <= 65536 || hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds) == hipSuccess)
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&v, fn, threads, lds) != hipSuccess) v = 0;
  if (n < 64) cache[n++] = Entry{fn, lds, threads, dev, v};
  return v;
}

// Persistent launches.  Every persistent grid here is sized to the device's resident
// capacity (cached_occupancy), and the loop inside needs all of its workgroups resident
// at once (look-back and grid-barrier waits on other workgroups).  By default the grid
// goes out through hipLaunchCooperativeKernel, which guarantees that co-residency even
// next to other work on the device (other streams, other persistent calls).  Every wait
// is also bounded: a wait that runs out records a fault, which the call reports as an
// error, never a hang.  PNR_COOPERATIVE=0 (read once per process) selects the ordinary
// launch, about 15-20 us cheaper per call, for callers that run nothing else on the
// device at the same time.
hipError_t launch_persistent(const void* fn, int grid, size_t lds, void** args, hipStream_t st, int threads) {
  static const bool coop = [] {
    const char* e = getenv("PNR_COOPERATIVE");
    return !(e && e[0] == '0');
  }();
  if (coop) return hipLaunchCooperativeKernel(fn, dim3(grid), dim3(threads), args, (unsigned)lds, st);
  return hipLaunchKernel(fn, dim3(grid), dim3(threads), args, lds, st);
}

__global__ void init_kernel(Ctrl* ctrl, uint64_t* slots, size_t n, uint64_t* partials, size_t np) {
  const size_t i0 = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i0 == 0) {
    ctrl->done = 0;
    ctrl->status = PNR_NOT_CONVERGED;
    ctrl->iters = -1;
    ctrl->result_buf = -1;
    ctrl->rho = 0.0;
    ctrl->ticket = 0;
    ctrl->bar_top = 0;
    ctrl->bar_gen = 0;
    ctrl->fault = 0;
    ctrl->refresh = 0;
    ctrl->jac_pass = 0;
    for (int g = 0; g < kBarGroups; ++g) ctrl->bar_group[g].count = 0;
    ctrl->dec = 0;
  }
  // epoch 0 is never a live epoch, so zeroed words read as "not yet written"
  for (size_t i = i0; i < n; i += (size_t)gridDim.x * blockDim.x) slots[i] = 0;
  for (size_t i = i0; i < np; i += (size_t)gridDim.x * blockDim.x) partials[i] = 0;
}

hipError_t launch_init(Ctrl* ctrl, uint64_t* slots, size_t slot_words, uint64_t* partials, size_t partial_words,
                       hipStream_t st) {
  size_t blocks = ((slot_words > partial_words ? slot_words : partial_words) + 255) / 256;
  if (blocks < 1) blocks = 1;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(init_kernel, dim3((unsigned)blocks), dim3(256), 0, st, ctrl, slots, slot_words, partials,
                     partial_words);
  return hipGetLastError();
}

struct Bufs3f { const float* p[3]; };

// [B][S][T] -> [B][T][S] through a 32 x 32 LDS tile; zeros when the result is the zero guess.
__global__ void __launch_bounds__(256) diag_output_kernel(Bufs3f bufs, const Ctrl* ctrl, float* out, int S,
                                                          int T) {
  __shared__ float tile[32][33];
  const int rb = ctrl->result_buf;
  const float* src = rb >= 0 ? bufs.p[rb] : nullptr;
  const int b = blockIdx.z;
  const int t0 = blockIdx.x * 32, s0 = blockIdx.y * 32;
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;   // 32 x 8
  for (int r = ty; r < 32; r += 8) {
    const int s = s0 + r, t = t0 + tx;
    float v = 0.f;
    if (src && s < S && t < T) v = src[((size_t)b * S + s) * T + t];
    tile[r][tx] = v;
  }
  __syncthreads();
  for (int r = ty; r < 32; r += 8) {
    const int t = t0 + r, s = s0 + tx;
    if (t < T && s < S) out[((size_t)b * T + t) * S + s] = tile[tx][r];
  }
}

// The same conversion 4 elements (16 B) per lane through a 64 x 65 tile, for S and T
// multiples of 4: 256 B runs on both sides, about copy speed.
__global__ void __launch_bounds__(256) diag_output4_kernel(Bufs3f bufs, const Ctrl* ctrl, float* out, int S,
                                                           int T) {
  __shared__ float tile[64][65];
  const int rb = ctrl->result_buf;
  const float* src = rb >= 0 ? bufs.p[rb] : nullptr;
  const size_t b = blockIdx.z;
  const int t0 = blockIdx.x * 64, s0 = blockIdx.y * 64;
  const int g = threadIdx.x & 15, q = threadIdx.x >> 4;   // 16 groups of 4 along a row, 16 rows
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int ss = q + 16 * i, s = s0 + ss, t = t0 + 4 * g;
    float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
    if (src && s < S && t < T) v = *reinterpret_cast<const float4*>(src + (b * S + s) * T + t);
    tile[ss][4 * g] = v.x; tile[ss][4 * g + 1] = v.y; tile[ss][4 * g + 2] = v.z; tile[ss][4 * g + 3] = v.w;
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int tt = q + 16 * i, t = t0 + tt, s = s0 + 4 * g;
    if (t < T && s < S)
      *reinterpret_cast<float4*>(out + (b * T + t) * S + s) =
          make_float4(tile[4 * g][tt], tile[4 * g + 1][tt], tile[4 * g + 2][tt], tile[4 * g + 3][tt]);
  }
}

hipError_t launch_diag_output(const float* const* bufs, const Ctrl* ctrl, float* h_out, int B, int S, int T,
                              hipStream_t st) {
  Bufs3f bb{{bufs[0], bufs[1], bufs[2]}};
  bool vec = S % 4 == 0 && T % 4 == 0 && (uintptr_t)h_out % 16 == 0;
  for (int i = 0; i < 3; ++i) vec = vec && (uintptr_t)bufs[i] % 16 == 0;
  if (vec) {
    dim3 grid4((T + 63) / 64, (S + 63) / 64, B);
    hipLaunchKernelGGL(diag_output4_kernel, grid4, dim3(256), 0, st, bb, ctrl, h_out, S, T);
    return hipGetLastError();
  }
  dim3 grid((T + 31) / 32, (S + 31) / 32, B);
  hipLaunchKernelGGL(diag_output_kernel, grid, dim3(256), 0, st, bb, ctrl, h_out, S, T);
  return hipGetLastError();
}

template <typename Tt> struct Bufs4 { const Tt* p[4]; };

template <typename Tt>
__global__ void dense_output_kernel(Bufs4<Tt> bufs, const Ctrl* ctrl, Tt* out, size_t n) {
  const int rb = ctrl->result_buf;
  const Tt* src = rb >= 0 ? bufs.p[rb] : nullptr;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
    out[i] = src ? src[i] : Tt(0);
}

template <typename Tt>
hipError_t launch_dense_output(const Tt* const* bufs, const Ctrl* ctrl, Tt* h_out, size_t n, hipStream_t st) {
  Bufs4<Tt> bb{{bufs[0], bufs[1], bufs[2], bufs[3]}};
  size_t blocks = (n + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL((dense_output_kernel<Tt>), dim3((unsigned)blocks), dim3(256), 0, st, bb, ctrl, h_out, n);
  return hipGetLastError();
}
template hipError_t launch_dense_output<float>(const float* const*, const Ctrl*, float*, size_t, hipStream_t);
template hipError_t launch_dense_output<double>(const double* const*, const Ctrl*, double*, size_t, hipStream_t);

// [Z][R][C] -> [Z][C][R] (fp32 or bf16 in, fp32 or bf16 out) through a 32 x 33 LDS tile:
// reads run along C and writes along R, both coalesced.
template <typename Tin, typename Tout>
__global__ void __launch_bounds__(256) transpose_kernel(const Tin* __restrict__ in, Tout* __restrict__ out, int R,
                                                        int C) {
  __shared__ float tile[32][33];
  const size_t z = blockIdx.z;
  const int c0 = blockIdx.x * 32, r0 = blockIdx.y * 32;
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;   // 32 x 8
  const Tin* src = in + z * (size_t)R * C;
  Tout* dst = out + z * (size_t)R * C;
  for (int k = ty; k < 32; k += 8) {
    const int r = r0 + k, c = c0 + tx;
    tile[k][tx] = (r < R && c < C) ? (float)src[(size_t)r * C + c] : 0.f;
  }
  __syncthreads();
  for (int k = ty; k < 32; k += 8) {
    const int c = c0 + k, r = r0 + tx;
    if (c < C && r < R) dst[(size_t)c * R + r] = (Tout)tile[tx][k];
  }
}

// The same for R and C multiples of 4 (and 4-element-aligned rows): a 64 x 64 tile, each
// thread moving 4 consecutive elements per access, so that a wave reads and writes whole
// 128-256 B row segments instead of 2-4 B per lane.  A 4-element group is entirely inside
// or entirely outside the matrix, so each group needs one bounds test.
template <typename T, int N> struct alignas(sizeof(T) * N) VecOf { T v[N]; };
template <typename Tin, typename Tout>
__global__ void __launch_bounds__(256) transpose4_kernel(const Tin* __restrict__ in, Tout* __restrict__ out, int R,
                                                         int C) {
  __shared__ float tile[64][65];
  const size_t z = blockIdx.z;
  const int c0 = blockIdx.x * 64, r0 = blockIdx.y * 64;
  const int g = threadIdx.x & 15, q = threadIdx.x >> 4;   // 16 groups of 4 along a row, 16 rows
  const Tin* src = in + z * (size_t)R * C;
  Tout* dst = out + z * (size_t)R * C;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int rr = q + 16 * i, r = r0 + rr, c = c0 + 4 * g;
    VecOf<Tin, 4> v;
    if (r < R && c < C) v = *reinterpret_cast<const VecOf<Tin, 4>*>(src + (size_t)r * C + c);
    else v = VecOf<Tin, 4>{};
#pragma unroll
    for (int j = 0; j < 4; ++j) tile[rr][4 * g + j] = (float)v.v[j];
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int cc = q + 16 * i, c = c0 + cc, r = r0 + 4 * g;
    if (c < C && r < R) {
      VecOf<Tout, 4> v;
#pragma unroll
      for (int j = 0; j < 4; ++j) v.v[j] = (Tout)tile[4 * g + j][cc];
      *reinterpret_cast<VecOf<Tout, 4>*>(dst + (size_t)c * R + r) = v;
    }
  }
}

hipError_t launch_transpose(const void* in, int in_dtype, void* out, int out_dtype, int Z, int R, int C,
                            hipStream_t st) {
  if (Z <= 0 || R <= 0 || C <= 0) return hipSuccess;
  const size_t ein = in_dtype == PNR_BF16 ? 2 : 4, eout = out_dtype == PNR_BF16 ? 2 : 4;
  const bool vec = R % 4 == 0 && C % 4 == 0 && (uintptr_t)in % (4 * ein) == 0 && (uintptr_t)out % (4 * eout) == 0;
  if (vec) {
    dim3 grid4((C + 63) / 64, (R + 63) / 64, Z);
#define PNR_TR4(TI, TO) \
  hipLaunchKernelGGL((transpose4_kernel<TI, TO>), grid4, dim3(256), 0, st, static_cast<const TI*>(in), static_cast<TO*>(out), R, C)
    if (in_dtype == PNR_BF16 && out_dtype == PNR_F32) PNR_TR4(__bf16, float);
    else if (in_dtype == PNR_F32 && out_dtype == PNR_F32) PNR_TR4(float, float);
    else if (in_dtype == PNR_BF16 && out_dtype == PNR_BF16) PNR_TR4(__bf16, __bf16);
    else if (in_dtype == PNR_F32 && out_dtype == PNR_BF16) PNR_TR4(float, __bf16);
    else return hipErrorInvalidValue;
#undef PNR_TR4
    return hipGetLastError();
  }
  dim3 grid((C + 31) / 32, (R + 31) / 32, Z);
#define PNR_TR(TI, TO) \
  hipLaunchKernelGGL((transpose_kernel<TI, TO>), grid, dim3(256), 0, st, static_cast<const TI*>(in), static_cast<TO*>(out), R, C)
  if (in_dtype == PNR_BF16 && out_dtype == PNR_F32) PNR_TR(__bf16, float);
  else if (in_dtype == PNR_F32 && out_dtype == PNR_F32) PNR_TR(float, float);
  else if (in_dtype == PNR_BF16 && out_dtype == PNR_BF16) PNR_TR(__bf16, __bf16);
  else if (in_dtype == PNR_F32 && out_dtype == PNR_BF16) PNR_TR(float, __bf16);
  else return hipErrorInvalidValue;
#undef PNR_TR
  return hipGetLastError();
}

// out_q[j] = sum_b part[b][q][j] for q = 0, 1, 2 (each output may be null); n values each.
__global__ void __launch_bounds__(256) sum_over_batch_kernel(const float* __restrict__ part, int B, int n,
                                                             float* o0, float* o1, float* o2) {
  const int j = blockIdx.x * blockDim.x + threadIdx.x;
  const int q = blockIdx.y;
  float* o = q == 0 ? o0 : (q == 1 ? o1 : o2);
  if (j >= n || !o) return;
  float s = 0.f;
  for (int b = 0; b < B; ++b) s += part[((size_t)b * 3 + q) * n + j];
  o[j] = s;
}

hipError_t launch_sum_over_batch(const float* part, int B, int n, float* o0, float* o1, float* o2,
                                 hipStream_t st) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(sum_over_batch_kernel, dim3((n + 255) / 256, 3), dim3(256), 0, st, part, B, n, o0, o1, o2);
  return hipGetLastError();
}

__global__ void __launch_bounds__(256) fill_zero_kernel(float* __restrict__ p, size_t n) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
    p[i] = 0.f;
}

hipError_t launch_fill_zero(float* p, size_t n, hipStream_t st) {
  if (!p || n == 0) return hipSuccess;
  size_t blocks = (n + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)blocks), dim3(256), 0, st, p, n);
  return hipGetLastError();
}

}  // namespace pnr
