// Proxy reuse costs for the training-free pattern search.
//
// The search (greedy F -> S conversion) needs, for every layer l and every
// earlier layer j, what layer l loses when it attends with j's index set
// instead of its own.  Two proxies for the calibration loss:
//   output: sum (o_l[T_j] - o_l[T_l])^2 / sum o_l[T_l]^2 over the bf16
//           attention outputs of layer l;
//   miss:   1 - sum_rows |T_j ∩ T_l| / sum_rows |T_l| over the index lists.
// Each value is a reduction: a grid of workgroups writes one (a, b) pair of
// fp64 partial sums each, then a single workgroup adds them in a fixed order
// and writes the matrix entry.  The grid depends only on the problem size, so
// the result is deterministic run to run.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "device_common.hpp"
#include "launchers.hpp"

namespace dsa {
namespace {

constexpr int kRedThreads = 256;
constexpr int kRedWaves = kRedThreads / kWave;

__device__ __forceinline__ double wave_sum(double v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, kWave);
  return v;
}

// Sum of (a, b) over the workgroup; the result is valid in thread 0.
__device__ __forceinline__ void block_sum2(double& a, double& b) {
  __shared__ double sa[kRedWaves], sb[kRedWaves];
  a = wave_sum(a);
  b = wave_sum(b);
  const int lane = threadIdx.x & (kWave - 1), wid = threadIdx.x / kWave;
  if (lane == 0) {
    sa[wid] = a;
    sb[wid] = b;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    a = 0.0;
    b = 0.0;
#pragma unroll
    for (int i = 0; i < kRedWaves; ++i) {
      a += sa[i];
      b += sb[i];
    }
  }
}

__device__ __forceinline__ double bf16_lo(uint32_t w) { return (double)__uint_as_float(w << 16); }
__device__ __forceinline__ double bf16_hi(uint32_t w) {
  return (double)__uint_as_float(w & 0xFFFF0000u);
}

// partials[g] = (sum (x - y)^2, sum y^2) over the 8-element chunks
// g*256 + tid, + G*256, ...  Differences and squares are formed in fp64 from
// the exact bf16 values.
__global__ __launch_bounds__(kRedThreads) void sq_err_partials(const uint32_t* __restrict__ x,
                                                               const uint32_t* __restrict__ y,
                                                               int64_t chunks,
                                                               double2* __restrict__ partials) {
  double e = 0.0, z = 0.0;
  const int64_t stride = (int64_t)gridDim.x * kRedThreads;
  for (int64_t c = (int64_t)blockIdx.x * kRedThreads + threadIdx.x; c < chunks; c += stride) {
    const i32x4 xv = ld16(x + 4 * c), yv = ld16(y + 4 * c);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t xw = (uint32_t)xv[i], yw = (uint32_t)yv[i];
      const double y0 = bf16_lo(yw), y1 = bf16_hi(yw);
      const double d0 = bf16_lo(xw) - y0, d1 = bf16_hi(xw) - y1;
      e = fma(d0, d0, e);
      e = fma(d1, d1, e);
      z = fma(y0, y0, z);
      z = fma(y1, y1, z);
    }
  }
  block_sum2(e, z);
  if (threadIdx.x == 0) partials[blockIdx.x] = make_double2(e, z);
}

// partials[g] = (sum |reused ∩ own|, sum |own|) over the work items of
// workgroup g.  A work item is (row, slice): the row's own list is staged in
// LDS and each thread looks one entry of the slice's 256 reused entries up by
// binary search; slice 0 also counts the own list.  Both lists are in the
// top-k output form (strictly ascending positions, then -1 padding) and
// every read stays inside its row.
__global__ __launch_bounds__(kRedThreads) void overlap_partials(const int32_t* __restrict__ reused,
                                                                const int32_t* __restrict__ own,
                                                                int64_t rows, int k,
                                                                double2* __restrict__ partials) {
  extern __shared__ int32_t own_row[];  // k entries
  __shared__ int wave_cnt[kRedWaves];
  const int lane = threadIdx.x & (kWave - 1), wid = threadIdx.x / kWave;
  const int slices = (k + kRedThreads - 1) / kRedThreads;
  const int64_t items = rows * slices;
  double hit_total = 0.0, own_total = 0.0;
  for (int64_t it = blockIdx.x; it < items; it += gridDim.x) {
    const int64_t r = it / slices;
    const int slice = (int)(it % slices);
    const int32_t* b = own + r * k;
    int cnt = 0;
    for (int i = threadIdx.x; i < k; i += kRedThreads) {
      const int32_t v = b[i];
      own_row[i] = v;
      cnt += v >= 0 ? 1 : 0;
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) cnt += __shfl_xor(cnt, off, kWave);
    if (lane == 0) wave_cnt[wid] = cnt;
    __syncthreads();
    int n_own = 0;
#pragma unroll
    for (int i = 0; i < kRedWaves; ++i) n_own += wave_cnt[i];
    const int i = slice * kRedThreads + threadIdx.x;
    int hit = 0;
    if (i < k) {
      const int32_t v = reused[r * k + i];
      if (v >= 0) {
        int lo = 0, hi = n_own;  // search [lo, hi)
        while (lo < hi) {
          const int mid = (lo + hi) >> 1;
          if (own_row[mid] < v)
            lo = mid + 1;
          else
            hi = mid;
        }
        hit = (lo < n_own && own_row[lo] == v) ? 1 : 0;
      }
    }
    hit_total += (double)hit;
    if (threadIdx.x == 0 && slice == 0) own_total += (double)n_own;
    __syncthreads();  // own_row and wave_cnt are rewritten by the next item
  }
  // per-thread totals are integers, so the sum is exact in any order
  block_sum2(hit_total, own_total);
  if (threadIdx.x == 0) partials[blockIdx.x] = make_double2(hit_total, own_total);
}

// dst = proxy value from the G partial pairs, added in index order per
// thread and then over threads in a fixed order.
__global__ __launch_bounds__(kRedThreads) void finish_cost(const double2* __restrict__ partials,
                                                           int G, int miss,
                                                           double* __restrict__ dst) {
  double a = 0.0, b = 0.0;
  for (int i = threadIdx.x; i < G; i += kRedThreads) {
    const double2 p = partials[i];
    a += p.x;
    b += p.y;
  }
  block_sum2(a, b);
  if (threadIdx.x == 0) {
    if (miss)
      *dst = b > 0.0 ? 1.0 - a / b : 0.0;
    else
      *dst = b > 0.0 ? a / b : (a == 0.0 ? 0.0 : (double)INFINITY);
  }
}

__global__ __launch_bounds__(kRedThreads) void fill_zero_f64(double* __restrict__ p, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * kRedThreads + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * kRedThreads)
    p[i] = 0.0;
}

int sq_err_grid(int64_t elems) {
  const int64_t chunks = elems / 8;
  const int64_t g = (chunks + kRedThreads - 1) / kRedThreads;
  return (int)(g < 1 ? 1 : (g > kReuseCostMaxGrid ? kReuseCostMaxGrid : g));
}

int overlap_grid(int64_t rows, int k) {
  const int64_t g = rows * ((k + kRedThreads - 1) / kRedThreads);
  return (int)(g < 1 ? 1 : (g > kReuseCostMaxGrid ? kReuseCostMaxGrid : g));
}

}  // namespace

hipError_t launch_fill_zero_f64(double* p, int64_t n, hipStream_t stream) {
  int64_t g = (n + kRedThreads - 1) / kRedThreads;
  g = g < 1 ? 1 : (g > 1024 ? 1024 : g);
  hipLaunchKernelGGL(fill_zero_f64, dim3((unsigned)g), dim3(kRedThreads), 0, stream, p, n);
  return hipGetLastError();
}

hipError_t launch_output_cost(const void* out, const void* ref, int64_t elems, double2* partials,
                              double* dst, hipStream_t stream) {
  const int G = sq_err_grid(elems);
  hipLaunchKernelGGL(sq_err_partials, dim3(G), dim3(kRedThreads), 0, stream,
                     static_cast<const uint32_t*>(out), static_cast<const uint32_t*>(ref),
                     elems / 8, partials);
  hipLaunchKernelGGL(finish_cost, dim3(1), dim3(kRedThreads), 0, stream, partials, G, 0, dst);
  return hipGetLastError();
}

hipError_t launch_miss_cost(const int32_t* reused, const int32_t* own, int64_t rows, int k,
                            double2* partials, double* dst, hipStream_t stream) {
  const int G = overlap_grid(rows, k);
  hipLaunchKernelGGL(overlap_partials, dim3(G), dim3(kRedThreads), (size_t)k * sizeof(int32_t),
                     stream, reused, own, rows, k, partials);
  hipLaunchKernelGGL(finish_cost, dim3(1), dim3(kRedThreads), 0, stream, partials, G, 1, dst);
  return hipGetLastError();
}

}  // namespace dsa
