// Per-row top-k over fp32 scores (IndexCache paper summary, technical §1:
// the indexer keeps the k most relevant previous tokens).
//
// Scores are mapped to order-preserving 32-bit keys and the k-th largest key
// tau is found by radix selection on 12 + 10 + 10 bits:
//   pass 1  histogram of the top 12 bits over the visible row      (HBM/L2)
//   pass 2  ordered copy of every element whose top 12 bits are >= the
//           threshold bin into an LDS list (keys + positions)       (HBM/L2)
//   pass 3  two more histogram rounds over the list's threshold-bin
//           entries give tau and the number of tau-valued elements to keep
//   pass 4  one ordered scan of the list emits key > tau, plus the first
//           `take_eq` entries equal to tau (lowest positions first).
// Every compaction is an ordered block-wide prefix sum, so the output comes
// out in ascending position order and is deterministic.  When the list would
// overflow LDS (heavily tied rows) passes 3 and 4 re-read the row from
// memory instead.
#include "device_common.hpp"
#include "launchers.hpp"

namespace dsa {
namespace {

constexpr int kTkThreads = 1024;
constexpr int kTkWaves = kTkThreads / kWave;
constexpr int kTkCap = 16384;     // LDS list capacity (entries)
constexpr int kBins1 = 4096;      // top 12 bits
constexpr int kBins2 = 1024;      // next 10, last 10

struct TopkSmem {
  uint32_t hist[kBins1];
  uint32_t list_key[kTkCap];
  int32_t list_pos[kTkCap];
  uint32_t scan[kTkWaves];
  uint32_t sel[4];
};

// Find the bin holding the kk-th largest element (bins scanned from the top):
// writes {bin, count strictly above it} to sel[0..1].  All threads call.
template <int NB>
__device__ void select_bin(const uint32_t* hist, uint32_t kk, TopkSmem& sm) {
  constexpr int PER = NB / kTkThreads;  // bins per thread (4 or 1)
  const int tid = threadIdx.x;
  uint32_t c[PER];
  uint32_t sum = 0;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    c[i] = hist[NB - 1 - (tid * PER + i)];
    sum += c[i];
  }
  uint32_t total;
  uint32_t above = block_excl_scan<kTkWaves>(sum, sm.scan, total);
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    if (above < kk && kk <= above + c[i]) {
      sm.sel[0] = NB - 1 - (tid * PER + i);
      sm.sel[1] = above;
    }
    above += c[i];
  }
  __syncthreads();
}

__device__ __forceinline__ void load4(const float* src, int s, int n, uint32_t (&key)[4],
                                      bool (&ok)[4]) {
  if (s < n) {
    const float4 v = *reinterpret_cast<const float4*>(src + s);
    key[0] = float_key(v.x); key[1] = float_key(v.y);
    key[2] = float_key(v.z); key[3] = float_key(v.w);
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) ok[j] = (s + j) < n;
}

// Ordered emission of the selected elements: key > tau, or key == tau and
// among the first take_eq such elements.  Elements arrive 4 per thread in
// position order through `fetch(base, key, pos, ok)`.
template <typename Fetch>
__device__ void emit_selected(int count, uint32_t tau, uint32_t take_eq, int32_t* out,
                              TopkSmem& sm, Fetch fetch) {
  const int tid = threadIdx.x;
  uint32_t run_gt = 0, run_eq = 0;
  for (int base = 0; base < count; base += 4 * kTkThreads) {
    uint32_t key[4] = {0, 0, 0, 0};
    int32_t pos[4] = {0, 0, 0, 0};
    bool ok[4];
    fetch(base + 4 * tid, key, pos, ok);
    uint32_t ngt = 0, neq = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      ngt += (ok[j] && key[j] > tau);
      neq += (ok[j] && key[j] == tau);
    }
    uint32_t tot;
    const uint32_t ex = block_excl_scan<kTkWaves>((ngt << 16) | neq, sm.scan, tot);
    uint32_t gt_b = run_gt + (ex >> 16), eq_b = run_eq + (ex & 0xFFFFu);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (!ok[j]) continue;
      if (key[j] > tau) {
        out[gt_b + min(eq_b, take_eq)] = pos[j];
        ++gt_b;
      } else if (key[j] == tau) {
        if (eq_b < take_eq) out[gt_b + eq_b] = pos[j];
        ++eq_b;
      }
    }
    run_gt += tot >> 16;
    run_eq += tot & 0xFFFFu;
  }
}

__global__ __launch_bounds__(kTkThreads) void topk_row_kernel(
    const float* __restrict__ scores, int64_t ld, const int32_t* __restrict__ ctx_len, int T,
    int Lmax, int k, int32_t* __restrict__ idx) {
  extern __shared__ __align__(16) unsigned char smem_raw[];
  TopkSmem& sm = *reinterpret_cast<TopkSmem*>(smem_raw);
  const int tid = threadIdx.x;
  const int row = blockIdx.x;
  const int b = row / T;
  const int t = row - b * T;
  const int64_t pos = (int64_t)ctx_len[b] - T + t;
  const int n = (int)max((int64_t)0, min(pos + 1, (int64_t)Lmax));
  int32_t* out = idx + (int64_t)row * k;

  if (n <= k) {  // everything visible is selected
    for (int i = tid; i < k; i += kTkThreads) out[i] = i < n ? i : -1;
    return;
  }
  const float* src = scores + (int64_t)row * ld;

  // ---- pass 1: histogram of the top 12 key bits
  for (int i = tid; i < kBins1; i += kTkThreads) sm.hist[i] = 0;
  __syncthreads();
  for (int s = 4 * tid; s < n; s += 4 * kTkThreads) {
    uint32_t key[4];
    bool ok[4];
    load4(src, s, n, key, ok);
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (ok[j]) atomicAdd(&sm.hist[key[j] >> 20], 1u);
  }
  __syncthreads();
  select_bin<kBins1>(sm.hist, (uint32_t)k, sm);
  const uint32_t b1 = sm.sel[0];
  const uint32_t above1 = sm.sel[1];
  const uint32_t listed = above1 + sm.hist[b1];
  __syncthreads();

  uint32_t b2, above2, b3, above3;
  if (listed <= (uint32_t)kTkCap) {
    // ---- pass 2: ordered copy of elements in bins >= b1 into LDS
    uint32_t run = 0;
    for (int base = 0; base < n; base += 4 * kTkThreads) {
      const int s = base + 4 * tid;
      uint32_t key[4] = {0, 0, 0, 0};
      bool ok[4];
      load4(src, s, n, key, ok);
      uint32_t c = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        ok[j] = ok[j] && (key[j] >> 20) >= b1;
        c += ok[j];
      }
      uint32_t tot;
      uint32_t at = run + block_excl_scan<kTkWaves>(c, sm.scan, tot);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (ok[j]) {
          sm.list_key[at] = key[j];
          sm.list_pos[at] = s + j;
          ++at;
        }
      run += tot;
    }
    const int M = (int)listed;
    // ---- pass 3: refine tau inside the threshold bin
    for (int i = tid; i < kBins2; i += kTkThreads) sm.hist[i] = 0;
    __syncthreads();
    for (int e = tid; e < M; e += kTkThreads) {
      const uint32_t key = sm.list_key[e];
      if ((key >> 20) == b1) atomicAdd(&sm.hist[(key >> 10) & 1023u], 1u);
    }
    __syncthreads();
    select_bin<kBins2>(sm.hist, (uint32_t)k - above1, sm);
    b2 = sm.sel[0];
    above2 = sm.sel[1];
    __syncthreads();
    const uint32_t pre2 = (b1 << 10) | b2;
    for (int i = tid; i < kBins2; i += kTkThreads) sm.hist[i] = 0;
    __syncthreads();
    for (int e = tid; e < M; e += kTkThreads) {
      const uint32_t key = sm.list_key[e];
      if ((key >> 10) == pre2) atomicAdd(&sm.hist[key & 1023u], 1u);
    }
    __syncthreads();
    select_bin<kBins2>(sm.hist, (uint32_t)k - above1 - above2, sm);
    b3 = sm.sel[0];
    above3 = sm.sel[1];
    __syncthreads();
    const uint32_t tau = (b1 << 20) | (b2 << 10) | b3;
    const uint32_t take_eq = (uint32_t)k - above1 - above2 - above3;
    // ---- pass 4: ordered emission from the list
    emit_selected(M, tau, take_eq, out, sm,
                  [&](int e, uint32_t(&key)[4], int32_t(&p)[4], bool(&ok)[4]) {
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                      ok[j] = (e + j) < M;
                      if (ok[j]) {
                        key[j] = sm.list_key[e + j];
                        p[j] = sm.list_pos[e + j];
                      }
                    }
                  });
  } else {
    // ---- overflow: the same refinement, reading the row again each pass
    for (int i = tid; i < kBins2; i += kTkThreads) sm.hist[i] = 0;
    __syncthreads();
    for (int s = 4 * tid; s < n; s += 4 * kTkThreads) {
      uint32_t key[4];
      bool ok[4];
      load4(src, s, n, key, ok);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (ok[j] && (key[j] >> 20) == b1) atomicAdd(&sm.hist[(key[j] >> 10) & 1023u], 1u);
    }
    __syncthreads();
    select_bin<kBins2>(sm.hist, (uint32_t)k - above1, sm);
    b2 = sm.sel[0];
    above2 = sm.sel[1];
    __syncthreads();
    const uint32_t pre2 = (b1 << 10) | b2;
    for (int i = tid; i < kBins2; i += kTkThreads) sm.hist[i] = 0;
    __syncthreads();
    for (int s = 4 * tid; s < n; s += 4 * kTkThreads) {
      uint32_t key[4];
      bool ok[4];
      load4(src, s, n, key, ok);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (ok[j] && (key[j] >> 10) == pre2) atomicAdd(&sm.hist[key[j] & 1023u], 1u);
    }
    __syncthreads();
    select_bin<kBins2>(sm.hist, (uint32_t)k - above1 - above2, sm);
    b3 = sm.sel[0];
    above3 = sm.sel[1];
    __syncthreads();
    const uint32_t tau = (b1 << 20) | (b2 << 10) | b3;
    const uint32_t take_eq = (uint32_t)k - above1 - above2 - above3;
    emit_selected(n, tau, take_eq, out, sm,
                  [&](int s, uint32_t(&key)[4], int32_t(&p)[4], bool(&ok)[4]) {
                    load4(src, s, n, key, ok);
#pragma unroll
                    for (int j = 0; j < 4; ++j) p[j] = s + j;
                  });
  }
}

}  // namespace

size_t topk_workspace_bytes(int, int, int, int) { return 0; }

hipError_t launch_topk(const float* scores, int64_t ld, const int32_t* ctx_len, int B, int T,
                       int Lmax, int k, int32_t* idx, void*, size_t, hipStream_t stream) {
  static bool attr_set = false;
  const size_t smem = sizeof(TopkSmem);
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute((const void*)topk_row_kernel,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  hipLaunchKernelGGL(topk_row_kernel, dim3(B * T), dim3(kTkThreads), smem, stream, scores, ld,
                     ctx_len, T, Lmax, k, idx);
  return hipGetLastError();
}

}  // namespace dsa
