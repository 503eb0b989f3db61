// Per-row top-k over fp32 scores (IndexCache paper summary, technical §1:
// the indexer keeps the k most relevant previous tokens).
//
// Scores are mapped to order-preserving 32-bit keys and the k-th largest key
// tau is found by radix selection on 12 + 10 + 10 bits:
//   1. histogram of the top 12 bits over the visible row -> threshold bin b1
//      and the count of elements in higher bins;
//   2. ordered copy of every element whose top 12 bits are >= b1 (a few
//      thousand for real score rows) into an LDS list (keys + positions);
//   3. two histogram rounds over the list's b1 entries give tau and the number
//      of tau-valued elements to keep;
//   4. one ordered scan of the list emits key > tau, plus the first take_eq
//      entries equal to tau (lowest positions first).
// Every compaction is an ordered block-wide prefix sum, so the output comes
// out in ascending position order and is deterministic.  When the list would
// overflow LDS (heavily tied rows) steps 3 and 4 re-read the row instead.
//
// Two launch shapes:
//   * many rows (prefill): one 1024-thread workgroup per row does 1-4;
//   * few long rows (decode): each row is cut into chunks; one kernel builds
//     the step-1 histogram with chunk workgroups (LDS histogram, then global
//     atomics into a per-row histogram), a second compacts each chunk's
//     candidates in order into its own slice of a candidate buffer, and a
//     per-row workgroup concatenates the slices and finishes 3-4.  The
//     per-row histogram is cleared again by that last kernel, so the
//     workspace holding it must be zero before the first call and is left
//     zero by every call.  The fused decode indexer produces the histogram
//     and the slices itself (against a lower bound of the threshold bin)
//     and runs only the finishing kernel, which then takes the threshold
//     from the finished histogram.
#include "device_common.hpp"
#include "launchers.hpp"

namespace dsa {
namespace {

constexpr int kTkThreads = 1024;
constexpr int kTkWaves = kTkThreads / kWave;
constexpr int kTkCap = 16384;     // LDS list capacity (entries)
constexpr int kBins1 = 4096;      // top 12 bits
constexpr int kBins2 = 1024;      // next 10, last 10
constexpr int kChThreads = 256;   // chunk workgroups
constexpr int kChWaves = kChThreads / kWave;
constexpr int kMaxChunks = kTopkMaxChunks;
constexpr int kPer = 16;         // scores per thread per chunk batch (4096 per workgroup)
constexpr int kGather = 8;       // candidate loads in flight per thread
constexpr int kFinGather = 16;   // ... in the decode finish (first batch of every slice)

struct TopkSmem {
  uint32_t hist[kBins1];
  uint32_t list_key[kTkCap];
  int32_t list_pos[kTkCap];
  uint32_t scan[kTkWaves];
  uint32_t scan2[kTkWaves];
  uint32_t sel[4];
  uint32_t chunk_off[kMaxChunks + 1];
};

// Word 3 of a raw (untyped, unswizzled) buffer resource on gfx9.
constexpr int kBufferWord3 = 0x00020000;

// Score loads go through a buffer resource over the first n scores of a row,
// rounded up to whole 16-byte vectors (rows are padded to a multiple of 4
// floats): a load is never partly in range, loads past the end read zero,
// and no branch separates issuing a batch of loads from using it, so a
// thread's loads are all in flight together.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t row_rsrc(const float* src, int n) {
  return __builtin_amdgcn_make_buffer_rsrc((void*)src, 0, ((n + 3) & ~3) * 4, kBufferWord3);
}

// Scores s..s+3 (s a multiple of 4) as keys; ok marks those below n.
__device__ __forceinline__ void load4(__amdgpu_buffer_rsrc_t r, int s, int n, uint32_t (&key)[4],
                                      bool (&ok)[4]) {
  const float4 v =
      __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(r, s * 4, 0, 0));
  key[0] = float_key(v.x); key[1] = float_key(v.y);
  key[2] = float_key(v.z); key[3] = float_key(v.w);
#pragma unroll
  for (int j = 0; j < 4; ++j) ok[j] = (s + j) < n;
}

// Unordered pass over the n visible scores of a row by a whole kTkThreads
// workgroup: f(key) for each, with kRowBatch 16-byte loads per thread in
// flight (vector v of a batch is at 4 * (tid + kTkThreads * v)).
constexpr int kRowBatch = 4;
template <typename F>
__device__ __forceinline__ void for_each_key(__amdgpu_buffer_rsrc_t r, int n, F f) {
  for (int base = 0; base < n; base += 4 * kTkThreads * kRowBatch) {
    uint32_t key[kRowBatch][4];
    bool ok[kRowBatch][4];
#pragma unroll
    for (int v = 0; v < kRowBatch; ++v)
      load4(r, base + 4 * ((int)threadIdx.x + kTkThreads * v), n, key[v], ok[v]);
#pragma unroll
    for (int v = 0; v < kRowBatch; ++v)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (ok[v][j]) f(key[v][j]);
  }
}

// Copy a 4096-bin histogram from global memory into LDS with 16-byte loads,
// all of a thread's loads issued before the first LDS write.
template <int NTH>
__device__ __forceinline__ void hist_to_lds(const uint32_t* __restrict__ g, uint32_t* l) {
  constexpr int V = kBins1 / (4 * NTH);
  static_assert(V * 4 * NTH == kBins1, "whole vectors per thread");
  i32x4 v[V];
#pragma unroll
  for (int u = 0; u < V; ++u) v[u] = ld16(g + 4 * (threadIdx.x + NTH * u));
#pragma unroll
  for (int u = 0; u < V; ++u) *reinterpret_cast<i32x4*>(l + 4 * (threadIdx.x + NTH * u)) = v[u];
}

// Ordered emission of the selected elements: key > tau, or key == tau and
// among the first take_eq such elements.  Elements arrive E per thread in
// position order through `fetch(base, key, pos, ok)` (E * kTkThreads < 2^16).
template <int E = 4, typename Fetch>
__device__ void emit_selected(int count, uint32_t tau, uint32_t take_eq, int32_t* out,
                              TopkSmem& sm, Fetch fetch) {
  static_assert(E * kTkThreads < 65536, "per-pass counts fit 16 bits");
  const int tid = threadIdx.x;
  uint32_t run_gt = 0, run_eq = 0;
  for (int base = 0; base < count; base += E * kTkThreads) {
    uint32_t key[E] = {};
    int32_t pos[E] = {};
    bool ok[E];
    fetch(base + E * tid, key, pos, ok);
    uint32_t ngt = 0, neq = 0;
#pragma unroll
    for (int j = 0; j < E; ++j) {
      ngt += (ok[j] && key[j] > tau);
      neq += (ok[j] && key[j] == tau);
    }
    uint32_t tot;
    const uint32_t ex = block_excl_scan<kTkWaves>((ngt << 16) | neq, sm.scan, tot);
    uint32_t gt_b = run_gt + (ex >> 16), eq_b = run_eq + (ex & 0xFFFFu);
#pragma unroll
    for (int j = 0; j < E; ++j) {
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

// Steps 3-4 from the LDS list of the M elements in bins >= b1.  The second-
// and third-digit histograms are sm.hist[0, 1024) and [1024, 2048) (zero on
// entry when `zeroed`); each digit is selected by one wave, so a digit costs
// two barriers.  The emission takes 8 list entries per thread, so a list of
// up to 8192 entries is emitted in one ordered pass.
__device__ __forceinline__ void finish_from_list(int M, uint32_t b1, uint32_t above1, int k, int32_t* out,
                                 TopkSmem& sm, bool zeroed = false) {
  const int tid = threadIdx.x;
  uint32_t* h2 = sm.hist;
  uint32_t* h3 = sm.hist + kBins2;
  if (!zeroed) {
    for (int i = tid; i < 2 * kBins2; i += kTkThreads) sm.hist[i] = 0;
    __syncthreads();
  }
  for (int e = tid; e < M; e += kTkThreads) {
    const uint32_t key = sm.list_key[e];
    if ((key >> 20) == b1) atomicAdd(&h2[(key >> 10) & 1023u], 1u);
  }
  __syncthreads();
  if (tid < kWave) wave_select_bin<kBins2>(h2, (uint32_t)k - above1, sm.sel);
  __syncthreads();
  const uint32_t b2 = sm.sel[0];
  const uint32_t above2 = sm.sel[1];
  const uint32_t pre2 = (b1 << 10) | b2;
  for (int e = tid; e < M; e += kTkThreads) {
    const uint32_t key = sm.list_key[e];
    if ((key >> 10) == pre2) atomicAdd(&h3[key & 1023u], 1u);
  }
  __syncthreads();
  if (tid < kWave) wave_select_bin<kBins2>(h3, (uint32_t)k - above1 - above2, sm.sel + 2);
  __syncthreads();
  const uint32_t b3 = sm.sel[2];
  const uint32_t above3 = sm.sel[3];
  const uint32_t tau = (b1 << 20) | (b2 << 10) | b3;
  const uint32_t take_eq = (uint32_t)k - above1 - above2 - above3;
  // (the reads are unconditional, two 16-byte reads per array: entries past
  // M are stale and masked, and the list has room for 8 kTkThreads entries)
  static_assert(8 * kTkThreads <= kTkCap, "whole emission pass inside the list");
  emit_selected<8>(M, tau, take_eq, out, sm,
                   [&](int e, uint32_t(&key)[8], int32_t(&p)[8], bool(&ok)[8]) {
                     const uint4 k0 = *reinterpret_cast<const uint4*>(&sm.list_key[e]);
                     const uint4 k1 = *reinterpret_cast<const uint4*>(&sm.list_key[e + 4]);
                     const int4 p0 = *reinterpret_cast<const int4*>(&sm.list_pos[e]);
                     const int4 p1 = *reinterpret_cast<const int4*>(&sm.list_pos[e + 4]);
                     key[0] = k0.x; key[1] = k0.y; key[2] = k0.z; key[3] = k0.w;
                     key[4] = k1.x; key[5] = k1.y; key[6] = k1.z; key[7] = k1.w;
                     p[0] = p0.x; p[1] = p0.y; p[2] = p0.z; p[3] = p0.w;
                     p[4] = p1.x; p[5] = p1.y; p[6] = p1.z; p[7] = p1.w;
#pragma unroll
                     for (int j = 0; j < 8; ++j) ok[j] = (e + j) < M;
                   });
}

// Steps 3-4 for a list of at most 8 kTkThreads entries whose second-digit
// histogram (sm.hist[0, 1024)) is already counted and whose third-digit one
// (sm.hist[1024, 2048)) is zero: each thread reads its 8 consecutive entries
// once, while one wave picks the second digit, and keeps them in registers
// for the third digit and the ordered emission.
__device__ __forceinline__ void finish_from_list_once(int M, uint32_t b1, uint32_t above1, int k,
                                                      int32_t* out, TopkSmem& sm) {
  const int tid = threadIdx.x;
  uint32_t* h2 = sm.hist;
  uint32_t* h3 = sm.hist + kBins2;
  const int e0 = 8 * tid;
  // (unconditional 16-byte reads: entries past M are stale and masked)
  const uint4 k0 = *reinterpret_cast<const uint4*>(&sm.list_key[e0]);
  const uint4 k1 = *reinterpret_cast<const uint4*>(&sm.list_key[e0 + 4]);
  const int4 p0 = *reinterpret_cast<const int4*>(&sm.list_pos[e0]);
  const int4 p1 = *reinterpret_cast<const int4*>(&sm.list_pos[e0 + 4]);
  const uint32_t key[8] = {k0.x, k0.y, k0.z, k0.w, k1.x, k1.y, k1.z, k1.w};
  const int32_t pos[8] = {p0.x, p0.y, p0.z, p0.w, p1.x, p1.y, p1.z, p1.w};
  bool ok[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) ok[j] = e0 + j < M;
  if (tid < kWave) wave_select_bin<kBins2>(h2, (uint32_t)k - above1, sm.sel);
  __syncthreads();
  const uint32_t b2 = sm.sel[0];
  const uint32_t above2 = sm.sel[1];
  const uint32_t pre2 = (b1 << 10) | b2;
#pragma unroll
  for (int j = 0; j < 8; ++j)
    if (ok[j] && (key[j] >> 10) == pre2) atomicAdd(&h3[key[j] & 1023u], 1u);
  __syncthreads();
  if (tid < kWave) wave_select_bin<kBins2>(h3, (uint32_t)k - above1 - above2, sm.sel + 2);
  __syncthreads();
  const uint32_t tau = (b1 << 20) | (b2 << 10) | sm.sel[2];
  const uint32_t take_eq = (uint32_t)k - above1 - above2 - sm.sel[3];
  emit_selected<8>(M, tau, take_eq, out, sm,
                   [&](int, uint32_t(&kk)[8], int32_t(&pp)[8], bool(&oo)[8]) {
#pragma unroll
                     for (int j = 0; j < 8; ++j) {
                       kk[j] = key[j];
                       pp[j] = pos[j];
                       oo[j] = ok[j];
                     }
                   });
}

// Steps 3-4 re-reading the row from memory (list would not fit in LDS).
__device__ __forceinline__ void finish_from_row(const float* src, int n, uint32_t b1, uint32_t above1, int k,
                                int32_t* out, TopkSmem& sm) {
  const int tid = threadIdx.x;
  const __amdgpu_buffer_rsrc_t r = row_rsrc(src, n);
  for (int i = tid; i < kBins2; i += kTkThreads) sm.hist[i] = 0;
  __syncthreads();
  for_each_key(r, n, [&](uint32_t key) {
    if ((key >> 20) == b1) atomicAdd(&sm.hist[(key >> 10) & 1023u], 1u);
  });
  __syncthreads();
  select_bin<kBins2, kTkThreads>(sm.hist, (uint32_t)k - above1, sm.scan, sm.sel);
  const uint32_t b2 = sm.sel[0];
  const uint32_t above2 = sm.sel[1];
  __syncthreads();
  const uint32_t pre2 = (b1 << 10) | b2;
  for (int i = tid; i < kBins2; i += kTkThreads) sm.hist[i] = 0;
  __syncthreads();
  for_each_key(r, n, [&](uint32_t key) {
    if ((key >> 10) == pre2) atomicAdd(&sm.hist[key & 1023u], 1u);
  });
  __syncthreads();
  select_bin<kBins2, kTkThreads>(sm.hist, (uint32_t)k - above1 - above2, sm.scan, sm.sel);
  const uint32_t b3 = sm.sel[0];
  const uint32_t above3 = sm.sel[1];
  __syncthreads();
  const uint32_t tau = (b1 << 20) | (b2 << 10) | b3;
  const uint32_t take_eq = (uint32_t)k - above1 - above2 - above3;
  emit_selected(n, tau, take_eq, out, sm,
                [&](int s, uint32_t(&key)[4], int32_t(&p)[4], bool(&ok)[4]) {
                  load4(r, s, n, key, ok);
#pragma unroll
                  for (int j = 0; j < 4; ++j) p[j] = s + j;
                });
}

// Steps 3-4 reading the candidate slices from memory (the list would not fit
// in LDS and there is no score row to re-read: the fused indexer keeps its
// scores on chip).  List entry e lives in the slice c with chunk_off[c] <= e <
// chunk_off[c + 1], at c * chunk + e - chunk_off[c]; sm.chunk_off holds the
// n_chunks + 1 slice offsets.  Slow (a binary search per entry) but only
// reached by rows whose threshold bin holds more than kTkCap elements.
__device__ void finish_from_slices(const uint32_t* ck, const int32_t* cp, int chunk,
                                   int n_chunks, int M, uint32_t b1, uint32_t above1, int k,
                                   int32_t* out, TopkSmem& sm) {
  const int tid = threadIdx.x;
  M = min(M, (int)sm.chunk_off[n_chunks]);  // never past the last slice (they agree)
  auto at = [&](int e) -> int64_t {
    int lo = 0, hi = n_chunks;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if ((int)sm.chunk_off[mid] <= e) lo = mid; else hi = mid;
    }
    return (int64_t)lo * chunk + (e - (int)sm.chunk_off[lo]);
  };
  for (int i = tid; i < kBins2; i += kTkThreads) sm.hist[i] = 0;
  __syncthreads();
  for (int e = tid; e < M; e += kTkThreads) {
    const uint32_t key = ck[at(e)];
    if ((key >> 20) == b1) atomicAdd(&sm.hist[(key >> 10) & 1023u], 1u);
  }
  __syncthreads();
  select_bin<kBins2, kTkThreads>(sm.hist, (uint32_t)k - above1, sm.scan, sm.sel);
  const uint32_t b2 = sm.sel[0];
  const uint32_t above2 = sm.sel[1];
  __syncthreads();
  const uint32_t pre2 = (b1 << 10) | b2;
  for (int i = tid; i < kBins2; i += kTkThreads) sm.hist[i] = 0;
  __syncthreads();
  for (int e = tid; e < M; e += kTkThreads) {
    const uint32_t key = ck[at(e)];
    if ((key >> 10) == pre2) atomicAdd(&sm.hist[key & 1023u], 1u);
  }
  __syncthreads();
  select_bin<kBins2, kTkThreads>(sm.hist, (uint32_t)k - above1 - above2, sm.scan, sm.sel);
  const uint32_t b3 = sm.sel[0];
  const uint32_t above3 = sm.sel[1];
  __syncthreads();
  const uint32_t tau = (b1 << 20) | (b2 << 10) | b3;
  const uint32_t take_eq = (uint32_t)k - above1 - above2 - above3;
  emit_selected(M, tau, take_eq, out, sm,
                [&](int e, uint32_t(&key)[4], int32_t(&p)[4], bool(&ok)[4]) {
#pragma unroll
                  for (int j = 0; j < 4; ++j) {
                    ok[j] = (e + j) < M;
                    if (ok[j]) {
                      const int64_t a = at(e + j);
                      key[j] = ck[a];
                      p[j] = cp[a];
                    }
                  }
                });
}

__device__ __forceinline__ int visible(const int32_t* ctx_len, int row, int T, int Lmax) {
  const int b = row / T;
  const int t = row - b * T;
  const int64_t pos = (int64_t)ctx_len[b] - T + t;
  return (int)max((int64_t)0, min(pos + 1, (int64_t)Lmax));
}

// A row of at most kRegRow scores held in registers (64 per thread), so it is
// read once, in one round trip: batch b of 16384 positions gives thread t
// positions 16384 b + 16 t .. + 15.  The first-digit histogram is counted
// from the registers, and the candidates (bins >= b1) are copied into the
// LDS list in position order from the same registers: one prefix scan of
// the four batches' per-thread counts (two 16-bit fields per word) places
// every thread's run.  (Reading the row twice, a batch in flight at a time,
// took 15 + 11 us per row of the 64K-context prefill chunk.)
constexpr int kRegBatches = 4;
constexpr int kRegRow = kRegBatches * 16 * kTkThreads;  // 65536
__device__ __forceinline__ void row_in_registers(__amdgpu_buffer_rsrc_t r, int n, int k,
                                                 int32_t* out, TopkSmem& sm, const float* src) {
  const int tid = threadIdx.x;
  uint32_t key[kRegBatches][16];
#pragma unroll
  for (int b = 0; b < kRegBatches; ++b)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const float4 x = __builtin_bit_cast(
          float4, __builtin_amdgcn_raw_buffer_load_b128(r, (16384 * b + 16 * tid + 4 * v) * 4, 0, 0));
      key[b][4 * v] = float_key(x.x);
      key[b][4 * v + 1] = float_key(x.y);
      key[b][4 * v + 2] = float_key(x.z);
      key[b][4 * v + 3] = float_key(x.w);
    }
  auto pos = [&](int b, int e) { return 16384 * b + 16 * tid + e; };
  // Only the bins at and above the k-th largest key's matter, and counting
  // every key piles the LDS atomics onto the few bins that hold the bulk of
  // the row (13 us per row here).  So a lower bound L of that bin is taken
  // first from a sample, one key per thread (positions 16 t): the bin of
  // the sample's kSample-th largest key.  Only keys in bins >= L are then
  // counted; if they number at least k, the k-th largest lies at or above L
  // and the counts above it are exact, otherwise (a sample that ran high)
  // every key is counted.  A row reaching this path has n > k; with fewer
  // than kSample valid sample keys the bound is bin 0 (every key).
  constexpr uint32_t kSample = 64;
  static_assert(kSample <= (uint32_t)kTkThreads, "one sample key per thread");
  const uint32_t valid = (uint32_t)min(kTkThreads, (n + 15) / 16);
  for (int i = tid; i < kBins1; i += kTkThreads) sm.hist[i] = 0;
  if (tid == 0) sm.sel[0] = 0;
  __syncthreads();
  if (pos(0, 0) < n) atomicAdd(&sm.hist[key[0][0] >> 20], 1u);
  __syncthreads();
  if (valid >= kSample && tid < kWave) wave_select_bin<kBins1>(sm.hist, kSample, sm.sel);
  __syncthreads();
  const uint32_t lb = sm.sel[0];
  for (int i = tid; i < kBins1; i += kTkThreads) sm.hist[i] = 0;
  __syncthreads();
  uint32_t counted = 0;
#pragma unroll
  for (int b = 0; b < kRegBatches; ++b)
#pragma unroll
    for (int e = 0; e < 16; ++e)
      if (pos(b, e) < n && (key[b][e] >> 20) >= lb) {
        atomicAdd(&sm.hist[key[b][e] >> 20], 1u);
        ++counted;
      }
  uint32_t total;
  block_excl_scan<kTkWaves>(counted, sm.scan, total);  // (its barriers follow the adds)
  if (total < (uint32_t)k) {  // the sample's bound ran above the k-th key: count them all
#pragma unroll
    for (int b = 0; b < kRegBatches; ++b)
#pragma unroll
      for (int e = 0; e < 16; ++e)
        if (pos(b, e) < n && (key[b][e] >> 20) < lb) atomicAdd(&sm.hist[key[b][e] >> 20], 1u);
    __syncthreads();
  }
  if (tid < kWave) wave_select_bin<kBins1>(sm.hist, (uint32_t)k, sm.sel);
  __syncthreads();
  const uint32_t b1 = sm.sel[0];
  const uint32_t above1 = sm.sel[1];
  const uint32_t listed = above1 + sm.hist[b1];
  __syncthreads();
  if (listed > (uint32_t)kTkCap) {
    finish_from_row(src, n, b1, above1, k, out, sm);
    return;
  }
  uint32_t c[kRegBatches];
#pragma unroll
  for (int b = 0; b < kRegBatches; ++b) {
    c[b] = 0;
#pragma unroll
    for (int e = 0; e < 16; ++e) c[b] += (pos(b, e) < n && (key[b][e] >> 20) >= b1) ? 1u : 0u;
  }
  // per-batch totals stay below 65536 (16384 positions), so two batches
  // share a word of 16-bit fields through the scan
  uint32_t tot01, tot23;
  const uint32_t ex01 = block_excl_scan<kTkWaves>(c[0] | (c[1] << 16), sm.scan, tot01);
  const uint32_t ex23 = block_excl_scan<kTkWaves>(c[2] | (c[3] << 16), sm.scan, tot23);
  const uint32_t t0 = tot01 & 0xffffu, t1 = tot01 >> 16, t2 = tot23 & 0xffffu;
  uint32_t at[kRegBatches] = {ex01 & 0xffffu, t0 + (ex01 >> 16), t0 + t1 + (ex23 & 0xffffu),
                              t0 + t1 + t2 + (ex23 >> 16)};
#pragma unroll
  for (int b = 0; b < kRegBatches; ++b)
#pragma unroll
    for (int e = 0; e < 16; ++e)
      if (pos(b, e) < n && (key[b][e] >> 20) >= b1) {
        sm.list_key[at[b]] = key[b][e];
        sm.list_pos[at[b]] = pos(b, e);
        ++at[b];
      }
  finish_from_list((int)listed, b1, above1, k, out, sm);  // (its first barrier publishes the list)
}

// ---------------------------------------------------------------- one workgroup per row
__global__ __launch_bounds__(kTkThreads) void topk_row_kernel(
    const float* __restrict__ scores, int64_t ld, const int32_t* __restrict__ ctx_len, int T,
    int Lmax, int k, int32_t* __restrict__ idx) {
  extern __shared__ __align__(16) unsigned char smem_raw[];
  TopkSmem& sm = *reinterpret_cast<TopkSmem*>(smem_raw);
  const int tid = threadIdx.x;
  const int row = blockIdx.x;
  const int n = visible(ctx_len, row, T, Lmax);
  int32_t* out = idx + (int64_t)row * k;
  if (n <= k) {  // everything visible is selected
    for (int i = tid; i < k; i += kTkThreads) out[i] = i < n ? i : -1;
    return;
  }
  const float* src = scores + (int64_t)row * ld;
  const __amdgpu_buffer_rsrc_t r = row_rsrc(src, n);
  if (n <= kRegRow) {
    row_in_registers(r, n, k, out, sm, src);
    return;
  }
  for (int i = tid; i < kBins1; i += kTkThreads) sm.hist[i] = 0;
  __syncthreads();
  for_each_key(r, n, [&](uint32_t key) { atomicAdd(&sm.hist[key >> 20], 1u); });
  __syncthreads();
  if (tid < kWave) wave_select_bin<kBins1>(sm.hist, (uint32_t)k, sm.sel);
  __syncthreads();
  const uint32_t b1 = sm.sel[0];
  const uint32_t above1 = sm.sel[1];
  const uint32_t listed = above1 + sm.hist[b1];
  __syncthreads();
  if (listed > (uint32_t)kTkCap) {
    finish_from_row(src, n, b1, above1, k, out, sm);
    return;
  }
  // Ordered copy of the candidates: a thread owns kPer consecutive scores of
  // each batch, and the next batch is in flight while this one is copied.
  constexpr int kBatch = kPer * kTkThreads;
  uint32_t key[kPer / 4][4], nkey[kPer / 4][4];
  bool ok[kPer / 4][4], nok[kPer / 4][4];
#pragma unroll
  for (int v = 0; v < kPer / 4; ++v) load4(r, kPer * tid + 4 * v, n, key[v], ok[v]);
  uint32_t run = 0;
  for (int base = 0; base < n; base += kBatch) {
    const int s0 = base + kPer * tid;
#pragma unroll
    for (int v = 0; v < kPer / 4; ++v) load4(r, s0 + kBatch + 4 * v, n, nkey[v], nok[v]);
    uint32_t c = 0;
#pragma unroll
    for (int v = 0; v < kPer / 4; ++v)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        ok[v][j] = ok[v][j] && (key[v][j] >> 20) >= b1;
        c += ok[v][j];
      }
    uint32_t tot;
    uint32_t at = run + block_excl_scan<kTkWaves>(c, sm.scan, tot);
#pragma unroll
    for (int v = 0; v < kPer / 4; ++v)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (ok[v][j]) {
          sm.list_key[at] = key[v][j];
          sm.list_pos[at] = s0 + 4 * v + j;
          ++at;
        }
    run += tot;
#pragma unroll
    for (int v = 0; v < kPer / 4; ++v)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        key[v][j] = nkey[v][j];
        ok[v][j] = nok[v][j];
      }
  }
  finish_from_list((int)listed, b1, above1, k, out, sm);
}

// ---------------------------------------------------------------- chunked rows
// Step 1 over one chunk: LDS histogram, then add its non-zero bins to the row's.
__global__ __launch_bounds__(kChThreads) void topk_chunk_hist_kernel(
    const float* __restrict__ scores, int64_t ld, const int32_t* __restrict__ ctx_len, int T,
    int Lmax, int k, int chunk, uint32_t* __restrict__ hist_g) {
  __shared__ __attribute__((aligned(16))) uint32_t h[kBins1];
  const int tid = threadIdx.x;
  const int row = blockIdx.y;
  const int n = visible(ctx_len, row, T, Lmax);
  if (n <= k) return;
  const int c0 = blockIdx.x * chunk;
  const int c1 = min(n, c0 + chunk);
  if (c0 >= c1) return;
  for (int i = tid; i < kBins1; i += kChThreads) h[i] = 0;
  __syncthreads();
  const __amdgpu_buffer_rsrc_t r = row_rsrc(scores + (int64_t)row * ld, c1);
  // a thread owns kPer consecutive scores of each batch; all loads first
  for (int base = c0; base < c1; base += kPer * kChThreads) {
    const int s0 = base + kPer * tid;
    uint32_t key[kPer / 4][4];
    bool ok[kPer / 4][4];
#pragma unroll
    for (int v = 0; v < kPer / 4; ++v) load4(r, s0 + 4 * v, c1, key[v], ok[v]);
#pragma unroll
    for (int v = 0; v < kPer / 4; ++v)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (ok[v][j]) atomicAdd(&h[key[v][j] >> 20], 1u);
  }
  __syncthreads();
  uint32_t* hg = hist_g + (int64_t)row * kBins1;
  for (int i = tid; i < kBins1; i += kChThreads)
    if (h[i]) atomicAdd(&hg[i], h[i]);
}

// Step 2 over one chunk: ordered copy of its elements in bins >= b1 into the
// chunk's own slice [c0, c0 + count) of the row's candidate buffer.
__global__ __launch_bounds__(kChThreads) void topk_chunk_collect_kernel(
    const float* __restrict__ scores, int64_t ld, const int32_t* __restrict__ ctx_len, int T,
    int Lmax, int k, int chunk, const uint32_t* __restrict__ hist_g,
    uint32_t* __restrict__ cand_key, int32_t* __restrict__ cand_pos,
    uint32_t* __restrict__ cand_cnt, int n_chunks, uint32_t* __restrict__ row_sel) {
  __shared__ uint32_t scan[kChWaves];
  __shared__ uint32_t sel[4];
  __shared__ __attribute__((aligned(16))) uint32_t h[kBins1];
  const int tid = threadIdx.x;
  const int row = blockIdx.y;
  const int n = visible(ctx_len, row, T, Lmax);
  if (n <= k) return;
  const int c0 = blockIdx.x * chunk;
  const int c1 = min(n, c0 + chunk);
  const __amdgpu_buffer_rsrc_t r = row_rsrc(scores + (int64_t)row * ld, c1);
  // the chunk's first batch of scores is requested before the histogram
  uint32_t key[kPer / 4][4];
  bool ok[kPer / 4][4];
#pragma unroll
  for (int v = 0; v < kPer / 4; ++v) load4(r, c0 + kPer * tid + 4 * v, c1, key[v], ok[v]);
  hist_to_lds<kChThreads>(hist_g + (int64_t)row * kBins1, h);
  __syncthreads();
  select_bin<kBins1, kChThreads>(h, (uint32_t)k, scan, sel);
  const uint32_t b1 = sel[0];
  if (blockIdx.x == 0 && tid == 0) {  // the row's selection, for the finishing pass
    row_sel[3 * row] = b1;
    row_sel[3 * row + 1] = sel[1];
    row_sel[3 * row + 2] = sel[1] + h[b1];
  }
  uint32_t* ck = cand_key + (int64_t)row * Lmax;
  int32_t* cp = cand_pos + (int64_t)row * Lmax;
  uint32_t run = 0;
  for (int base = c0; base < c1; base += kPer * kChThreads) {
    const int s0 = base + kPer * tid;
    if (base != c0) {
#pragma unroll
      for (int v = 0; v < kPer / 4; ++v) load4(r, s0 + 4 * v, c1, key[v], ok[v]);
    }
    uint32_t c = 0;
#pragma unroll
    for (int v = 0; v < kPer / 4; ++v)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        ok[v][j] = ok[v][j] && (key[v][j] >> 20) >= b1;
        c += ok[v][j];
      }
    uint32_t tot;
    uint32_t at = run + block_excl_scan<kChWaves>(c, scan, tot);
#pragma unroll
    for (int v = 0; v < kPer / 4; ++v)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (ok[v][j]) {
          ck[c0 + at] = key[v][j];
          cp[c0 + at] = s0 + 4 * v + j;
          ++at;
        }
    run += tot;
  }
  if (tid == 0) cand_cnt[(int64_t)row * n_chunks + blockIdx.x] = (c0 < c1) ? run : 0u;
}

// Steps 3-4 for one row from the chunk slices; clears the row's histogram.
// scores is null after the fused indexer (no score row in memory): an
// overflowing list is then read from the slices.  With sel_from_hist (after
// the fused indexer) the threshold bin comes from the finished histogram and
// the slices may also hold keys below it, which are never emitted; otherwise
// row_sel holds it (written by the collect pass).
// (The arguments its first loads need come first: the leading argument
// dwords are preloaded into scalar registers at launch.)
__global__ __launch_bounds__(kTkThreads) void topk_finish_kernel(
    uint32_t* __restrict__ hist_g, const uint32_t* __restrict__ cand_key,
    const int32_t* __restrict__ cand_pos, const uint32_t* __restrict__ cand_cnt,
    const int32_t* __restrict__ ctx_len, int T, int Lmax, int chunk, int n_chunks, int k,
    const uint32_t* __restrict__ row_sel, int sel_from_hist, const float* __restrict__ scores,
    int64_t ld, int32_t* __restrict__ idx) {
  extern __shared__ __align__(16) unsigned char smem_raw[];
  TopkSmem& sm = *reinterpret_cast<TopkSmem*>(smem_raw);
  const int tid = threadIdx.x;
  const int row = blockIdx.x;
  uint32_t* hg = hist_g + (int64_t)row * kBins1;
  // The slice counts, the histogram and the row's selection (written by
  // the collect pass when the histogram is not finished): unconditional
  // loads, through buffer resources where a count or a pointer may be short
  // (the selection's range is empty when it is not used).
  const uint32_t cnt = __builtin_amdgcn_raw_buffer_load_b32(
      __builtin_amdgcn_make_buffer_rsrc((void*)(cand_cnt + (int64_t)row * n_chunks), 0,
                                        n_chunks * 4, kBufferWord3),
      tid * 4, 0, 0);
  static_assert(kBins1 == 4 * kTkThreads, "one 16-byte histogram load per thread");
  const i32x4 hv = ld16(hg + 4 * tid);
  const __amdgpu_buffer_rsrc_t sr = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(row_sel + 3 * (int64_t)row), 0, sel_from_hist ? 0 : 12, kBufferWord3);
  uint32_t b1 = __builtin_amdgcn_raw_buffer_load_b32(sr, 0, 0, 0);
  uint32_t above1 = __builtin_amdgcn_raw_buffer_load_b32(sr, 4, 0, 0);
  uint32_t listed = __builtin_amdgcn_raw_buffer_load_b32(sr, 8, 0, 0);
  // Each slice is copied by its own group of tpc threads.  The first batch
  // of every slice is requested now, before its length is known (slice c
  // starts at c * chunk; entries past its length are ignored), so the copy
  // does not wait for a second round trip.  These loads and the context
  // length are all in flight together: the kernel starts on one round trip
  // to memory.
  const int tpc = kTkThreads / n_chunks;
  const int cq = tid / tpc;  // this thread's slice (none when >= n_chunks)
  const int sub = tid - cq * tpc;
  const int64_t base = (int64_t)min(cq, n_chunks - 1) * chunk;
  const int cap = (int)min((int64_t)chunk, (int64_t)Lmax - base);  // room of the slice
  const uint32_t* ck = cand_key + (int64_t)row * Lmax + base;
  const int32_t* cp = cand_pos + (int64_t)row * Lmax + base;
  uint32_t kv[kFinGather];
  int32_t pv[kFinGather];
#pragma unroll
  for (int u = 0; u < kFinGather; ++u) {
    const int e = min(sub + u * tpc, cap - 1);
    kv[u] = ck[e];
    pv[u] = cp[e];
  }
  const int n = visible(ctx_len, row, T, Lmax);
  // (every load above has returned before the branch: otherwise the
  // compiler moves the slice loads below it, after the context length)
#pragma unroll
  for (int u = 0; u < kFinGather; ++u) asm volatile("" ::"v"(kv[u]), "v"(pv[u]));
  asm volatile("" ::"v"(cnt), "v"(hv[0]), "v"(hv[1]), "v"(hv[2]), "v"(hv[3]), "v"(b1),
               "v"(above1), "v"(listed));
  int32_t* out = idx + (int64_t)row * k;
  if (n <= k) {
    for (int i = tid; i < k; i += kTkThreads) out[i] = i < n ? i : -1;
    // the chunk kernels touched nothing for this row, but a fused
    // histogram from the indexer may have
    for (int i = tid; i < kBins1; i += kTkThreads) hg[i] = 0;
    return;
  }
  // The second- and third-digit histograms start at zero (cleared now, in
  // LDS that nothing else uses before the list is complete).
  for (int i = tid; i < 2 * kBins2; i += kTkThreads) sm.hist[i] = 0;
  // One block-wide scan of two values per thread: the slice counts (their
  // exclusive prefix places each slice in the list) and, after the fused
  // indexer, the sums of this thread's four histogram bins (4 tid .. 4 tid
  // + 3), whose inclusive prefix gives the count above each bin.
  {
    const int lane = tid & (kWave - 1);
    const int wid = __builtin_amdgcn_readfirstlane(tid / kWave);
    const uint32_t hs = sel_from_hist ? (uint32_t)(hv[0] + hv[1] + hv[2] + hv[3]) : 0u;
    const uint32_t hin = wave_incl_scan(hs);
    const uint32_t cin = wave_incl_scan(cnt);
    if (lane == kWave - 1) {
      sm.scan[wid] = hin;
      sm.scan2[wid] = cin;
    }
    if (tid == 0) {  // (overwritten after the barrier by the bin's thread)
      sm.sel[0] = 0;
      sm.sel[1] = 0;
    }
    // ready for the next call (every thread's histogram load has returned)
    *reinterpret_cast<i32x4*>(hg + 4 * tid) = i32x4{0, 0, 0, 0};
    __syncthreads();
    // (lane i scans wave i's totals; the wave reads its own prefix back)
    const uint32_t hw = row16_incl_scan(lane < kTkWaves ? sm.scan[lane] : 0u);
    const uint32_t cw = row16_incl_scan(lane < kTkWaves ? sm.scan2[lane] : 0u);
    const uint32_t htot = (uint32_t)__builtin_amdgcn_readlane((int)hw, kTkWaves - 1);
    const uint32_t ctot = (uint32_t)__builtin_amdgcn_readlane((int)cw, kTkWaves - 1);
    const uint32_t hbefore = wid > 0 ? (uint32_t)__builtin_amdgcn_readlane((int)hw, wid - 1) : 0u;
    const uint32_t cbefore = wid > 0 ? (uint32_t)__builtin_amdgcn_readlane((int)cw, wid - 1) : 0u;
    if (tid < n_chunks) sm.chunk_off[tid] = cbefore + cin - cnt;
    if (tid == 0) sm.chunk_off[n_chunks] = ctot;
    if (sel_from_hist) {
      // exactly one bin holds the k-th largest key (the histogram counts
      // every visible key and n > k): its thread records it
      uint32_t above = htot - (hbefore + hin);
#pragma unroll
      for (int j = 3; j >= 0; --j) {
        const uint32_t c = (uint32_t)hv[j];
        if (above < (uint32_t)k && (uint32_t)k <= above + c) {
          sm.sel[0] = 4 * tid + j;
          sm.sel[1] = above;
        }
        above += c;
      }
      listed = ctot;  // every slice entry, extra ones included
    }
    __syncthreads();
  }
  if (sel_from_hist) {
    b1 = sm.sel[0];
    above1 = sm.sel[1];
  }
  if (listed > (uint32_t)kTkCap) {
    if (scores != nullptr)
      finish_from_row(scores + (int64_t)row * ld, n, b1, above1, k, out, sm);
    else
      finish_from_slices(cand_key + (int64_t)row * Lmax, cand_pos + (int64_t)row * Lmax, chunk,
                         n_chunks, (int)listed, b1, above1, k, out, sm);
    return;
  }
  // A list that one emission pass covers has its second-digit histogram
  // counted here, from the registers, while it is copied.
  const bool count2 = listed <= (uint32_t)(8 * kTkThreads);
  uint32_t* h2 = sm.hist;
  if (cq < n_chunks) {
    const uint32_t off = sm.chunk_off[cq];
    const int cn = (int)(sm.chunk_off[cq + 1] - off);
#pragma unroll
    for (int u = 0; u < kFinGather; ++u) {
      const int e = sub + u * tpc;
      if (e < cn) {
        sm.list_key[off + e] = kv[u];
        sm.list_pos[off + e] = pv[u];
        if (count2 && (kv[u] >> 20) == b1) atomicAdd(&h2[(kv[u] >> 10) & 1023u], 1u);
      }
    }
    // the rest (long slices), batches of kFinGather entries per thread with
    // all loads issued first
    for (int e0 = sub + kFinGather * tpc; e0 < cn; e0 += kFinGather * tpc) {
#pragma unroll
      for (int u = 0; u < kFinGather; ++u) {
        const int e = min(e0 + u * tpc, cn - 1);
        kv[u] = ck[e];
        pv[u] = cp[e];
      }
#pragma unroll
      for (int u = 0; u < kFinGather; ++u) {
        const int e = e0 + u * tpc;
        if (e < cn) {
          sm.list_key[off + e] = kv[u];
          sm.list_pos[off + e] = pv[u];
          if (count2 && (kv[u] >> 20) == b1) atomicAdd(&h2[(kv[u] >> 10) & 1023u], 1u);
        }
      }
    }
  }
  __syncthreads();
  if (!count2) {
    finish_from_list((int)listed, b1, above1, k, out, sm, /*zeroed=*/true);
    return;
  }
  finish_from_list_once((int)listed, b1, above1, k, out, sm);
}

// Top-k per row among a position-ordered candidate list that holds every
// key of the row's top k (the fused prefill indexer's output): the list is
// copied into LDS (kGather entries per thread in flight) while its first
// radix digit is counted, then steps 3-4 run on it; the extra candidates
// below the threshold are never emitted.  A list longer than the LDS list is
// finished from memory.
__global__ __launch_bounds__(kTkThreads) void topk_cand_kernel(
    const int32_t* __restrict__ ctx_len, int T, int Lmax, int k,
    const uint32_t* __restrict__ cand_key, const int32_t* __restrict__ cand_pos,
    const uint32_t* __restrict__ cand_cnt, int32_t* __restrict__ idx) {
  extern __shared__ __align__(16) unsigned char smem_raw[];
  TopkSmem& sm = *reinterpret_cast<TopkSmem*>(smem_raw);
  const int tid = threadIdx.x;
  const int row = blockIdx.x;
  const int n = visible(ctx_len, row, T, Lmax);
  int32_t* out = idx + (int64_t)row * k;
  if (n <= k) {
    for (int i = tid; i < k; i += kTkThreads) out[i] = i < n ? i : -1;
    return;
  }
  const int M = (int)cand_cnt[row];  // >= k: the row's top k are all listed
  const uint32_t* ck = cand_key + (int64_t)row * Lmax;
  const int32_t* cp = cand_pos + (int64_t)row * Lmax;
  for (int i = tid; i < kBins1; i += kTkThreads) sm.hist[i] = 0;
  __syncthreads();
  const bool fits = M <= kTkCap;
  if (fits) {
    for (int e0 = tid; e0 < M; e0 += kGather * kTkThreads) {
      uint32_t kv[kGather];
      int32_t pv[kGather];
#pragma unroll
      for (int u = 0; u < kGather; ++u) {
        const int e = min(e0 + u * kTkThreads, M - 1);
        kv[u] = ck[e];
        pv[u] = cp[e];
      }
#pragma unroll
      for (int u = 0; u < kGather; ++u) {
        const int e = e0 + u * kTkThreads;
        if (e < M) {
          sm.list_key[e] = kv[u];
          sm.list_pos[e] = pv[u];
          atomicAdd(&sm.hist[kv[u] >> 20], 1u);
        }
      }
    }
  } else {
    for (int e = tid; e < M; e += kTkThreads) atomicAdd(&sm.hist[ck[e] >> 20], 1u);
  }
  __syncthreads();
  if (tid < kWave) wave_select_bin<kBins1>(sm.hist, (uint32_t)k, sm.sel);
  __syncthreads();
  const uint32_t b1 = sm.sel[0];
  const uint32_t above1 = sm.sel[1];
  __syncthreads();
  if (fits) {
    finish_from_list(M, b1, above1, k, out, sm);
    return;
  }
  if (tid == 0) {
    sm.chunk_off[0] = 0;
    sm.chunk_off[1] = (uint32_t)M;
  }
  __syncthreads();
  finish_from_slices(ck, cp, Lmax, 1, M, b1, above1, k, out, sm);
}

struct TopkPlan {
  bool chunked;
  int chunk, n_chunks;
};

TopkPlan plan_topk(int B, int T, int Lmax) {
  TopkPlan p{false, 0, 0};
  const int rows = B * T;
  if (rows > 128 || Lmax < 16384) return p;
  // ~512 chunk workgroups, chunks of at least 4096 scores
  int nc = (512 + rows - 1) / rows;
  int chunk = (Lmax + nc - 1) / nc;
  chunk = max(4096, (chunk + 4095) / 4096 * 4096);
  nc = (Lmax + chunk - 1) / chunk;
  if (nc > kMaxChunks) return p;
  p.chunked = true;
  p.chunk = chunk;
  p.n_chunks = nc;
  return p;
}

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

}  // namespace

// Workspace of the chunked selection: per-row histograms (kept zero between
// calls), per-row selection {b1, count above b1, listed}, per-chunk counts,
// candidate keys and positions.
TopkWs topk_chunk_ws(void* ws, int rows, int Lmax, int n_chunks) {
  unsigned char* p = reinterpret_cast<unsigned char*>(ws);
  TopkWs w;
  w.hist = reinterpret_cast<uint32_t*>(p);
  p += align256((size_t)rows * kBins1 * 4);
  w.sel = reinterpret_cast<uint32_t*>(p);
  p += align256((size_t)rows * 3 * 4);
  w.cnt = reinterpret_cast<uint32_t*>(p);
  p += align256((size_t)rows * n_chunks * 4);
  w.key = reinterpret_cast<uint32_t*>(p);
  p += align256((size_t)rows * Lmax * 4);
  w.pos = reinterpret_cast<int32_t*>(p);
  return w;
}

size_t topk_chunk_ws_bytes(int rows, int Lmax, int n_chunks) {
  return align256((size_t)rows * kBins1 * 4) + align256((size_t)rows * 3 * 4) + align256((size_t)rows * n_chunks * 4) +
         2 * align256((size_t)rows * Lmax * 4);
}

namespace {

hipError_t set_smem_attr(const void* fn, size_t bytes) {
  return hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
}

}  // namespace

size_t topk_workspace_bytes(int B, int T, int Lmax, int) {
  const TopkPlan p = plan_topk(B, T, Lmax);
  if (!p.chunked) return 0;
  return topk_chunk_ws_bytes(B * T, Lmax, p.n_chunks);
}

uint32_t* topk_row_hist(void* workspace, int B, int T, int Lmax, int) {
  const TopkPlan p = plan_topk(B, T, Lmax);
  if (!p.chunked || workspace == nullptr) return nullptr;
  return topk_chunk_ws(workspace, B * T, Lmax, p.n_chunks).hist;
}

hipError_t launch_topk(const float* scores, int64_t ld, const int32_t* ctx_len, int B, int T,
                       int Lmax, int k, int32_t* idx, void* workspace, size_t,
                       bool hist_ready, hipStream_t stream) {
  const size_t smem = sizeof(TopkSmem);
  const TopkPlan p = plan_topk(B, T, Lmax);
  const int rows = B * T;
  if (!p.chunked) {
    hipError_t e = set_smem_attr((const void*)topk_row_kernel, smem);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(topk_row_kernel, dim3(rows), dim3(kTkThreads), smem, stream, scores, ld,
                       ctx_len, T, Lmax, k, idx);
    return hipGetLastError();
  }
  const TopkWs w = topk_chunk_ws(workspace, rows, Lmax, p.n_chunks);
  const dim3 grid(p.n_chunks, rows);
  if (!hist_ready)
    hipLaunchKernelGGL(topk_chunk_hist_kernel, grid, dim3(kChThreads), 0, stream, scores, ld,
                       ctx_len, T, Lmax, k, p.chunk, w.hist);
  hipLaunchKernelGGL(topk_chunk_collect_kernel, grid, dim3(kChThreads), 0, stream, scores, ld,
                     ctx_len, T, Lmax, k, p.chunk, w.hist, w.key, w.pos, w.cnt, p.n_chunks,
                     w.sel);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_topk_finish(scores, ld, ctx_len, B, T, Lmax, k, p.chunk, p.n_chunks, w, false,
                            idx, stream);
}

hipError_t launch_topk_candidates(const int32_t* ctx_len, int B, int T, int Lmax, int k,
                                  const uint32_t* key, const int32_t* pos, const uint32_t* cnt,
                                  int32_t* idx, hipStream_t stream) {
  const size_t smem = sizeof(TopkSmem);
  hipError_t e = set_smem_attr((const void*)topk_cand_kernel, smem);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(topk_cand_kernel, dim3(B * T), dim3(kTkThreads), smem, stream, ctx_len, T,
                     Lmax, k, key, pos, cnt, idx);
  return hipGetLastError();
}

hipError_t launch_topk_finish(const float* scores, int64_t ld, const int32_t* ctx_len, int B,
                              int T, int Lmax, int k, int chunk, int n_chunks, const TopkWs& w,
                              bool sel_from_hist, int32_t* idx, hipStream_t stream) {
  const size_t smem = sizeof(TopkSmem);
  hipError_t e = set_smem_attr((const void*)topk_finish_kernel, smem);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(topk_finish_kernel, dim3(B * T), dim3(kTkThreads), smem, stream, w.hist,
                     w.key, w.pos, w.cnt, ctx_len, T, Lmax, chunk, n_chunks, k, w.sel,
                     (int)sel_from_hist, scores, ld, idx);
  return hipGetLastError();
}

}  // namespace dsa
